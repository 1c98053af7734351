"""Pins of the packed weight layout: hand-worked byte examples, exhaustive
round trips through the generator's independent packer, the identity of the
packed forms with the int8 container, and the blob size the pages state."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packed_format_examples.json")


def _cases():
    return json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "int%d-%s" % (c["bits"], c["bytes_hex"][:6]))
def test_hand_worked_bytes(case):
    codes = np.zeros(32, np.int8)
    for k, v in case["nonzero_codes"].items():
        codes[int(k)] = v
    raw = np.frombuffer(bytes.fromhex(case["bytes_hex"]), np.uint8)
    assert oracle.unpack(raw, 32, case["bits"]).tolist() == codes.tolist()
    assert synth.pack_codes(codes[None, :], case["bits"]).ravel().tolist() == raw.tolist()


@pytest.mark.parametrize("bits,lo,hi", [(8, -128, 127), (4, -8, 7), (2, -2, 1)])
def test_every_code_at_every_position_round_trips(bits, lo, hi):
    vals = np.arange(lo, hi + 1)
    rows = []
    for shift in range(len(vals)):
        rows.append(np.resize(np.roll(vals, shift), 32 * 4))
    codes = np.array(rows, np.int8)
    packed = synth.pack_codes(codes, bits)
    for r in range(codes.shape[0]):
        assert np.array_equal(oracle.unpack(packed[r], codes.shape[1], bits), codes[r])


@pytest.mark.parametrize("bits", [4, 2])
def test_packed_identical_to_int8_container(bits):
    lo, hi = synth.QRANGE[bits]
    rng = np.random.default_rng(bits)
    codes = rng.integers(lo, hi + 1, size=(8, 256)).astype(np.int8)
    q = rng.integers(-127, 128, size=256).astype(np.int8)
    d = rng.random(8).astype(np.float32)
    p8 = synth.pack_codes(codes, 8)
    pk = synth.pack_codes(codes, bits)
    for r in range(8):
        a = oracle.unpack(p8[r], 256, 8)
        b = oracle.unpack(pk[r], 256, bits)
        assert np.array_equal(a, b)
        assert oracle.row_dot(a, q, d, 0.37) == oracle.row_dot(b, q, d, 0.37)


def test_blob_layout_and_glm_expert_size():
    for H, I, bits in [(256, 128, 4), (6144, 2048, 4), (6144, 2048, 8), (6144, 2048, 2), (512, 96, 2)]:
        assert oracle.blob_layout(H, I, bits) == synth.blob_layout(H, I, bits)
    assert synth.blob_layout(256, 128, 4)["total"] == 51200
    # the pages: about 19 MB per routed expert at int4 (GLM-5.2: hidden 6144, expert inter 2048)
    total = synth.blob_layout(6144, 2048, 4)["total"]
    assert total == 18915328 and 18.5e6 < total < 19.5e6


def test_generator_codes_survive_packing_in_a_blob():
    blob, parts = synth.gaussian_expert(0, 0, 3, synth.TINY)
    lay = oracle.blob_layout(256, 128, 4)
    rb = 256 * 4 // 8
    for i in (0, 17, 127):
        row = blob[lay["up"] + i * rb: lay["up"] + (i + 1) * rb]
        assert np.array_equal(oracle.unpack(row, 256, 4), parts["up"][i])
    s = blob[lay["s_down"]: lay["s_down"] + 4 * 256].view(np.float32)
    assert np.array_equal(s, parts["s_down"])
