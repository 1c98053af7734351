"""Pins of the oracle at the extremes of the code formats (the inputs the GPU
edge-case parity tests use): every code of a width, its minimum included,
unpacks from the blob to the generator's value at every block position;
block sums reach their largest magnitudes exactly; and the expert stages on
those inputs stay within the float64 bounds."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.ref_f64 import matvec_q, matvec_qg, swiglu64, ulp32

SPECS = {
    "int8": dataclasses.replace(synth.TINY, wbits=8),
    "int4": synth.TINY,
    "int2": dataclasses.replace(synth.TINY, wbits=2),
    "gs64": synth.TINY_GS64,
}


def _unpack_matrix(blob, off, rows, cols, bits):
    rb = cols * bits // 8
    return np.stack([oracle.unpack(blob[off + r * rb: off + (r + 1) * rb], cols, bits) for r in range(rows)])


@pytest.mark.parametrize("name", list(SPECS))
def test_extreme_blob_codes_round_trip(name):
    spec = SPECS[name]
    H, I, b = spec.hidden, spec.inter, spec.wbits
    lo, hi = synth.FULL_RANGE[b]
    parts = synth.extreme_parts(4, 0, 1, spec)
    blob = synth.extreme_expert(4, 0, 1, spec)
    lay = oracle.blob_layout(H, I, b, spec.group)
    for name_m, rows, cols in (("gate", I, H), ("up", I, H), ("down", H, I)):
        got = _unpack_matrix(blob, lay[name_m], rows, cols, b)
        assert np.array_equal(got, parts[name_m])
        # the minimum sits at every position of a block in some row, and
        # both ends of the range occur
        pos = {int(p) for r in range(rows) for p in np.nonzero(got[r, :32] == lo)[0]
               if np.count_nonzero(got[r, :32] == lo) == 1}
        assert pos == set(range(32))
        assert got.min() == lo and got.max() == hi


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_largest_block_sums_are_exact(bits):
    lo, hi = synth.FULL_RANGE[bits]
    for qv in (127, -127):
        assert oracle.block_isum(np.full(32, lo, np.int8), np.full(32, qv, np.int8)) == 32 * lo * qv
        assert oracle.block_isum(np.full(32, hi, np.int8), np.full(32, qv, np.int8)) == 32 * hi * qv


def test_extreme_activations_quantise_to_127():
    x = synth.extreme_hidden_states(3, 0, 5, 512)
    qx, dx = oracle.q8_0(x)
    assert np.all(np.abs(qx) == 127)
    assert np.all(qx.reshape(5, 16, 32)[0, 0] == 127)      # block 0 of token 0: positive
    assert np.all(qx.reshape(5, 16, 32)[0, 1] == -127)     # block 1: negative


@pytest.mark.parametrize("name", list(SPECS))
def test_expert_stages_at_the_extremes(name):
    """The oracle's expert on edge-case weights and activations against the
    float64 brute force, stage by stage; h is constant over rows 32..63, so
    that block of Q8_0(h) is +-127 and the down sums reach the extremes."""
    spec = SPECS[name]
    H, I, b, G = spec.hidden, spec.inter, spec.wbits, spec.group
    mv = (lambda c, s, q, d: matvec_qg(c, s, q, d)) if G else matvec_q
    x = synth.extreme_hidden_states(9, 0, 2, H)
    parts = synth.extreme_parts(9, 0, 2, spec)
    blob = synth.extreme_expert(9, 0, 2, spec)
    for t in range(2):
        qx, dx = oracle.q8_0(x[t])
        o = oracle.expert(blob, H, I, b, qx, dx, group=G)
        g64, gb = mv(parts["gate"], parts["s_gate"], qx, dx)
        u64, ub = mv(parts["up"], parts["s_up"], qx, dx)
        assert np.all(np.abs(o["g"] - g64) <= gb)
        assert np.all(np.abs(o["u"] - u64) <= ub)
        assert np.all(o["h"][32:64] == o["h"][32])
        assert np.all(np.abs(o["qh"][32:64]) == 127)
        h64 = swiglu64(o["g"], o["u"])
        assert np.all(np.abs(o["h"] - h64) <= 4 * ulp32(h64))
        y64, yb = mv(parts["down"], parts["s_down"], o["qh"], o["dh"])
        assert np.all(np.abs(o["y"] - y64) <= yb)
