"""Pins of the oracle's MXFP4 experts (E2M1 codes, one E8M0 scale per 32
codes of a row): the element and scale values against the format's
definition worked by hand, the packed byte order, an exact power-of-two
case, the float64 bound that a shifted or misread scale violates, the
expert stages and the whole tiny layer against the float64 pipeline."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.ref_f64 import expert64, matvec_qg, q8_0_f64, swiglu64, ulp32

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "mxfp4_examples.json")))
SPEC = synth.TINY_MX


def test_e2m1_values_match_the_definition():
    for c, v in GOLD["e2m1_values"].items():
        got = float(oracle.e2m1(int(c)))
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (c, got, v)


def test_e8m0_values_match_the_definition():
    for x, v in GOLD["e8m0_values"].items():
        got = float(oracle.e8m0(int(x)))
        if v == "NaN":
            assert math.isnan(got)
        else:
            assert got == 2.0 ** int(v[2:]), (x, got, v)
    # every finite byte is an exact power of two, the subnormal ones included
    for x in range(255):
        assert float(oracle.e8m0(x)) == math.ldexp(1.0, x - 127)


def test_unpack_byte_order_worked_examples():
    for case in GOLD["unpack_cases"]:
        b = np.frombuffer(bytes.fromhex(case["bytes_hex"]), np.uint8)
        n = len(case["twice_values"])
        assert oracle.unpack_mx(b, n).tolist() == case["twice_values"]


def test_unpack_round_trips_the_generator_packer():
    """Every code at every position of a block, packed by the generator's own
    packer, unpacks to twice its E2M1 value."""
    rows = np.array([[(j + r) % 16 for j in range(64)] for r in range(16)], np.uint8)
    packed = synth.pack_mx(rows)
    for r in range(16):
        want = [int(2 * GOLD["e2m1_values"][str(c)]) for c in rows[r]]
        assert oracle.unpack_mx(packed[r], 64).tolist() == want


def _rows_t_and_x(rng, R, n, x_lo=120, x_hi=136):
    codes = rng.integers(0, 16, size=(R, n)).astype(np.uint8)
    t = np.array([[int(2 * GOLD["e2m1_values"][str(c)]) for c in row] for row in codes], np.int8)
    x = rng.integers(x_lo, x_hi, size=(R, n // 32)).astype(np.uint8)
    return codes, t, x


def test_exact_when_every_step_is_exact():
    """Power-of-two activation scales and a few blocks: every product and sum
    of the chain is exact, so the result is the exact sum
    sum_b d_b * 2^(x_b - 127) * sum_j v_j q_j whatever the order; a missing
    halving, an exponent bias off by one or a block reading its neighbour's
    scale changes it."""
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = 32 * int(rng.integers(1, 5))
        _, t, x = _rows_t_and_x(rng, 1, n, 124, 131)
        q = rng.integers(-127, 128, n).astype(np.int8)
        d = (np.float32(2.0) ** rng.integers(-12, -4, n // 32)).astype(np.float32)
        exact = sum(Fraction(float(d[b])) * Fraction(2) ** (int(x[0, b]) - 127)
                    * Fraction(int(np.dot(t[0, 32 * b:32 * b + 32].astype(np.int64),
                                          q[32 * b:32 * b + 32].astype(np.int64))), 2)
                    for b in range(n // 32))
        got = oracle.row_dot_mx(t[0], q, d, x[0])
        assert Fraction(float(got)) == exact


def test_row_dot_within_float64_bound_and_sees_a_shifted_scale():
    rng = np.random.default_rng(6)
    R, n = 48, 6144
    _, t, x = _rows_t_and_x(rng, R, n)
    q = rng.integers(-127, 128, n).astype(np.int8)
    d = (rng.random(n // 32) * 0.03).astype(np.float32)
    gs = np.exp2(x.astype(np.float64) - 128).astype(np.float32)   # one scale per block, t = 2 v
    y64, bound = matvec_qg(t, gs, q, d)
    got = np.array([oracle.row_dot_mx(t[r], q, d, x[r]) for r in range(R)], np.float64)
    assert np.all(np.abs(got - y64) <= bound)
    shifted = np.array([oracle.row_dot_mx(t[r], q, d, np.roll(x[r], 1)) for r in range(R)], np.float64)
    assert np.any(np.abs(shifted - y64) > bound)
    off_by_one = np.array([oracle.row_dot_mx(t[r], q, d, x[r] + 1) for r in range(R)], np.float64)
    assert np.any(np.abs(off_by_one - y64) > bound)


def _parts64(parts):
    """Generator codes / scale bytes as the float64 model's integer codes
    (twice the E2M1 values) and per-block scales 2^(x - 128)."""
    out = {}
    for m in ("gate", "up", "down"):
        c = parts[m]
        out[m] = np.where(c >= 8, -1, 1) * np.asarray(synth.E2M1_MAG)[c & 7] * 2
        out[m] = out[m].astype(np.int64)
        out["s_" + m] = np.exp2(parts["s_" + m].astype(np.float64) - 128)
    return out


@pytest.fixture(scope="module")
def tiny():
    d = synth.tiny_layer(seed=0, S=4, spec=SPEC)
    d["parts"] = [_parts64(synth.mx_expert(0, 0, e, SPEC)[1]) for e in range(SPEC.n_experts + 1)]
    return d


def test_mx_blob_layout():
    H, I = 6144, 2048
    lay = oracle.blob_layout(H, I, 4, 0, 1)
    assert lay == synth.blob_layout(H, I, 4, 0, 1)
    assert lay["total"] == 20054016   # 18 874 368 B of codes + 3 x 393 216 B of scale bytes, 256-aligned


def test_mx_expert_stages_against_float64(tiny):
    H, I = SPEC.hidden, SPEC.inter
    blobs = tiny["blobs"] + [tiny["shared"]]
    for t in range(tiny["x"].shape[0]):
        qx, dx = oracle.q8_0(tiny["x"][t])
        for e in range(SPEC.n_experts + 1):
            o = oracle.expert(blobs[e], H, I, 4, qx, dx, fmt=1)
            p = tiny["parts"][e]
            g64, gb = matvec_qg(p["gate"], p["s_gate"], qx, dx)
            u64, ub = matvec_qg(p["up"], p["s_up"], qx, dx)
            assert np.all(np.abs(o["g"] - g64) <= gb)
            assert np.all(np.abs(o["u"] - u64) <= ub)
            h64 = swiglu64(o["g"], o["u"])
            assert np.all(np.abs(o["h"] - h64) <= 4 * ulp32(h64))
            y64, yb = matvec_qg(p["down"], p["s_down"], o["qh"], o["dh"])
            assert np.all(np.abs(o["y"] - y64) <= yb)


def test_mx_layer_end_to_end_against_float64(tiny):
    out, idx, w = oracle.layer(SPEC, tiny["x"], tiny["router_w"], tiny["bias"], tiny["blobs"], tiny["shared"])
    H, I = SPEC.hidden, SPEC.inter
    flips = 0
    for t in range(tiny["x"].shape[0]):
        x = tiny["x"][t]
        qx, dx, nt = q8_0_f64(x)
        qx32, dx32 = oracle.q8_0(x)
        assert np.array_equal(np.where(nt, qx32, qx), qx32)
        lg = tiny["router_w"].astype(np.float64) @ x.astype(np.float64)
        sig = 1 / (1 + np.exp(-lg))
        wt = sig[idx[t]] / sig[idx[t]].sum() * SPEC.routed_scaling_factor
        ref = np.zeros(H)
        for k, e in enumerate(list(idx[t]) + [SPEC.n_experts]):
            blob = tiny["shared"] if e == SPEC.n_experts else tiny["blobs"][e]
            o32 = oracle.expert(blob, H, I, 4, qx32, dx32, fmt=1)
            r = expert64(tiny["parts"][e], qx, dx, qh_override=o32["qh"])
            flips += r["nflips"]
            ref += (wt[k] if k < SPEC.top_k else 1.0) * r["y"]
        rel = np.linalg.norm(out[t] - ref) / np.linalg.norm(ref)
        assert rel <= 1e-5, rel
        assert np.max(np.abs(out[t] - ref)) <= 1e-3 * np.sqrt(np.mean(ref ** 2))
    assert flips <= 2


def test_mx_format_is_refused_with_other_widths_or_groups():
    qx, dx = oracle.q8_0(np.ones(256, np.float32))
    blob = np.zeros(synth.TINY_MX.blob_bytes, np.uint8)
    for bits, group in ((8, 0), (4, 64)):
        with pytest.raises(oracle.OracleError):
            oracle.expert(blob, 256, 128, bits, qx, dx, group=group, fmt=1)
