"""Pins of the oracle's group-scaled int4 weights (one f32 scale per 64
codes of a row; JustVugg/colibri, "Get started" and "Other supported
models"): the blob layout's closed form, an exact special case whose value
does not depend on the rounding order, the reduction to the per-row chain
when every group of a row has the same power-of-two scale, the float64
bound on long rows, and the expert and whole layer against the float64
brute force."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.ref_f64 import block_isums, expert64, matvec_qg, q8_0_f64, ulp32

SPEC = synth.TINY_GS64


def test_glm_gs64_blob_layout_closed_form():
    H, I = 6144, 2048
    lay = oracle.blob_layout(H, I, 4, 64)
    codes = H * I // 2
    assert lay["up"] == codes and lay["down"] == 2 * codes and lay["s_gate"] == 3 * codes
    assert lay["s_up"] - lay["s_gate"] == 4 * I * (H // 64)
    assert lay["s_down"] - lay["s_up"] == 4 * I * (H // 64)
    assert lay["total"] - lay["s_down"] == 4 * H * (I // 64)
    assert lay["total"] == 21_233_664
    assert synth.GLM_GS64.blob_bytes == lay["total"]
    # group 0 is the per-row layout
    assert oracle.blob_layout(H, I, 4, 0) == oracle.blob_layout(H, I, 4)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_exact_when_every_step_is_exact(group):
    """Power-of-two block and group scales and short rows: every product and
    partial sum is exact in binary32, so the result is the exact sum
    sum_b d_b s_g(b) isum_b whatever the order; a wrong group index or a
    dropped scale changes it."""
    rng = np.random.default_rng(11 + group)
    n = 256
    for _ in range(50):
        w = rng.integers(-8, 8, n).astype(np.int8)
        q = rng.integers(-127, 128, n).astype(np.int8)
        d = np.float32(2.0) ** rng.integers(-2, 1, n // 32).astype(np.float32)
        gs = np.float32(2.0) ** rng.integers(-2, 1, n // group).astype(np.float32)
        isum = block_isums(w, q)
        exact = sum(Fraction(float(d[b])) * Fraction(float(gs[32 * b // group])) * int(isum[b])
                    for b in range(n // 32))
        got = oracle.row_dot_g(w, q, d, gs, group)
        assert Fraction(float(got)) == exact


def test_equal_power_of_two_group_scales_reduce_to_the_row_chain():
    """All groups of a row scaled by the same 2^k: the group chain is the
    per-row chain times 2^k, step by step (scaling by a power of two is
    exact), so it equals the per-row result with row scale 2^k bit for bit."""
    rng = np.random.default_rng(12)
    for n in (64, 6144):
        for k in (-9, -6, 0):
            w = rng.integers(-8, 8, n).astype(np.int8)
            q = rng.integers(-127, 128, n).astype(np.int8)
            d = (rng.random(n // 32) * 0.05).astype(np.float32)
            s = np.float32(2.0 ** k)
            gs = np.full(n // 64, s, np.float32)
            assert oracle.row_dot_g(w, q, d, gs, 64) == oracle.row_dot(w, q, d, s)


def test_row_dot_g_within_float64_bound():
    rng = np.random.default_rng(13)
    R, n = 48, 6144
    codes = rng.integers(-7, 8, size=(R, n)).astype(np.int8)
    q = rng.integers(-127, 128, n).astype(np.int8)
    d = (rng.random(n // 32) * 0.03).astype(np.float32)
    gs = (0.001 + rng.random((R, n // 64)) * 0.01).astype(np.float32)
    y64, bound = matvec_qg(codes, gs, q, d)
    got = np.array([oracle.row_dot_g(codes[r], q, d, gs[r], 64) for r in range(R)], np.float64)
    assert np.all(np.abs(got - y64) <= bound)
    # the bound is tight enough to see a shifted group index
    shifted = np.array([oracle.row_dot_g(codes[r], q, d, np.roll(gs[r], 1), 64) for r in range(R)], np.float64)
    assert np.any(np.abs(shifted - y64) > bound)


@pytest.fixture(scope="module")
def tiny():
    d = synth.tiny_layer(seed=0, S=4, spec=SPEC)
    d["parts"] = [synth.gaussian_expert(0, 0, e, SPEC)[1] for e in range(SPEC.n_experts + 1)]
    return d


def test_gs64_expert_stages_against_float64(tiny):
    H, I, b, G = SPEC.hidden, SPEC.inter, SPEC.wbits, SPEC.group
    blobs = tiny["blobs"] + [tiny["shared"]]
    for t in range(tiny["x"].shape[0]):
        qx, dx = oracle.q8_0(tiny["x"][t])
        for e in range(SPEC.n_experts + 1):
            o = oracle.expert(blobs[e], H, I, b, qx, dx, group=G)
            p = tiny["parts"][e]
            assert p["s_gate"].shape == (I, H // G) and p["s_down"].shape == (H, I // G)
            g64, gb = matvec_qg(p["gate"], p["s_gate"], qx, dx)
            u64, ub = matvec_qg(p["up"], p["s_up"], qx, dx)
            assert np.all(np.abs(o["g"] - g64) <= gb)
            assert np.all(np.abs(o["u"] - u64) <= ub)
            y64, yb = matvec_qg(p["down"], p["s_down"], o["qh"], o["dh"])
            assert np.all(np.abs(o["y"] - y64) <= yb)


def test_gs64_layer_end_to_end_against_float64(tiny):
    """Whole group-scaled layer vs the float64 pipeline (its own Q8_0
    decisions; h codes within 1e-4 of a rounding boundary follow the oracle)."""
    out, idx, w = oracle.layer(SPEC, tiny["x"], tiny["router_w"], tiny["bias"], tiny["blobs"], tiny["shared"])
    H, I, b, G = SPEC.hidden, SPEC.inter, SPEC.wbits, SPEC.group
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
            o32 = oracle.expert(blob, H, I, b, qx32, dx32, group=G)
            r = expert64(tiny["parts"][e], qx, dx, qh_override=o32["qh"])
            flips += r["nflips"]
            ref += (wt[k] if k < SPEC.top_k else 1.0) * r["y"]
        rel = np.linalg.norm(out[t] - ref) / np.linalg.norm(ref)
        assert rel <= 1e-5, rel
        assert np.max(np.abs(out[t] - ref)) <= 1e-3 * np.sqrt(np.mean(ref ** 2))
    assert flips <= 2


def test_group_changes_the_result_and_per_row_blobs_still_work(tiny):
    """The same codes read with group scales differ from the per-row layer
    (the group path is taken), and group 0 keeps the per-row definition."""
    per_row = synth.tiny_layer(seed=0, S=4)
    out_row, _, _ = oracle.layer(synth.TINY, per_row["x"], per_row["router_w"], per_row["bias"],
                                 per_row["blobs"], per_row["shared"])
    out_g, _, _ = oracle.layer(SPEC, tiny["x"], tiny["router_w"], tiny["bias"], tiny["blobs"], tiny["shared"])
    assert not np.array_equal(out_row, out_g)
    with pytest.raises(oracle.OracleError):
        qx, dx = oracle.q8_0(tiny["x"][0])
        oracle.expert(tiny["shared"], SPEC.hidden, SPEC.inter, 4, qx, dx, group=48)
