"""Pins of the oracle's expert FFN and whole layer against the float64
brute force in ref_f64 (stage by stage and end to end), special cases that
reduce to a single expert, and the error contract."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.ref_f64 import U32, expert64, matvec_q, q8_0_f64, swiglu64, ulp32

SPEC = synth.TINY


@pytest.fixture(scope="module")
def tiny():
    d = synth.tiny_layer(seed=0, S=4)
    d["parts"] = [synth.gaussian_expert(0, 0, e, SPEC)[1] for e in range(SPEC.n_experts + 1)]
    return d


def _check_q8(v, q, d):
    """Q8_0 block rule checked in float64 against the values it quantised."""
    v = np.asarray(v, np.float64)
    dd = np.repeat(np.asarray(d, np.float64), 32)
    amax = np.abs(v.reshape(-1, 32)).max(1)
    assert np.all(np.abs(np.asarray(d, np.float64) - amax / 127) <= ulp32(amax / 127) / 2)
    assert np.all(np.abs(v - dd * q) <= dd * (0.5 + 2.0 ** -16))


def test_expert_stages_against_float64(tiny):
    H, I, b = SPEC.hidden, SPEC.inter, SPEC.wbits
    blobs = tiny["blobs"] + [tiny["shared"]]
    for t in range(tiny["x"].shape[0]):
        qx, dx = oracle.q8_0(tiny["x"][t])
        _check_q8(tiny["x"][t], qx, dx)
        for e in range(SPEC.n_experts + 1):
            o = oracle.expert(blobs[e], H, I, b, qx, dx)
            p = tiny["parts"][e]
            g64, gb = matvec_q(p["gate"], p["s_gate"], qx, dx)
            u64, ub = matvec_q(p["up"], p["s_up"], qx, dx)
            assert np.all(np.abs(o["g"] - g64) <= gb)
            assert np.all(np.abs(o["u"] - u64) <= ub)
            h64 = swiglu64(o["g"], o["u"])
            assert np.all(np.abs(o["h"] - h64) <= 4 * ulp32(h64))
            _check_q8(o["h"], o["qh"], o["dh"])
            y64, yb = matvec_q(p["down"], p["s_down"], o["qh"], o["dh"])
            assert np.all(np.abs(o["y"] - y64) <= yb)


def test_combine_against_float64(tiny):
    idx, w, _, _ = oracle.route(SPEC, tiny["x"], tiny["router_w"], tiny["bias"])
    out = oracle.forward(SPEC, tiny["x"], idx, w, tiny["blobs"], tiny["shared"])
    H, I, b = SPEC.hidden, SPEC.inter, SPEC.wbits
    for t in range(tiny["x"].shape[0]):
        qx, dx = oracle.q8_0(tiny["x"][t])
        ys = [oracle.expert(tiny["blobs"][e], H, I, b, qx, dx)["y"].astype(np.float64) for e in idx[t]]
        ysh = oracle.expert(tiny["shared"], H, I, b, qx, dx)["y"].astype(np.float64)
        terms = np.array([w[t, k] * ys[k] for k in range(SPEC.top_k)])
        ref = terms.sum(0) + ysh
        bound = (SPEC.top_k + 2) * U32 * (np.abs(terms).sum(0) + np.abs(ysh))
        assert np.all(np.abs(out[t] - ref) <= bound)


def test_layer_end_to_end_against_float64(tiny):
    """Whole layer vs a float64 pipeline that takes its own quantisation
    decisions; h codes within 1e-4 of a rounding boundary follow the oracle."""
    out, idx, w = oracle.layer(SPEC, tiny["x"], tiny["router_w"], tiny["bias"], tiny["blobs"], tiny["shared"])
    H, I, b = SPEC.hidden, SPEC.inter, SPEC.wbits
    flips = 0
    for t in range(tiny["x"].shape[0]):
        x = tiny["x"][t]
        lg = tiny["router_w"].astype(np.float64) @ x.astype(np.float64)
        sig = 1 / (1 + np.exp(-lg))
        sel = np.lexsort((np.arange(SPEC.n_experts), -(sig + tiny["bias"])))[:SPEC.top_k]
        assert np.array_equal(sel, idx[t])
        wt = sig[sel] / sig[sel].sum() * SPEC.routed_scaling_factor
        assert np.allclose(wt, w[t], rtol=1e-6)
        qx, dx, nt = q8_0_f64(x)
        qx32, dx32 = oracle.q8_0(x)
        assert np.array_equal(np.where(nt, qx32, qx), qx32)
        ref = np.zeros(H)
        for k, e in enumerate(list(sel) + [SPEC.n_experts]):
            blob = tiny["shared"] if e == SPEC.n_experts else tiny["blobs"][e]
            o32 = oracle.expert(blob, H, I, b, qx32, dx32)
            r = expert64(tiny["parts"][e], qx, dx, qh_override=o32["qh"])
            flips += r["nflips"]
            ref += (wt[k] if k < SPEC.top_k else 1.0) * r["y"]
        rel = np.linalg.norm(out[t] - ref) / np.linalg.norm(ref)
        assert rel <= 1e-5, rel
        assert np.max(np.abs(out[t] - ref)) <= 1e-3 * np.sqrt(np.mean(ref ** 2))
    assert flips <= 2


def test_single_expert_special_case(tiny):
    spec = dataclasses.replace(SPEC, top_k=1, n_shared=0, routed_scaling_factor=1.0)
    out, idx, w = oracle.layer(spec, tiny["x"], tiny["router_w"], tiny["bias"], tiny["blobs"], None)
    assert np.all(w == 1.0)
    for t in range(4):
        qx, dx = oracle.q8_0(tiny["x"][t])
        y = oracle.expert(tiny["blobs"][idx[t, 0]], SPEC.hidden, SPEC.inter, SPEC.wbits, qx, dx)["y"]
        assert np.array_equal(out[t], y)


def test_tokens_are_independent(tiny):
    idx, w, _, _ = oracle.route(SPEC, tiny["x"], tiny["router_w"], tiny["bias"])
    full = oracle.forward(SPEC, tiny["x"], idx, w, tiny["blobs"], tiny["shared"])
    for t in range(4):
        one = oracle.forward(SPEC, tiny["x"][t:t + 1], idx[t:t + 1], w[t:t + 1], tiny["blobs"], tiny["shared"])
        assert np.array_equal(one[0], full[t])


def test_error_contract(tiny):
    x = tiny["x"].copy()
    idx, w, _, _ = oracle.route(SPEC, x, tiny["router_w"], tiny["bias"])
    bad = x.copy()
    bad[2, 7] = np.nan
    with pytest.raises(oracle.OracleError) as e:
        oracle.route(SPEC, bad, tiny["router_w"], tiny["bias"])
    assert e.value.rc == oracle.ENONFINITE
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(SPEC, bad, idx, w, tiny["blobs"], tiny["shared"])
    assert e.value.rc == oracle.ENONFINITE
    i2 = idx.copy()
    i2[1, 0] = SPEC.n_experts
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(SPEC, x, i2, w, tiny["blobs"], tiny["shared"])
    assert e.value.rc == oracle.EINVAL
    i3 = idx.copy()
    i3[1, 1] = i3[1, 0]
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(SPEC, x, i3, w, tiny["blobs"], tiny["shared"])
    assert e.value.rc == oracle.EINVAL
    blobs = list(tiny["blobs"])
    blobs[int(idx[0, 0])] = None
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(SPEC, x, idx, w, blobs, tiny["shared"])
    assert e.value.rc == oracle.ENOTRESIDENT
    empty = oracle.forward(SPEC, x[:0], idx[:0], w[:0], tiny["blobs"], tiny["shared"])
    assert empty.shape == (0, SPEC.hidden)


@pytest.mark.parametrize("bits", [8, 2])
def test_other_widths_stage_bounds(bits):
    spec = dataclasses.replace(SPEC, wbits=bits)
    blob, p = synth.gaussian_expert(1, 0, 5, spec)
    x = synth.hidden_states(1, 0, 1, spec.hidden)[0]
    qx, dx = oracle.q8_0(x)
    o = oracle.expert(blob, spec.hidden, spec.inter, bits, qx, dx)
    g64, gb = matvec_q(p["gate"], p["s_gate"], qx, dx)
    assert np.all(np.abs(o["g"] - g64) <= gb)
    y64, yb = matvec_q(p["down"], p["s_down"], o["qh"], o["dh"])
    assert np.all(np.abs(o["y"] - y64) <= yb)
