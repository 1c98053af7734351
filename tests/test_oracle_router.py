"""Pins of the oracle's router: the worked examples the router article
prints, equivalence with a full stable sort, gate-weight invariants, and
exact cases of the logit."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from fractions import Fraction

from tests.ref_f64 import U32, full_sort_topk, rn32, sigmoid64

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "router_worked_examples.json")))


def test_worked_example_exact_tie_goes_to_lower_id():
    ex = GOLDEN["tie_break"]
    idx, w, _ = oracle.select(np.float32(ex["logits"]), np.float32(ex["bias"]), ex["top_k"], 1.0)
    assert sorted(idx.tolist()) == ex["expected_sorted_set"]
    assert int(idx[-1]) == ex["expected_last"]


def test_worked_example_near_tie_flips_under_nudge():
    ex = GOLDEN["near_tie"]
    lg = np.float32(ex["logits"])
    before, _, _ = oracle.select(lg, np.float32(ex["bias"]), ex["top_k"], 1.0)
    lg2 = np.array(ex["logits"], np.float64)
    lg2[ex["nudge_expert"]] += ex["nudge"]
    after, _, _ = oracle.select(lg2.astype(np.float32), np.float32(ex["bias"]), ex["top_k"], 1.0)
    assert int(before[-1]) == ex["expected_last_before"]
    assert int(after[-1]) == ex["expected_last_after"]


def test_worked_example_full_sort_equivalence():
    ex = GOLDEN["equivalence"]
    rng = np.random.default_rng(5)
    logits = rng.normal(size=(64, 256))
    bias = rng.normal(scale=0.05, size=256)
    lg32, b32 = logits.astype(np.float32), bias.astype(np.float32)
    matched = 0
    for t in range(64):
        idx, w, _ = oracle.select(lg32[t], b32, ex["top_k"], 1.0)
        ref = full_sort_topk(sigmoid64(lg32[t]) + b32.astype(np.float64), ex["top_k"])
        matched += int(np.array_equal(idx, ref))
        assert abs(float(w.astype(np.float64).sum()) - 1.0) <= 2 * ex["top_k"] * U32
    assert matched == ex["expected_tokens_matched"]


def test_worked_example_non_finite_is_rejected():
    ex = GOLDEN["non_finite"]
    rng = np.random.default_rng(5)
    logits = rng.normal(size=(64, 256)).astype(np.float32)
    logits[ex["token"], ex["expert"]] = np.nan
    with pytest.raises(oracle.OracleError) as e:
        oracle.select(logits[ex["token"]], np.zeros(256, np.float32), 8, 1.0)
    assert e.value.rc == oracle.ENONFINITE
    bias = np.zeros(256, np.float32)
    bias[4] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.select(logits[0], bias, 8, 1.0)


def test_selection_equals_stable_full_sort_of_binary32_scores():
    rng = np.random.default_rng(11)
    for t in range(200):
        lg = rng.normal(size=256).astype(np.float32)
        b = (rng.normal(size=256) * 0.01).astype(np.float32)
        if t % 7 == 0:   # many exact ties
            lg = np.round(lg * 2).astype(np.float32) / 2
            b[:] = 0
        idx, _, sig = oracle.select(lg, b, 8, 2.5)
        score = (sig + b).astype(np.float32)
        assert np.array_equal(idx, full_sort_topk(score, 8))


def test_gate_weight_invariants():
    rng = np.random.default_rng(12)
    rsf = np.float32(2.5)
    for _ in range(100):
        lg = rng.normal(size=64).astype(np.float32)
        b = (rng.normal(size=64) * 0.05).astype(np.float32)
        idx, w, sig = oracle.select(lg, b, 6, rsf)
        # weights sum to routed_scaling_factor
        assert abs(float(w.astype(np.float64).sum()) - 2.5) <= 2 * 6 * 2.5 * U32 * 2
        # ratios follow the unbiased sigmoids (the bias only ranks)
        s = sig[idx].astype(np.float64)
        ratio = w.astype(np.float64) / w[0]
        assert np.allclose(ratio, s / s[0], rtol=8 * U32, atol=0)
        # unnormalised form
        _, w0, _ = oracle.select(lg, b, 6, rsf, norm=0)
        assert np.array_equal(w0, (sig[idx] * rsf).astype(np.float32))
    idx, w, sig = oracle.select(rng.normal(size=16).astype(np.float32), None, 1, rsf)
    assert w[0] == rsf
    assert oracle.sigmoid(np.float32([0.0]))[0] == 0.5


def test_logit_exact_cases():
    H = 512
    rng = np.random.default_rng(13)
    x = rng.normal(size=H).astype(np.float32)
    for h in (0, 3, 4, 255, 256, 300, 511):
        w = np.zeros(H, np.float32)
        w[h] = 1.0
        assert oracle.router_logit(x, w) == x[h]
    xi = rng.integers(-3, 4, H).astype(np.float32)
    wi = rng.integers(-3, 4, H).astype(np.float32)
    assert oracle.router_logit(xi, wi) == np.float32(np.dot(xi.astype(np.int64), wi.astype(np.int64)))


def test_logit_within_float64_bound():
    spec = synth.GLM
    x = synth.hidden_states(0, 0, 2, spec.hidden)
    W = synth.router_weights(0, 0, spec)[:32]
    for t in range(2):
        for e in range(32):
            got = float(oracle.router_logit(x[t], W[e]))
            prod = x[t].astype(np.float64) * W[e].astype(np.float64)
            bound = (spec.hidden // 256 * 4 + 7) * U32 * np.abs(prod).sum()
            assert abs(got - prod.sum()) <= bound


def test_route_on_tiny_layer_is_full_sort_of_its_scores():
    d = synth.tiny_layer()
    spec = d["spec"]
    idx, w, logits, sig = oracle.route(spec, d["x"], d["router_w"], d["bias"])
    for t in range(idx.shape[0]):
        score = (sig[t] + d["bias"]).astype(np.float32)
        assert np.array_equal(idx[t], full_sort_topk(score, spec.top_k))
        lg = np.array([oracle.router_logit(d["x"][t], d["router_w"][e]) for e in range(spec.n_experts)])
        assert np.array_equal(lg, logits[t])


def test_logit_matches_exact_rational_model_of_the_reduction_order():
    """Each binary32 rounding of the stated order (64 strided fmaf chains, then
    six xor-butterfly additions) modelled exactly in rationals."""
    rng = np.random.default_rng(14)
    for H in (256, 512):
        for _ in range(3):
            x = rng.normal(size=H).astype(np.float32)
            w = (rng.normal(size=H) * rng.lognormal(size=H)).astype(np.float32)
            p = []
            for l in range(64):
                a = Fraction(0)
                for j in range(H // 256):
                    for c in range(4):
                        h = 256 * j + 4 * l + c
                        a = rn32(Fraction(float(x[h])) * Fraction(float(w[h])) + a)
                p.append(a)
            for o in (32, 16, 8, 4, 2, 1):
                p = [rn32(p[l] + p[l ^ o]) for l in range(64)]
            assert Fraction(float(oracle.router_logit(x, w))) == p[0]
