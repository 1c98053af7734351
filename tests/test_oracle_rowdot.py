"""Pins of the oracle's integer block dots and binary32 row dot: exact
integer sums, an exact rational model of the block chain on small rows, and
the float64 bound on larger ones."""
from fractions import Fraction

import numpy as np

import oracle
from tests.ref_f64 import block_isums, matvec_q, rn32


def test_block_isum_exact_including_extremes():
    rng = np.random.default_rng(2)
    for _ in range(200):
        w = rng.integers(-128, 128, 32).astype(np.int8)
        q = rng.integers(-127, 128, 32).astype(np.int8)
        assert oracle.block_isum(w, q) == int(np.dot(w.astype(np.int64), q.astype(np.int64)))
    w = np.full(32, -128, np.int8)
    q = np.full(32, -127, np.int8)
    assert oracle.block_isum(w, q) == 32 * 128 * 127


def test_row_dot_matches_exact_rational_model_of_the_block_chain():
    rng = np.random.default_rng(3)
    for n in (32, 96, 256):
        for _ in range(20):
            w = rng.integers(-8, 8, n).astype(np.int8)
            q = rng.integers(-127, 128, n).astype(np.int8)
            d = (rng.random(n // 32) * 0.05).astype(np.float32)
            s = np.float32(rng.random() * 0.01)
            isum = block_isums(w, q)
            acc = Fraction(0)
            for b in range(n // 32):
                acc = rn32(Fraction(float(d[b])) * int(isum[b]) + acc)
            want = rn32(acc * Fraction(float(s)))
            got = oracle.row_dot(w, q, d, s)
            assert Fraction(float(got)) == want


def test_single_block_closed_form():
    w = np.zeros(128, np.int8)
    q = np.zeros(128, np.int8)
    w[64:96] = 3
    q[64:96] = -5
    d = np.float32([0.25, 0.5, 0.125, 2.0])
    got = oracle.row_dot(w, q, d, np.float32(0.5))
    assert got == np.float32(32 * 3 * -5 * 0.125 * 0.5)


def test_row_dot_within_float64_bound():
    rng = np.random.default_rng(4)
    R, n = 64, 6144
    codes = rng.integers(-7, 8, size=(R, n)).astype(np.int8)
    q = rng.integers(-127, 128, n).astype(np.int8)
    d = (rng.random(n // 32) * 0.03).astype(np.float32)
    s = (rng.random(R) * 0.01).astype(np.float32)
    y64, bound = matvec_q(codes, s, q, d)
    got = np.array([oracle.row_dot(codes[r], q, d, s[r]) for r in range(R)], np.float64)
    assert np.all(np.abs(got - y64) <= bound)
