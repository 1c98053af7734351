"""Pins of the oracle's Q8_0 activation quantiser: closed forms of the block
rule and exact rational bounds on every code."""
from fractions import Fraction

import numpy as np

import oracle


def test_zero_block():
    q, d = oracle.q8_0(np.zeros(64, np.float32))
    assert np.all(q == 0) and np.all(d == 0)


def test_constant_block_saturates():
    for c in (1e-3, 0.7, 3.0, 1e6):
        q, d = oracle.q8_0(np.full(32, c, np.float32))
        assert np.all(q == 127), c
        q, d = oracle.q8_0(np.full(32, -c, np.float32))
        assert np.all(q == -127), c


def test_half_way_cases_round_away_from_zero():
    v = np.zeros(32, np.float32)
    v[0] = 127.0            # amax = 127 -> d = 1 exactly
    v[1], v[2], v[3], v[4] = 2.5, -2.5, 0.5, -0.5
    q, d = oracle.q8_0(v)
    assert d[0] == 1.0
    assert q[:5].tolist() == [127, 3, -3, 1, -1]


def test_codes_are_nearest_integers_and_scales_correctly_rounded():
    rng = np.random.default_rng(7)
    v = (rng.normal(size=(64, 32)) * rng.lognormal(size=(64, 1))).astype(np.float32)
    v[3, 5] = 0.0
    q, d = oracle.q8_0(v)
    for r in range(v.shape[0]):
        amax = max(abs(Fraction(float(t))) for t in v[r])
        dd = Fraction(float(d[r, 0]))
        # d is amax/127 rounded once to binary32
        assert abs(dd - amax / 127) <= Fraction(float(np.spacing(np.float32(d[r, 0])))) / 2
        j = int(np.argmax(np.abs(v[r])))
        assert abs(int(q[r, j])) == 127
        for k in range(32):
            exact = Fraction(float(v[r, k])) / dd
            # the code is the exact quotient rounded, up to the binary32 rounding of v/d
            assert abs(int(q[r, k]) - exact) <= Fraction(1, 2) + Fraction(1, 2 ** 16)
            assert int(q[r, k]) == 0 or np.sign(q[r, k]) == np.sign(v[r, k])


def test_reconstruction_bound():
    rng = np.random.default_rng(8)
    v = rng.normal(size=4096).astype(np.float32)
    q, d = oracle.q8_0(v)
    dd = np.repeat(d.astype(np.float64), 32)
    err = np.abs(v.astype(np.float64) - dd * q)
    assert np.all(err <= dd * (0.5 + 2.0 ** -16))
