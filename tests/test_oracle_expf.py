"""Pins of the oracle's exponential, logistic and SwiGLU functions against
float64 libm values, closed forms and the binary32 range limits."""
import numpy as np

import oracle
from tests.ref_f64 import sigmoid64, swiglu64, ulp32

F32MAX = float(np.finfo(np.float32).max)


def _sweep(stride=997):
    bits = np.arange(-2 ** 31, 2 ** 31, stride, dtype=np.int64).astype(np.int32)
    x = bits.view(np.float32)
    return x[np.isfinite(x) & (x > -104.0) & (x < 89.0)]


def test_expf_within_one_ulp_on_sweep():
    x = _sweep()
    y = oracle.expf(x).astype(np.float64)
    e = np.exp(x.astype(np.float64))
    ok = e <= F32MAX
    err = np.abs(y[ok] - e[ok]) / ulp32(e[ok])
    assert err.max() <= 1.0, err.max()


def test_expf_monotone_on_sweep():
    x = np.sort(_sweep(331))
    y = oracle.expf(x)
    assert np.all(y[1:] >= y[:-1])


def test_expf_closed_forms():
    assert oracle.expf(np.float32([0.0, -0.0])).tolist() == [1.0, 1.0]
    # exact powers of two reachable exactly: e^(k ln2) is not exact, but e^0 is;
    # the result for small |x| is 1 + x to within one ulp
    x = np.float32([1e-8, -1e-8, 2 ** -30])
    assert np.all(oracle.expf(x) == np.float32(1.0))


def test_expf_range_edges_match_correct_rounding():
    top = np.float32(float.fromhex("0x1.62e42ep+6"))
    above = np.nextafter(top, np.float32(100))
    low = np.float32(-float.fromhex("0x1.9fe368p+6"))
    below = np.nextafter(low, np.float32(-200))
    y = oracle.expf(np.array([top, above, low, below], np.float32))
    assert np.isfinite(y[0]) and y[0] <= F32MAX
    assert y[1] == np.inf
    assert y[2] == np.float32(2.0 ** -149)
    assert y[3] == 0.0
    # correctly rounded values from float64 at the same points
    ref = np.float32(np.exp(np.float64([top, low])))
    assert abs(float(y[0]) - float(ref[0])) <= float(ulp32(ref[0]))
    assert y[2] == ref[1]


def test_expf_nan_and_infinities():
    y = oracle.expf(np.float32([np.nan, np.inf, -np.inf]))
    assert np.isnan(y[0]) and y[1] == np.inf and y[2] == 0.0


def test_sigmoid_closed_forms_and_bound():
    assert oracle.sigmoid(np.float32([0.0]))[0] == np.float32(0.5)
    assert oracle.sigmoid(np.float32([200.0]))[0] == np.float32(1.0)
    assert oracle.sigmoid(np.float32([-200.0]))[0] == np.float32(0.0)
    x = _sweep(7919)
    x = x[np.abs(x) < 30]
    y = oracle.sigmoid(x).astype(np.float64)
    r = sigmoid64(x)
    err = np.abs(y - r) / ulp32(r)
    assert err.max() <= 3.0, err.max()


def test_swiglu_closed_forms_and_bound():
    h = oracle.swiglu(np.float32([0.0, 100.0, -200.0]), np.float32([3.0, 2.0, 5.0]))
    assert h[0] == 0.0 and h[1] == np.float32(200.0) and h[2] == 0.0
    rng = np.random.default_rng(1)
    g = rng.normal(size=20000).astype(np.float32) * 3
    u = rng.normal(size=20000).astype(np.float32)
    y = oracle.swiglu(g, u).astype(np.float64)
    r = swiglu64(g, u)
    err = np.abs(y - r) / ulp32(r)
    assert err.max() <= 4.0, err.max()
