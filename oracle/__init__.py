"""CPU oracle of the routed-expert MoE layer (ctypes wrapper of moe_oracle.c).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path never
imports it, and it shares no code with the HIP library.

Functions take and return numpy arrays; every call is a plain C loop over
the definitions in moe_oracle.c.  Two builds of that one source exist:
liboracle.so (single-threaded) and liboracle_omp.so (OpenMP: the loops over
independent tokens of route / forward run on several threads; each token's
arithmetic is the same sequential code, so the bits are the same).  The
layer-level calls take parallel=True to use the second build.  Errors come
back as OracleError carrying the C return code (-1 invalid argument, -2
non-finite input, -4 expert not resident).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
OMP_LIB_PATH = os.path.join(_HERE, "_build", "liboracle_omp.so")
# a test may point the wrapper at another build of the same source
LIB_OVERRIDE = os.environ.get("ORACLE_LIB_OVERRIDE")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]
# the multi-threaded build: the same flags plus OpenMP (the token loops)
OMP_CFLAGS = CFLAGS + ["-fopenmp"]

EINVAL, ENONFINITE, ENOTRESIDENT = -1, -2, -4


class OracleError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what}: oracle error {rc}")
        self.rc = rc


def _compile(path: str, flags, force: bool) -> str:
    if force or not os.path.exists(path):
        os.makedirs(os.path.dirname(path), exist_ok=True)
        tmp = path + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *flags, os.path.join(_HERE, "moe_oracle.c"), "-lm", "-o", tmp])
        os.replace(tmp, path)
    return path


def build(force: bool = False) -> str:
    """Compiles moe_oracle.c into oracle/_build/liboracle.so and, with
    OpenMP, liboracle_omp.so; returns the first."""
    _compile(OMP_LIB_PATH, OMP_CFLAGS, force)
    return _compile(LIB_PATH, CFLAGS, force)


_lib = None
_omp_lib = None
P = ctypes.c_void_p
I32 = ctypes.c_int
F32 = ctypes.c_float


def lib(parallel: bool = False):
    """The single-threaded build, or with parallel the OpenMP build."""
    global _lib, _omp_lib
    if parallel:
        if _omp_lib is None:
            build()
            _omp_lib = _bind(ctypes.CDLL(OMP_LIB_PATH))
        return _omp_lib
    if _lib is None:
        _lib = _bind(ctypes.CDLL(LIB_OVERRIDE or build()))
    return _lib


def threads(n: int = 0) -> int:
    """Threads of the OpenMP build's token loops: n > 0 sets them; returns
    the count in use."""
    return int(lib(True).oq_threads(int(n)))


def _bind(L):
    """Declares the C signatures on a loaded build."""
    sig = {
        "oq_expf": (F32, [F32]),
        "oq_sigmoid": (F32, [F32]),
        "oq_swiglu": (F32, [F32, F32]),
        "oq_expf_n": (None, [P, P, ctypes.c_uint64]),
        "oq_sigmoid_n": (None, [P, P, ctypes.c_uint64]),
        "oq_swiglu_n": (None, [P, P, P, ctypes.c_uint64]),
        "oq_q8_0": (None, [P, I32, P, P]),
        "oq_unpack": (None, [P, I32, I32, P]),
        "oq_blob_layout": (None, [I32, I32, I32, P]),
        "oq_block_isum": (ctypes.c_int32, [P, P]),
        "oq_row_dot": (F32, [P, P, P, I32, F32]),
        "oq_router_logit": (F32, [P, P, I32]),
        "oq_select": (I32, [P, P, I32, I32, F32, I32, P, P, P]),
        "oq_expert": (I32, [P, I32, I32, I32, P, P, P, P, P, P, P, P]),
        "oq_moe_route": (I32, [I32, I32, I32, F32, I32, I32, P, P, P, P, P, P, P]),
        "oq_moe_forward": (I32, [I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P]),
        "oq_blob_layout_g": (None, [I32, I32, I32, I32, P]),
        "oq_row_dot_g": (F32, [P, P, P, I32, P, I32]),
        "oq_expert_g": (I32, [P, I32, I32, I32, I32, P, P, P, P, P, P, P, P]),
        "oq_moe_forward_g": (I32, [I32, I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P]),
        "oq_threads": (I32, [I32]),
        "oq_e2m1": (F32, [I32]),
        "oq_e8m0": (F32, [I32]),
        "oq_unpack_mx": (None, [P, I32, P]),
        "oq_row_dot_mx": (F32, [P, P, P, I32, P]),
        "oq_blob_layout_mx": (None, [I32, I32, P]),
        "oq_expert_f": (I32, [P, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P]),
        "oq_moe_forward_f": (I32, [I32, I32, I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise OracleError(rc, what)


# ---------------------------------------------------------------- scalars
def expf(v) -> np.ndarray:
    v = _c(v, np.float32)
    y = np.empty_like(v)
    lib().oq_expf_n(_p(v), _p(y), v.size)
    return y


def sigmoid(v) -> np.ndarray:
    v = _c(v, np.float32)
    y = np.empty_like(v)
    lib().oq_sigmoid_n(_p(v), _p(y), v.size)
    return y


def swiglu(g, u) -> np.ndarray:
    g, u = _c(g, np.float32), _c(u, np.float32)
    assert g.shape == u.shape
    h = np.empty_like(g)
    lib().oq_swiglu_n(_p(g), _p(u), _p(h), g.size)
    return h


# ---------------------------------------------------------------- vectors
def q8_0(v) -> tuple[np.ndarray, np.ndarray]:
    v = _c(v, np.float32)
    n = v.shape[-1]
    flat = v.reshape(-1, n)
    q = np.empty(flat.shape, np.int8)
    d = np.empty((flat.shape[0], n // 32), np.float32)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        qr = np.empty(n, np.int8)
        dr = np.empty(n // 32, np.float32)
        lib().oq_q8_0(_p(row), n, _p(qr), _p(dr))
        q[r], d[r] = qr, dr
    return q.reshape(v.shape), d.reshape(v.shape[:-1] + (n // 32,))


def unpack(src, n: int, bits: int) -> np.ndarray:
    src = _c(src, np.uint8)
    assert src.size * 8 >= n * bits
    out = np.empty(n, np.int8)
    lib().oq_unpack(_p(src), n, bits, _p(out))
    return out


def blob_layout(H: int, I: int, bits: int, group: int = 0, fmt: int = 0) -> dict:
    """Section offsets of an expert blob; group > 0: group-scaled scales;
    fmt = 1: MXFP4 (4-bit codes, one E8M0 byte per 32 codes of a row)."""
    off = np.zeros(7, np.uint64)
    if fmt == 1:
        lib().oq_blob_layout_mx(H, I, _p(off))
    else:
        lib().oq_blob_layout_g(H, I, bits, group, _p(off))
    keys = ("gate", "up", "down", "s_gate", "s_up", "s_down", "total")
    return {k: int(v) for k, v in zip(keys, off)}


def block_isum(w, q) -> int:
    w, q = _c(w, np.int8), _c(q, np.int8)
    assert w.size == 32 and q.size == 32
    return int(lib().oq_block_isum(_p(w), _p(q)))


def row_dot(w, q, d, scale: float) -> np.float32:
    w, q, d = _c(w, np.int8), _c(q, np.int8), _c(d, np.float32)
    n = w.size
    assert q.size == n and d.size == n // 32
    return np.float32(lib().oq_row_dot(_p(w), _p(q), _p(d), n, float(scale)))


def row_dot_g(w, q, d, gs, group: int) -> np.float32:
    """Row dot with one scale per `group` codes (gs[n / group])."""
    w, q, d, gs = _c(w, np.int8), _c(q, np.int8), _c(d, np.float32), _c(gs, np.float32)
    n = w.size
    assert q.size == n and d.size == n // 32 and gs.size == n // group
    return np.float32(lib().oq_row_dot_g(_p(w), _p(q), _p(d), n, _p(gs), int(group)))


def e2m1(code: int) -> np.float32:
    """Value of a 4-bit E2M1 code."""
    return np.float32(lib().oq_e2m1(int(code)))


def e8m0(x: int) -> np.float32:
    """Value of an E8M0 scale byte (NaN for 255)."""
    return np.float32(lib().oq_e8m0(int(x)))


def unpack_mx(src, n: int) -> np.ndarray:
    """Twice the E2M1 values of the n codes of an MXFP4 row, as int8."""
    src = _c(src, np.uint8)
    assert src.size * 2 >= n
    out = np.empty(n, np.int8)
    lib().oq_unpack_mx(_p(src), n, _p(out))
    return out


def row_dot_mx(t, q, d, x) -> np.float32:
    """Row dot of an MXFP4 row (t from unpack_mx) with a Q8_0 vector; x the
    row's E8M0 bytes, one per 32 codes."""
    t, q, d, x = _c(t, np.int8), _c(q, np.int8), _c(d, np.float32), _c(x, np.uint8)
    n = t.size
    assert q.size == n and d.size == n // 32 and x.size == n // 32
    return np.float32(lib().oq_row_dot_mx(_p(t), _p(q), _p(d), n, _p(x)))


def router_logit(x, w) -> np.float32:
    x, w = _c(x, np.float32), _c(w, np.float32)
    return np.float32(lib().oq_router_logit(_p(x), _p(w), x.size))


def select(logits, bias, K: int, rsf: float, norm: int = 1):
    """(idx[K] int32, w[K] f32, sig[E] f32) for one token's logits."""
    logits = _c(logits, np.float32)
    E = logits.size
    bias = None if bias is None else _c(bias, np.float32)
    idx = np.empty(K, np.int32)
    w = np.empty(K, np.float32)
    sig = np.empty(E, np.float32)
    rc = lib().oq_select(_p(logits), _p(bias), E, K, float(rsf), int(norm), _p(idx), _p(w), _p(sig))
    _check(rc, "select")
    return idx, w, sig


def expert(blob, H: int, I: int, bits: int, qx, dx, group: int = 0, fmt: int = 0) -> dict:
    """One SwiGLU expert on one token; returns y and the intermediates."""
    blob = _c(blob, np.uint8)
    qx, dx = _c(qx, np.int8), _c(dx, np.float32)
    out = {"y": np.empty(H, np.float32), "g": np.empty(I, np.float32), "u": np.empty(I, np.float32),
           "h": np.empty(I, np.float32), "qh": np.empty(I, np.int8), "dh": np.empty(I // 32, np.float32)}
    rc = lib().oq_expert_f(_p(blob), H, I, bits, int(group), int(fmt), _p(qx), _p(dx), _p(out["y"]),
                           _p(out["g"]), _p(out["u"]), _p(out["h"]), _p(out["qh"]), _p(out["dh"]))
    _check(rc, "expert")
    return out


# ---------------------------------------------------------------- layer
def route(spec, x, router_w, bias, parallel: bool = False):
    """Routing of x [S,H]: (idx [S,K] int32, w [S,K] f32, logits [S,E], sig [S,E])."""
    x = _c(x, np.float32)
    S = x.shape[0]
    E, K = spec.n_experts, spec.top_k
    router_w = _c(router_w, np.float32)
    bias = None if bias is None else _c(bias, np.float32)
    idx = np.empty((S, K), np.int32)
    w = np.empty((S, K), np.float32)
    logits = np.empty((S, E), np.float32)
    sig = np.empty((S, E), np.float32)
    rc = lib(parallel).oq_moe_route(spec.hidden, E, K, float(spec.routed_scaling_factor),
                            int(spec.norm_topk_prob), S, _p(x), _p(router_w), _p(bias),
                            _p(idx), _p(w), _p(logits), _p(sig))
    _check(rc, "route")
    return idx, w, logits, sig


def forward(spec, x, idx, w, blobs, shared_blob, parallel: bool = False):
    """Expert FFNs + combine for x [S,H] with given routing; blobs[e] may be None."""
    x = _c(x, np.float32)
    S = x.shape[0]
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    keep = [None if b is None else _c(b, np.uint8) for b in blobs]
    ptrs = (ctypes.c_void_p * spec.n_experts)(*[None if b is None else b.ctypes.data for b in keep])
    sh = None if shared_blob is None else _c(shared_blob, np.uint8)
    out = np.empty((S, spec.hidden), np.float32)
    rc = lib(parallel).oq_moe_forward_f(spec.hidden, spec.inter, spec.n_experts, spec.top_k, spec.n_shared,
                                        spec.wbits, int(getattr(spec, "group", 0)), int(getattr(spec, "fmt", 0)), S,
                                        _p(x), _p(idx), _p(w), ptrs, _p(sh), _p(out))
    _check(rc, "forward")
    return out


def layer(spec, x, router_w, bias, blobs, shared_blob, parallel: bool = False):
    """Whole layer: returns (out [S,H], idx [S,K], w [S,K])."""
    idx, w, _, _ = route(spec, x, router_w, bias, parallel)
    return forward(spec, x, idx, w, blobs, shared_blob, parallel), idx, w
