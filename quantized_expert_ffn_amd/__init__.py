"""Python binding of libcolimoe, the routed-expert MoE layer for MI355X.

Argument marshalling only: every function here has the name of the C entry
point it calls (include/coli_moe.h), turns torch tensors into device
pointers and the current torch stream into a hipStream_t, and raises
ColiError on a non-zero return.  All computation happens in the HIP kernels.
Importing fails if the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libcolimoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m quantized_expert_ffn_amd.build` "
        "(or __graft_entry__.build()); the MoE layer has no non-HIP implementation")

# torch's HIP runtime is loaded first, so that the library's libamdhip64.so.7
# and libhsa-runtime64.so.1 resolve to the copies torch already holds (same
# sonames): loaded the other way round, the process ends up with the
# /opt/rocm runtime under torch as well, and the library's device queries
# have been seen to report no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

COLI_OK, COLI_EINVAL, COLI_ENONFINITE, COLI_EHIP, COLI_ENOTRESIDENT, COLI_EWORKSPACE = 0, -1, -2, -3, -4, -5
COLI_WFMT_INT, COLI_WFMT_MXFP4, COLI_MXFP4 = 0, 1, -4
COLI_MAX_TOKENS = 65536  # most tokens one call takes

EXPORTS = (
    "coli_moe_expert_bytes", "coli_moe_workspace_bytes", "coli_moe_route", "coli_moe_forward",
    "coli_moe_stage_experts", "coli_moe_status", "coli_moe_last_error", "coli_moe_timing_enable",
    "coli_moe_timing_read", "coli_moe_debug_unpack", "coli_moe_debug_block_dots",
    "coli_moe_debug_logits", "coli_moe_debug_expf", "coli_moe_debug_q8_0",
    "coli_moe_debug_force_path", "coli_moe_layer", "coli_moe_debug_mfma_i8",
    "coli_moe_roof_sink_words", "coli_moe_roof_stream_read", "coli_moe_roof_mfma_i8",
    "coli_moe_layer_noalloc", "coli_moe_debug_mfma_f8f6f4", "coli_moe_debug_route_wait",
    "coli_moe_debug_mfma_i8_16",
)

KIND_ROUTER_LOGITS, KIND_ROUTER_SELECT, KIND_GATEUP, KIND_DOWN, KIND_COMBINE = 0, 1, 2, 3, 4
KIND_LAYER, KIND_FORWARD_PERSISTENT, KIND_QUANT_X, KIND_GROUP = 5, 6, 7, 8
PATH_AUTO, PATH_MULTI, PATH_PERSISTENT, PATH_GROUPED = 0, 1, 2, 3


class coli_moe_dims(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("wbits", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float), ("norm_topk_prob", ctypes.c_int32),
        ("group_size", ctypes.c_int32), ("wformat", ctypes.c_int32),
    ]


class ColiError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib.coli_moe_last_error().decode(errors="replace")
        super().__init__(f"{where} failed ({code}): {msg}")
        self.code = code


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32
_D = ctypes.POINTER(coli_moe_dims)
_sigs = {
    "coli_moe_expert_bytes": (_SZ, [_D]),
    "coli_moe_workspace_bytes": (_SZ, [_D, _I32]),
    "coli_moe_route": (ctypes.c_int, [_D, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "coli_moe_forward": (ctypes.c_int, [_D, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "coli_moe_stage_experts": (ctypes.c_int, [_I32, _P, _P, _SZ, _P, _P]),
    "coli_moe_status": (ctypes.c_int, [_P, _P]),
    "coli_moe_last_error": (ctypes.c_char_p, []),
    "coli_moe_timing_enable": (ctypes.c_int, [_I32]),
    "coli_moe_timing_read": (ctypes.c_int, [_I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "coli_moe_debug_unpack": (ctypes.c_int, [_I32, _I32, _I32, _P, _P, _P]),
    "coli_moe_debug_block_dots": (ctypes.c_int, [_I32, _I32, _I32, _P, _P, _P, _P]),
    "coli_moe_debug_logits": (ctypes.c_int, [_D, _I32, _P, _P, _P, _P]),
    "coli_moe_debug_expf": (ctypes.c_int, [ctypes.c_int64, _P, _P, _P]),
    "coli_moe_debug_q8_0": (ctypes.c_int, [_I32, _I32, _P, _P, _P, _P]),
    "coli_moe_debug_force_path": (ctypes.c_int, [_I32]),
    "coli_moe_debug_route_wait": (ctypes.c_int, [ctypes.c_uint32, _I32]),
    "coli_moe_layer": (ctypes.c_int, [_D, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "coli_moe_debug_mfma_i8": (ctypes.c_int, [_P, _P, _P, _P]),
    "coli_moe_debug_mfma_i8_16": (ctypes.c_int, [_P, _P, _P, _P]),
    "coli_moe_debug_mfma_f8f6f4": (ctypes.c_int, [_I32, _I32, _P, _P, _P, _P, _P, _P]),
    "coli_moe_roof_sink_words": (_SZ, []),
    "coli_moe_roof_stream_read": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "coli_moe_roof_mfma_i8": (ctypes.c_int, [_I32, _P, _P]),
    "coli_moe_layer_noalloc": (ctypes.c_int, [_D, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


# ---------------------------------------------------------------- marshalling
def make_dims(spec) -> coli_moe_dims:
    """coli_moe_dims from any object with the dims' field names."""
    return coli_moe_dims(int(spec.hidden), int(spec.inter), int(spec.n_experts), int(spec.top_k),
                         int(spec.n_shared), int(spec.wbits), float(spec.routed_scaling_factor),
                         int(spec.norm_topk_prob), int(getattr(spec, "group", 0)), int(getattr(spec, "fmt", 0)))


def _dims(d):
    return ctypes.byref(d if isinstance(d, coli_moe_dims) else make_dims(d))


def _ptr(t, dtype=None, what="tensor"):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor or an address")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    return t.data_ptr()


def _dev(t, dtype, what):
    import torch
    if isinstance(t, torch.Tensor) and not t.is_cuda:
        raise ValueError(f"{what}: must be a device tensor")
    return _ptr(t, dtype, what)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _event_handle(ev, what, create_on=None):
    """hipEvent_t of a torch.cuda.Event (or a raw address, or None).  torch
    creates an event's HIP handle lazily, at its first record(); until then
    the handle is 0, which the library would read as "no event".  An event
    the library is to record is therefore created here first, by recording
    it on the stream it will be recorded on (create_on; the library records
    it again after its own work); an event the library is to wait for must
    already have been recorded."""
    if ev is None or isinstance(ev, int):
        return ev
    if not ev.cuda_event:
        if create_on is None:
            raise ValueError(f"{what}: this torch.cuda.Event has never been recorded, so it has no HIP event "
                             "to wait for")
        ev.record(create_on if not isinstance(create_on, int) else None)
        if not ev.cuda_event:
            raise RuntimeError(f"{what}: torch did not create the HIP event on record()")
    return ev.cuda_event


def _check(rc, where):
    if rc != COLI_OK:
        raise ColiError(rc, where)


def _nbytes(t):
    return t.numel() * t.element_size()


# ---------------------------------------------------------------- entry points
def coli_moe_expert_bytes(dims) -> int:
    return int(_lib.coli_moe_expert_bytes(_dims(dims)))


def coli_moe_workspace_bytes(dims, max_tokens: int) -> int:
    return int(_lib.coli_moe_workspace_bytes(_dims(dims), int(max_tokens)))


def coli_moe_route(dims, x, router_w, router_bias, topk_idx, topk_w, ws, stream=None):
    import torch
    S = x.shape[0]
    _check(_lib.coli_moe_route(
        _dims(dims), S, _dev(x, torch.float32, "x"), _dev(router_w, torch.float32, "router_w"),
        _dev(router_bias, torch.float32, "router_bias"), _dev(topk_idx, torch.int32, "topk_idx"),
        _dev(topk_w, torch.float32, "topk_w"), _dev(ws, torch.uint8, "ws"), _nbytes(ws),
        _stream(stream)), "coli_moe_route")


def coli_moe_forward(dims, x, topk_idx, topk_w, expert_blobs, shared_blob, out, ws,
                     pending_mask=None, pending_ready=None, stream=None):
    """expert_blobs: device int64 tensor [E] of blob addresses (0 = not
    resident); pending_mask: host sequence of E flags or None; pending_ready:
    a torch.cuda.Event (or raw hipEvent_t address) or None."""
    import numpy as np
    import torch
    S = x.shape[0]
    mask_ptr = None
    if pending_mask is not None:
        mask = np.ascontiguousarray(np.asarray(pending_mask, dtype=np.uint8))
        mask_ptr = mask.ctypes.data
    ev = _event_handle(pending_ready, "pending_ready")
    _check(_lib.coli_moe_forward(
        _dims(dims), S, _dev(x, torch.float32, "x"), _dev(topk_idx, torch.int32, "topk_idx"),
        _dev(topk_w, torch.float32, "topk_w"), _dev(expert_blobs, torch.int64, "expert_blobs"),
        _ptr(shared_blob, None, "shared_blob"), mask_ptr, ev, _dev(out, torch.float32, "out"),
        _dev(ws, torch.uint8, "ws"), _nbytes(ws), _stream(stream)), "coli_moe_forward")


def coli_moe_layer(dims, x, router_w, router_bias, expert_blobs, shared_blob, topk_idx, topk_w, out, ws,
                   stream=None):
    """Route + forward in one call (the kernel family is chosen as the header describes)."""
    import torch
    S = x.shape[0]
    _check(_lib.coli_moe_layer(
        _dims(dims), S, _dev(x, torch.float32, "x"), _dev(router_w, torch.float32, "router_w"),
        _dev(router_bias, torch.float32, "router_bias"), _dev(expert_blobs, torch.int64, "expert_blobs"),
        _ptr(shared_blob, None, "shared_blob"), _dev(topk_idx, torch.int32, "topk_idx"),
        _dev(topk_w, torch.float32, "topk_w"), _dev(out, torch.float32, "out"), _dev(ws, torch.uint8, "ws"),
        _nbytes(ws), _stream(stream)), "coli_moe_layer")


def coli_moe_layer_noalloc(dims, x, router_w, router_bias, expert_blobs, shared_blob, topk_idx, topk_w, out,
                           status_out=None, stream=None):
    """coli_moe_layer on the library's own scratch (no workspace argument);
    status_out: device int32/uint32 tensor of one element, or None."""
    import torch
    S = x.shape[0]
    st = None
    if status_out is not None:
        if status_out.numel() != 1 or status_out.dtype not in (torch.int32, torch.uint32):
            raise ValueError("status_out: one 32-bit device word")
        st = _dev(status_out, None, "status_out")
    _check(_lib.coli_moe_layer_noalloc(
        _dims(dims), S, _dev(x, torch.float32, "x"), _dev(router_w, torch.float32, "router_w"),
        _dev(router_bias, torch.float32, "router_bias"), _dev(expert_blobs, torch.int64, "expert_blobs"),
        _ptr(shared_blob, None, "shared_blob"), _dev(topk_idx, torch.int32, "topk_idx"),
        _dev(topk_w, torch.float32, "topk_w"), _dev(out, torch.float32, "out"), st, _stream(stream)),
        "coli_moe_layer_noalloc")


def coli_moe_stage_experts(host_src, dev_dst, bytes_each: int, copy_stream=None, done_event=None):
    n = len(host_src)
    if len(dev_dst) != n:
        raise ValueError("host_src and dev_dst differ in length")
    src = (ctypes.c_void_p * max(n, 1))(*[_ptr(s, None, "host_src") for s in host_src])
    dst = (ctypes.c_void_p * max(n, 1))(*[_ptr(d, None, "dev_dst") for d in dev_dst])
    ev = _event_handle(done_event, "done_event", create_on=copy_stream)
    _check(_lib.coli_moe_stage_experts(n, src, dst, int(bytes_each), _stream(copy_stream), ev),
           "coli_moe_stage_experts")


def coli_moe_status(ws, stream=None) -> int:
    """Synchronises the stream and returns (and clears) the device status code."""
    return int(_lib.coli_moe_status(_ptr(ws, None, "ws"), _stream(stream)))


def coli_moe_last_error() -> str:
    return _lib.coli_moe_last_error().decode(errors="replace")


def coli_moe_timing_enable(enable: bool) -> None:
    _check(_lib.coli_moe_timing_enable(1 if enable else 0), "coli_moe_timing_enable")


def coli_moe_timing_read(kind: int) -> tuple[float, int]:
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_lib.coli_moe_timing_read(int(kind), ctypes.byref(ms), ctypes.byref(n)), "coli_moe_timing_read")
    return ms.value, n.value


def coli_moe_debug_unpack(bits, n_rows, cols, src, out, stream=None):
    import torch
    _check(_lib.coli_moe_debug_unpack(bits, n_rows, cols, _ptr(src, None, "src"),
                                      _dev(out, torch.int8, "out"), _stream(stream)), "coli_moe_debug_unpack")


def coli_moe_debug_block_dots(bits, n_rows, cols, src, q, out, stream=None):
    import torch
    _check(_lib.coli_moe_debug_block_dots(bits, n_rows, cols, _ptr(src, None, "src"),
                                          _dev(q, torch.int8, "q"), _dev(out, torch.int32, "out"),
                                          _stream(stream)), "coli_moe_debug_block_dots")


def coli_moe_debug_logits(dims, x, router_w, logits, stream=None):
    import torch
    _check(_lib.coli_moe_debug_logits(_dims(dims), x.shape[0], _dev(x, torch.float32, "x"),
                                      _dev(router_w, torch.float32, "router_w"),
                                      _dev(logits, torch.float32, "logits"), _stream(stream)),
           "coli_moe_debug_logits")


def coli_moe_debug_expf(x, y, stream=None):
    import torch
    _check(_lib.coli_moe_debug_expf(x.numel(), _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"),
                                    _stream(stream)), "coli_moe_debug_expf")


def coli_moe_debug_q8_0(v, q, d, stream=None):
    import torch
    rows, cols = v.shape
    _check(_lib.coli_moe_debug_q8_0(rows, cols, _dev(v, torch.float32, "v"), _dev(q, torch.int8, "q"),
                                    _dev(d, torch.float32, "d"), _stream(stream)), "coli_moe_debug_q8_0")


def coli_moe_debug_force_path(path: int) -> None:
    _check(_lib.coli_moe_debug_force_path(int(path)), "coli_moe_debug_force_path")


def coli_moe_debug_route_wait(spins: int, unreachable: int) -> None:
    _check(_lib.coli_moe_debug_route_wait(int(spins), int(unreachable)), "coli_moe_debug_route_wait")


def coli_moe_debug_mfma_i8(a, b, c, stream=None):
    """a, b: device int8 [64, 16] raw lane registers; c: device int32 [64, 16]."""
    import torch
    if a.numel() != 1024 or b.numel() != 1024 or c.numel() != 1024:
        raise ValueError("a, b and c hold 64 lanes x 16 registers")
    _check(_lib.coli_moe_debug_mfma_i8(_dev(a, torch.int8, "a"), _dev(b, torch.int8, "b"),
                                       _dev(c, torch.int32, "c"), _stream(stream)), "coli_moe_debug_mfma_i8")


def coli_moe_debug_mfma_i8_16(a, b, c, stream=None):
    """a, b: device int8 [64, 8] raw lane registers; c: device int32 [64, 4]."""
    import torch
    if a.numel() != 512 or b.numel() != 512 or c.numel() != 256:
        raise ValueError("a, b hold 64 lanes x 8 bytes and c 64 lanes x 4 words")
    _check(_lib.coli_moe_debug_mfma_i8_16(_dev(a, torch.int8, "a"), _dev(b, torch.int8, "b"),
                                          _dev(c, torch.int32, "c"), _stream(stream)), "coli_moe_debug_mfma_i8_16")


def coli_moe_debug_mfma_f8f6f4(fmt_a: int, fmt_b: int, a, b, sa, sb, c, stream=None):
    """a, b: device uint8 [64, 32] raw lane registers; sa, sb: device uint8
    [64] E8M0 scales; c: device float32 [64, 16]."""
    import torch
    if a.numel() != 2048 or b.numel() != 2048 or sa.numel() != 64 or sb.numel() != 64 or c.numel() != 1024:
        raise ValueError("a, b: 64 lanes x 32 bytes; sa, sb: 64 bytes; c: 64 lanes x 16 floats")
    _check(_lib.coli_moe_debug_mfma_f8f6f4(int(fmt_a), int(fmt_b), _dev(a, torch.uint8, "a"), _dev(b, torch.uint8, "b"),
                                           _dev(sa, torch.uint8, "sa"), _dev(sb, torch.uint8, "sb"),
                                           _dev(c, torch.float32, "c"), _stream(stream)),
           "coli_moe_debug_mfma_f8f6f4")


def coli_moe_roof_sink_words() -> int:
    return int(_lib.coli_moe_roof_sink_words())


def coli_moe_roof_stream_read(src, sink, stream=None):
    """Streaming read of the whole device tensor `src` (bytes a multiple of 16)."""
    import torch
    nbytes = src.numel() * src.element_size()
    _check(_lib.coli_moe_roof_stream_read(_ptr(src, None, "src"), nbytes, _dev(sink, torch.int32, "sink"),
                                          _stream(stream)), "coli_moe_roof_stream_read")


def coli_moe_roof_mfma_i8(iters: int, sink, stream=None):
    import torch
    _check(_lib.coli_moe_roof_mfma_i8(int(iters), _dev(sink, torch.int32, "sink"), _stream(stream)),
           "coli_moe_roof_mfma_i8")
