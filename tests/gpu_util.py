"""Helpers shared by the GPU parity tests (imported lazily by test modules)."""
from __future__ import annotations

import sys

import numpy as np

REL_L2 = 1e-5          # tolerance on binary32 layer outputs (relative L2 error)
MAX_ABS_RMS = 1e-3     # and on the max abs error, relative to the output RMS


def say(*a):
    """Names the case being run, flushed before each GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


def q():
    import quantized_expert_ffn_amd as qm
    return qm


def parity(got: np.ndarray, want: np.ndarray, bitwise: bool = True) -> dict:
    """Asserts the layer tolerance; with bitwise, also exact equality."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape
    assert np.all(np.isfinite(got))
    diff = got.astype(np.float64) - want.astype(np.float64)
    nrm = np.linalg.norm(want.astype(np.float64))
    rel = float(np.linalg.norm(diff) / nrm) if nrm > 0 else float(np.linalg.norm(diff))
    rms = float(np.sqrt(np.mean(want.astype(np.float64) ** 2))) if want.size else 0.0
    mx = float(np.max(np.abs(diff))) if want.size else 0.0
    assert rel <= REL_L2, f"rel-L2 {rel:.3e}"
    assert mx <= MAX_ABS_RMS * rms + 1e-30, f"max-abs {mx:.3e} vs rms {rms:.3e}"
    n_diff = int(np.sum(got.view(np.uint32) != want.view(np.uint32)))
    if bitwise:
        assert n_diff == 0, f"{n_diff} of {got.size} elements differ in bits (rel-L2 {rel:.3e})"
    return {"rel_l2": rel, "max_abs": mx, "rms": rms, "bit_diffs": n_diff}


def workspace(dims, max_tokens):
    import torch
    n = q().coli_moe_workspace_bytes(dims, max_tokens)
    assert n > 0
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def gpu_route(dims, dl, ws, S=None):
    import torch
    S = dl["x"].shape[0] if S is None else S
    idx = torch.empty((S, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((S, dims.top_k), dtype=torch.float32, device="cuda")
    q().coli_moe_route(dims, dl["x"], dl["router_w"], dl["bias"], idx, w, ws)
    return idx, w


def gpu_forward(dims, dl, idx, w, ws, pending_mask=None, pending_ready=None):
    import torch
    out = torch.full((dl["x"].shape[0], dims.hidden), float("nan"), dtype=torch.float32, device="cuda")
    q().coli_moe_forward(dims, dl["x"], idx, w, dl["table"], dl["shared"], out, ws,
                         pending_mask=pending_mask, pending_ready=pending_ready)
    return out


def status(ws) -> int:
    return q().coli_moe_status(ws)
