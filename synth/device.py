"""Moves synthetic inputs into device memory (torch tensors).

Plumbing only: byte-exact copies of the arrays the generators in this package
produce, plus the device table of expert-blob addresses the forward call
takes.  No arithmetic of the layer happens here.
"""
from __future__ import annotations

import numpy as np
import torch


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def blob_table(blobs, n_experts: int, device="cuda") -> torch.Tensor:
    """int64 device tensor [E] of blob addresses; None/absent -> 0 (not resident)."""
    addrs = [0] * n_experts
    for e, b in enumerate(blobs):
        if b is not None:
            addrs[e] = b.data_ptr()
    return torch.tensor(addrs, dtype=torch.int64, device=device)


def upload_layer(d: dict, device="cuda", experts=None) -> dict:
    """Device copies of a layer dict from synth.tiny_layer-like builders.

    experts: optional iterable of expert ids to upload; the others stay
    non-resident (address 0)."""
    spec = d["spec"]
    keep = set(range(spec.n_experts)) if experts is None else set(int(e) for e in experts)
    blobs = [to_device(b, device) if (e in keep and b is not None) else None for e, b in enumerate(d["blobs"])]
    out = {
        "spec": spec,
        "x": to_device(d["x"], device),
        "router_w": to_device(d["router_w"], device),
        "bias": None if d.get("bias") is None else to_device(d["bias"], device),
        "blobs": blobs,
        "table": blob_table(blobs, spec.n_experts, device),
        "shared": None if d.get("shared") is None else to_device(d["shared"], device),
    }
    return out
