"""GPU parity at the extremes of the code formats: blobs whose codes include
the minimum of each width (int8 -128, int4 -8, int2 -2) at every position
of a 32-code block, whole rows of it, and alternations with the maximum,
against Q8_0 activations that are all +-127 (so block sums reach their
largest magnitudes), through every kernel family: the decode kernels, the
persistent kernel, the grouped matrix-core kernels (forced at small batches
and chosen automatically from 9 tokens), with per-row scales and with
groups of 64.  Gate and up rows 32..63 are all at the minimum with one
scale, so h is constant over that block and Q8_0(h) is +-127 there too,
which takes the down projection to the same extremes.  Routing must be
bit-exact and outputs bitwise equal to the oracle's."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import parity, q, say, status, workspace

pytestmark = pytest.mark.gpu

SPECS = {
    "int8": dataclasses.replace(synth.TINY, wbits=8),
    "int4": synth.TINY,
    "int2": dataclasses.replace(synth.TINY, wbits=2),
    "gs64": synth.TINY_GS64,
    "int4-h512-i256": dataclasses.replace(synth.TINY, hidden=512, inter=256, n_experts=12, top_k=3),
}

# (kernel family forced, entry point, tokens)
CASES = [
    ("multi", "split", 1), ("multi", "split", 3), ("multi", "layer", 1), ("multi", "layer", 2),
    ("multi", "split", 12), ("persistent", "layer", 2), ("grouped", "split", 4), ("grouped", "layer", 5),
    ("auto", "layer", 12), ("auto", "split", 40),
]


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "no GPU visible"
    return t


def _force(path):
    qm = q()
    qm.coli_moe_debug_force_path({"auto": qm.PATH_AUTO, "multi": qm.PATH_MULTI,
                                  "persistent": qm.PATH_PERSISTENT, "grouped": qm.PATH_GROUPED}[path])


@pytest.mark.parametrize("name", list(SPECS))
@pytest.mark.parametrize("path,entry,S", CASES, ids=[f"{p}-{e}-S{s}" for p, e, s in CASES])
def test_extreme_codes(torch, name, path, entry, S):
    from synth.device import upload_layer
    spec = SPECS[name]
    if path == "persistent" and spec.group:
        pytest.skip("the persistent kernel takes per-row scales only")
    say(f"extreme codes {name} [{path}, {entry}, S={S}]")
    d = synth.extreme_layer(seed=400 + S, S=S, spec=spec)
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    qm = q()
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    idx = torch.full((S, spec.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((S, spec.top_k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, spec.hidden), float("nan"), dtype=torch.float32, device="cuda")
    _force(path)
    try:
        if entry == "layer":
            qm.coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out, ws)
        else:
            qm.coli_moe_route(dims, dl["x"], dl["router_w"], dl["bias"], idx, w, ws)
            qm.coli_moe_forward(dims, dl["x"], idx, w, dl["table"], dl["shared"], out, ws)
        rc = status(ws)
    finally:
        _force("auto")
    assert rc == 0, qm.coli_moe_last_error()
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))
    parity(out.cpu().numpy(), o_out)
