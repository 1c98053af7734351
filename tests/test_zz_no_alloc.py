"""coli_moe_layer_noalloc: the layer on the library's own scratch array, for
callers that cannot allocate.  Its outputs must be the bits coli_moe_layer
gives with a caller workspace, on two calls in a row (the second with fewer
tokens, so stale scratch contents of the first call are present), for the
decode kernels and the grouped ones; the device status arrives in the
caller's word; too many tokens are refused before anything is launched."""
import dataclasses

import numpy as np
import pytest

import synth
from tests.gpu_util import q, say, status, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "no GPU visible"
    return t


def _calls(torch, spec, d, dl, S):
    qm = q()
    dims = qm.make_dims(spec)
    x = dl["x"][:S].contiguous()
    ws = workspace(dims, S)
    ref = [torch.full((S, spec.top_k), -7, dtype=torch.int32, device="cuda"),
           torch.full((S, spec.top_k), float("nan"), dtype=torch.float32, device="cuda"),
           torch.full((S, spec.hidden), float("nan"), dtype=torch.float32, device="cuda")]
    qm.coli_moe_layer(dims, x, dl["router_w"], dl["bias"], dl["table"], dl["shared"], *ref, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()
    got = [torch.full_like(t, -7 if t.dtype == torch.int32 else float("nan")) for t in ref]
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    qm.coli_moe_layer_noalloc(dims, x, dl["router_w"], dl["bias"], dl["table"], dl["shared"], *got,
                              status_out=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for a, b in zip(ref, got):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("first,second", [(12, 3), (40, 9), (5, 1)])
def test_noalloc_matches_layer_twice(torch, first, second):
    from synth.device import upload_layer
    spec = synth.TINY
    say(f"no-alloc layer: {first} then {second} tokens")
    d = synth.tiny_layer(seed=61, S=first, spec=spec)
    dl = upload_layer(d)
    _calls(torch, spec, d, dl, first)
    _calls(torch, spec, d, dl, second)


def test_noalloc_glm_decode(torch):
    """GLM-5.2 shape, 4 tokens then 1 (the experts they route to resident)."""
    from synth.device import blob_table
    spec = synth.GLM
    S = 4
    say("no-alloc layer: GLM-5.2 shape, 4 then 1 tokens")
    d = synth.layer_inputs(3, 0, spec, S)
    qm = q()
    dims = qm.make_dims(spec)
    dl = {"x": torch.from_numpy(d["x"]).cuda(), "router_w": torch.from_numpy(d["router_w"]).cuda(),
          "bias": torch.from_numpy(d["bias"]).cuda()}
    ws = workspace(dims, S)
    idx = torch.empty((S, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((S, spec.top_k), dtype=torch.float32, device="cuda")
    qm.coli_moe_route(dims, dl["x"], dl["router_w"], dl["bias"], idx, w, ws)
    assert status(ws) == 0
    used = sorted(set(idx.cpu().numpy().ravel().tolist()))
    blobs = [torch.from_numpy(synth.expert_blob(3, 0, e, spec)).cuda() if e in used else None
             for e in range(spec.n_experts)]
    dl["table"] = blob_table(blobs, spec.n_experts)
    dl["shared"] = torch.from_numpy(synth.expert_blob(3, 0, spec.n_experts, spec)).cuda()
    _calls(torch, spec, d, dl, 4)
    _calls(torch, spec, d, dl, 1)


def test_noalloc_reports_device_status(torch):
    """A NaN in the hidden states reaches status_out (bit 0); the next clean
    call reads 0."""
    from synth.device import upload_layer
    spec = synth.TINY
    say("no-alloc layer: status word")
    d = synth.tiny_layer(seed=62, S=3, spec=spec)
    dl = upload_layer(d)
    qm = q()
    dims = qm.make_dims(spec)
    x = dl["x"].clone()
    x[1, 5] = float("nan")
    idx = torch.empty((3, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((3, spec.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((3, spec.hidden), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    qm.coli_moe_layer_noalloc(dims, x, dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out,
                              status_out=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 1
    qm.coli_moe_layer_noalloc(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out,
                              status_out=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0


def test_noalloc_refuses_too_many_tokens(torch):
    spec = synth.GLM
    qm = q()
    dims = qm.make_dims(spec)
    S = 133
    assert qm.coli_moe_workspace_bytes(dims, S) > 32 << 20
    x = torch.zeros((S, spec.hidden), dtype=torch.float32, device="cuda")
    W = torch.zeros((spec.n_experts, spec.hidden), dtype=torch.float32, device="cuda")
    table = torch.zeros(spec.n_experts, dtype=torch.int64, device="cuda")
    sh = torch.zeros(spec.blob_bytes, dtype=torch.uint8, device="cuda")
    idx = torch.empty((S, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((S, spec.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((S, spec.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(qm.ColiError) as e:
        qm.coli_moe_layer_noalloc(dims, x, W, None, table, sh, idx, w, out)
    assert e.value.code == qm.COLI_EWORKSPACE
    assert "scratch" in qm.coli_moe_last_error()
