"""GPU parity of group-scaled int4 weights (one f32 scale per 64 codes of a
row; JustVugg/colibri, "Get started" and "Other supported models") through
the C ABI against the CPU oracle: the router launch's shared-expert tiles
(up to two tokens), gate/up, down + combine by output rows, the down and
combine kernels of larger batches, and the error contract of the kernel
families that take per-row scales only."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import gpu_forward, gpu_route, parity, q, say, status, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "no GPU visible"
    return t


def _layer_call(torch, dims, dl, ws):
    S = dl["x"].shape[0]
    idx = torch.full((S, dims.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((S, dims.top_k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, dims.hidden), float("nan"), dtype=torch.float32, device="cuda")
    q().coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out, ws)
    return idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("S", [1, 2, 3, 8, 13])
def test_tiny_gs_layer_entry(torch, S, group):
    """coli_moe_layer on group-scaled tiny layers: up to two tokens the
    shared expert's tiles run in the router launch; up to 8 tokens down and
    combine run by output rows; above, route + forward with the down and
    combine kernels."""
    from synth.device import upload_layer
    spec = dataclasses.replace(synth.TINY_GS64, group=group)
    say(f"gs layer tiny S={S} group={group}")
    d = synth.tiny_layer(seed=5, S=S, spec=spec)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    idx, w, out = _layer_call(torch, dims, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)


@pytest.mark.parametrize("S", [1, 4, 40])
def test_tiny_gs64_forward_entry(torch, S):
    """coli_moe_route + coli_moe_forward (the gate/up launch runs the shared
    expert too; above 8 tokens the per-unit down kernel and the combine)."""
    from synth.device import upload_layer
    spec = synth.TINY_GS64
    say(f"gs64 forward tiny S={S}")
    d = synth.tiny_layer(seed=6, S=S, spec=spec)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    idx, w = gpu_route(dims, dl, ws)
    out = gpu_forward(dims, dl, idx, w, ws).cpu().numpy()
    assert status(ws) == 0, q().coli_moe_last_error()
    o_out, o_idx, _ = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    parity(out, o_out)


@pytest.mark.parametrize("S", [1, 4])
def test_glm_gs64_layer_entry(torch, S):
    """The GLM-5.2 shape with gs64 experts (21.2 MB each), the experts the
    oracle routes to resident, every output element against the oracle."""
    from synth.device import blob_table
    spec = synth.GLM_GS64
    say(f"gs64 glm layer S={S}")
    d = synth.layer_inputs(0, 0, spec, S)
    o_idx, o_w, _, _ = oracle.route(spec, d["x"], d["router_w"], d["bias"])
    used = sorted(set(o_idx.ravel().tolist()))
    host = {e: synth.expert_blob(0, 0, e, spec) for e in used}
    shared = synth.expert_blob(0, 0, spec.n_experts, spec)
    assert shared.size == 21_233_664
    blobs = [torch.from_numpy(host[e]).cuda() if e in host else None for e in range(spec.n_experts)]
    dl = {"x": torch.from_numpy(d["x"]).cuda(), "router_w": torch.from_numpy(d["router_w"]).cuda(),
          "bias": torch.from_numpy(d["bias"]).cuda(), "table": blob_table(blobs, spec.n_experts),
          "shared": torch.from_numpy(shared).cuda()}
    dims = q().make_dims(spec)
    assert q().coli_moe_expert_bytes(dims) == 21_233_664
    ws = workspace(dims, S)
    idx, w, out = _layer_call(torch, dims, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    assert np.array_equal(idx, o_idx)
    want = oracle.forward(spec, d["x"], o_idx, o_w, [host.get(e) for e in range(spec.n_experts)], shared)
    say("gs64 glm parity", parity(out, want))


def test_gs_error_contract(torch):
    """Group scales need int4 and a power-of-two group dividing H and I; the
    persistent and grouped kernel families refuse them when forced."""
    from synth.device import upload_layer
    qm = q()
    for bad in (dataclasses.replace(synth.TINY_GS64, wbits=8), dataclasses.replace(synth.TINY_GS64, group=48),
                dataclasses.replace(synth.TINY_GS64, group=256)):   # 256 does not divide inter 128
        assert qm.coli_moe_expert_bytes(qm.make_dims(bad)) == 0
    spec = synth.TINY_GS64
    d = synth.tiny_layer(seed=7, S=3, spec=spec)
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, 3)
    for path in (qm.PATH_PERSISTENT, qm.PATH_GROUPED):
        qm.coli_moe_debug_force_path(path)
        try:
            with pytest.raises(qm.ColiError) as err:
                _layer_call(torch, dims, dl, ws)
            assert err.value.code == qm.COLI_EINVAL
        finally:
            qm.coli_moe_debug_force_path(qm.PATH_AUTO)
    assert status(ws) == 0
