"""GPU parity of group-scaled int4 weights (one f32 scale per 64 codes of a
row; JustVugg/colibri, "Get started" and "Other supported models") through
the C ABI against the CPU oracle: the router launch's shared-expert tiles
(up to two tokens), gate/up, down + combine by output rows, the down and
combine kernels, the grouped matrix-core kernels of large batches (with the
exact fallback for tiny group scales), and the error contract."""
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


@pytest.mark.parametrize("group,H,I", [(256, 256, 256), (256, 512, 256), (512, 512, 512), (512, 1024, 512)],
                         ids=["g256-h256", "g256-h512", "g512-h512", "g512-h1024"])
@pytest.mark.parametrize("S", [1, 3, 12])
def test_large_groups(torch, S, group, H, I):
    """Groups of 256 and 512 codes (one or two scales per gate/up row, and
    fewer scales per row than a 64-block chunk holds) through
    coli_moe_layer and coli_moe_route + coli_moe_forward; these group sizes
    run the decode kernels at every batch size."""
    from synth.device import upload_layer
    spec = dataclasses.replace(synth.TINY_GS64, group=group, hidden=H, inter=I)
    say(f"gs large groups S={S} group={group} H={H} I={I}")
    d = synth.tiny_layer(seed=15, S=S, spec=spec)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    idx, w, out = _layer_call(torch, dims, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)
    idx2, w2 = gpu_route(dims, dl, ws)
    out2 = gpu_forward(dims, dl, idx2, w2, ws).cpu().numpy()
    assert status(ws) == 0, q().coli_moe_last_error()
    parity(out2, o_out)


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


MID_GS64 = synth.LayerSpec(hidden=512, inter=256, n_experts=64, top_k=8, n_shared=1, wbits=4, group=64)


def _zipf_layer(spec, S, seed=0):
    d = synth.layer_inputs(seed, 0, spec, S)
    d["x"] = synth.prefill_hidden_states(seed, 0, spec, S)
    d["bias"] = np.zeros(spec.n_experts, np.float32)
    d["blobs"] = [synth.expert_blob(seed, 0, e, spec) for e in range(spec.n_experts)]
    d["shared"] = synth.expert_blob(seed, 0, spec.n_experts, spec)
    return d


@pytest.mark.parametrize("S", [160])
def test_mid_gs64_grouped_prefill(torch, S):
    """Batches of 9 or more tokens take the int8 matrix-core kernels with the
    group scales staged per stage: a Zipf-routed mid-size layer, every output
    element against the oracle."""
    from synth.device import upload_layer
    spec = MID_GS64
    say(f"gs64 grouped mid layer S={S}")
    d = _zipf_layer(spec, S, seed=3)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    idx, w, out = _layer_call(torch, dims, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx, o_idx)
    assert int(np.bincount(idx.ravel()).max()) > 64   # one expert spans three tiles
    say("parity", parity(out, o_out))


@pytest.mark.parametrize("S", [3, 40])
def test_tiny_gs64_forced_grouped(torch, S):
    """The grouped kernels forced at small and ragged batches (tiles of one
    to a few pairs), against the oracle."""
    from synth.device import upload_layer
    qm = q()
    spec = synth.TINY_GS64
    say(f"gs64 forced grouped tiny S={S}")
    d = synth.tiny_layer(seed=8, S=S, spec=spec)
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    qm.coli_moe_debug_force_path(qm.PATH_GROUPED)
    try:
        idx, w, out = _layer_call(torch, dims, dl, ws)
    finally:
        qm.coli_moe_debug_force_path(qm.PATH_AUTO)
    assert status(ws) == 0, qm.coli_moe_last_error()
    o_out, o_idx, _ = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx, o_idx)
    parity(out, o_out)


def test_gs64_grouped_tiny_group_scales_take_the_exact_path(torch):
    """Group scales below 2^-60 would make the folded chain inexact: the
    grouped kernels then recompute the tile with the shifting chain, and the
    result still equals the oracle's."""
    from synth.device import upload_layer
    qm = q()
    spec = synth.TINY_GS64
    S = 20
    say(f"gs64 grouped tiny group scales S={S}")
    d = synth.tiny_layer(seed=10, S=S, spec=spec)
    lay = oracle.blob_layout(spec.hidden, spec.inter, spec.wbits, spec.group)
    blobs = []
    for b in d["blobs"] + [d["shared"]]:
        b = b.copy()
        for sec in ("s_gate", "s_down"):
            sc = b[lay[sec]:lay[sec] + 64].view(np.float32)   # the first 16 scales of the section
            sc[:8] = sc[:8] * np.float32(2.0 ** -70)
        blobs.append(b)
    d["blobs"], d["shared"] = blobs[:-1], blobs[-1]
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    qm.coli_moe_debug_force_path(qm.PATH_GROUPED)
    try:
        idx, w, out = _layer_call(torch, dims, dl, ws)
    finally:
        qm.coli_moe_debug_force_path(qm.PATH_AUTO)
    assert status(ws) == 0, qm.coli_moe_last_error()
    o_out, o_idx, _ = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx, o_idx)
    parity(out, o_out)


def test_gs_error_contract(torch):
    """Group scales need int4 and a power-of-two group dividing H and I; the
    persistent kernel refuses them when forced, the grouped kernels every
    group size but 64."""
    from synth.device import upload_layer
    qm = q()
    for bad in (dataclasses.replace(synth.TINY_GS64, wbits=8), dataclasses.replace(synth.TINY_GS64, group=48),
                dataclasses.replace(synth.TINY_GS64, group=256)):   # 256 does not divide inter 128
        assert qm.coli_moe_expert_bytes(qm.make_dims(bad)) == 0
    for spec, path in ((synth.TINY_GS64, qm.PATH_PERSISTENT),
                       (dataclasses.replace(synth.TINY_GS64, group=32), qm.PATH_GROUPED)):
        d = synth.tiny_layer(seed=7, S=3, spec=spec)
        dims = qm.make_dims(spec)
        dl = upload_layer(d)
        ws = workspace(dims, 3)
        qm.coli_moe_debug_force_path(path)
        try:
            with pytest.raises(qm.ColiError) as err:
                _layer_call(torch, dims, dl, ws)
            assert err.value.code == qm.COLI_EINVAL
        finally:
            qm.coli_moe_debug_force_path(qm.PATH_AUTO)
        assert status(ws) == 0
