"""GPU parity of MXFP4 routed experts (E2M1 codes, one E8M0 scale per 32
codes of a row; JustVugg/colibri "Other supported models": experts streamed
in their checkpoints' native MXFP4) through the C ABI against the CPU
oracle: the device decode of every code at every position and its exact
block sums (the debug hooks), the layer through coli_moe_layer and through
coli_moe_route + coli_moe_forward at several batch sizes (the router
launch's shared-expert tiles, gate/up, down + combine by rows, the per-unit
down and the combine), edge-case codes and subnormal scales, and the
GLM-5.2 shape.  Routing bit-exact, outputs bitwise equal to the oracle's."""
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


def test_mx_decode_every_code_every_position(torch):
    say("mx hooks: unpack and block dots")
    qm = q()
    rows, cols = 48, 512
    codes = ((np.arange(cols)[None, :] * 7 + np.arange(rows)[:, None] * 3) % 16).astype(np.uint8)
    rng = np.random.default_rng(4)
    codes[24:] = rng.integers(0, 16, size=(rows - 24, cols)).astype(np.uint8)
    packed = synth.pack_mx(codes)
    src = torch.from_numpy(np.ascontiguousarray(packed)).cuda()
    out = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    qm.coli_moe_debug_unpack(qm.COLI_MXFP4, rows, cols, src, out)
    want = np.stack([oracle.unpack_mx(packed[r], cols) for r in range(rows)])
    assert np.array_equal(out.cpu().numpy(), want)
    for qv in (rng.integers(-127, 128, cols), np.full(cols, 127), np.full(cols, -127), np.full(cols, -128)):
        qv = qv.astype(np.int8)
        dots = torch.empty((rows, cols // 32), dtype=torch.int32, device="cuda")
        qm.coli_moe_debug_block_dots(qm.COLI_MXFP4, rows, cols, src, torch.from_numpy(qv).cuda(), dots)
        ref = (want.astype(np.int64) * qv.astype(np.int64)[None, :]).reshape(rows, cols // 32, 32).sum(-1)
        assert np.array_equal(dots.cpu().numpy(), ref)


def _layer_call(torch, dims, dl, S):
    ws = workspace(dims, S)
    idx = torch.full((S, dims.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((S, dims.top_k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, dims.hidden), float("nan"), dtype=torch.float32, device="cuda")
    q().coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out, ws)
    return ws, idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy()


SPECS = {
    "tiny": synth.TINY_MX,
    "h512-i256-e24-k4": dataclasses.replace(synth.TINY_MX, hidden=512, inter=256, n_experts=24, top_k=4),
    "noshared-nonorm": dataclasses.replace(synth.TINY_MX, n_shared=0, norm_topk_prob=0, routed_scaling_factor=1.5),
}


@pytest.mark.parametrize("name", list(SPECS))
@pytest.mark.parametrize("S", [1, 2, 3, 8, 12, 40])
def test_mx_layer(torch, name, S):
    from synth.device import upload_layer
    spec = SPECS[name]
    say(f"mx layer {name} S={S}")
    d = synth.tiny_layer(seed=70 + S, S=S, spec=spec)
    dims = q().make_dims(spec)
    assert q().coli_moe_expert_bytes(dims) == spec.blob_bytes
    dl = upload_layer(d)
    ws, idx, w, out = _layer_call(torch, dims, dl, S)
    assert status(ws) == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)
    ws2 = workspace(dims, S)
    idx2, w2 = gpu_route(dims, dl, ws2)
    out2 = gpu_forward(dims, dl, idx2, w2, ws2).cpu().numpy()
    assert status(ws2) == 0, q().coli_moe_last_error()
    parity(out2, o_out)


@pytest.mark.parametrize("S", [1, 2, 5, 12, 40])
def test_mx_extreme_codes_and_subnormal_scales(torch, S):
    from synth.device import upload_layer
    spec = synth.TINY_MX
    say(f"mx extreme codes S={S}")
    d = synth.extreme_mx_layer(seed=90 + S, S=S, spec=spec)
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws, idx, w, out = _layer_call(torch, dims, dl, S)
    assert status(ws) == 0, q().coli_moe_last_error()
    assert np.array_equal(idx, o_idx)
    parity(out, o_out)


def test_mx_pending_experts(torch):
    """A pending mask with MXFP4 experts: resident ones first, pending ones
    after the event; the same bits as the unmasked call."""
    from synth.device import upload_layer
    spec = synth.TINY_MX
    say("mx pending mask")
    d = synth.tiny_layer(seed=77, S=3, spec=spec)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, 3)
    idx, w = gpu_route(dims, dl, ws)
    ref = gpu_forward(dims, dl, idx, w, ws).cpu().numpy()
    mask = np.zeros(spec.n_experts, np.uint8)
    mask[idx[0].cpu().numpy()] = 1
    ev = torch.cuda.Event()
    ev.record()
    out = gpu_forward(dims, dl, idx, w, ws, pending_mask=mask, pending_ready=ev).cpu().numpy()
    assert status(ws) == 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_mx_refusals(torch):
    """Shapes and kernel families the MXFP4 experts do not take are refused
    on the host."""
    qm = q()
    spec = synth.TINY_MX
    bad = qm.make_dims(dataclasses.replace(spec, inter=96))
    assert qm.coli_moe_expert_bytes(bad) == 0 and "MXFP4" in qm.coli_moe_last_error()
    bad = qm.make_dims(dataclasses.replace(spec, wbits=8))
    assert qm.coli_moe_expert_bytes(bad) == 0
    from synth.device import upload_layer
    d = synth.tiny_layer(seed=78, S=2, spec=spec)
    dl = upload_layer(d)
    dims = qm.make_dims(spec)
    qm.coli_moe_debug_force_path(qm.PATH_PERSISTENT)
    try:
        with pytest.raises(qm.ColiError) as e:
            _layer_call(torch, dims, dl, 2)
        assert e.value.code == qm.COLI_EINVAL
    finally:
        qm.coli_moe_debug_force_path(qm.PATH_AUTO)


@pytest.mark.parametrize("S", [1, 3, 8])
@pytest.mark.parametrize("extreme", [False, True])
def test_mx_forced_grouped(torch, S, extreme):
    """The MXFP4 grouped kernels (FP4 matrix cores) forced at small batch
    sizes: tiles of one to a few pairs, with ordinary scales (the scaled
    products) and with extreme codes and E8M0 bytes 0, 1 and 2 (the tiles
    recomputed with unscaled products); bitwise equal to the oracle."""
    from synth.device import upload_layer
    qm = q()
    spec = synth.TINY_MX
    say(f"mx forced grouped S={S} extreme={extreme}")
    d = (synth.extreme_mx_layer(seed=95 + S, S=S, spec=spec) if extreme
         else synth.tiny_layer(seed=85 + S, S=S, spec=spec))
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    qm.coli_moe_debug_force_path(qm.PATH_GROUPED)
    try:
        ws, idx, w, out = _layer_call(torch, dims, dl, S)
    finally:
        qm.coli_moe_debug_force_path(qm.PATH_AUTO)
    assert status(ws) == 0, qm.coli_moe_last_error()
    assert np.array_equal(idx, o_idx)
    parity(out, o_out)


@pytest.mark.parametrize("S", [1, 4])
def test_glm_mx_layer(torch, S):
    """The GLM-5.2 shape with MXFP4 experts (20.05 MB each), the experts the
    oracle routes to resident, every output element against the oracle."""
    from synth.device import blob_table
    spec = synth.GLM_MX
    say(f"mx glm layer S={S}")
    d = synth.layer_inputs(0, 0, spec, S)
    o_idx, o_w, _, _ = oracle.route(spec, d["x"], d["router_w"], d["bias"])
    used = sorted(set(o_idx.ravel().tolist()))
    host = {e: synth.expert_blob(0, 0, e, spec) for e in used}
    shared = synth.expert_blob(0, 0, spec.n_experts, spec)
    assert shared.size == 20_054_016
    blobs = [torch.from_numpy(host[e]).cuda() if e in host else None for e in range(spec.n_experts)]
    dl = {"x": torch.from_numpy(d["x"]).cuda(), "router_w": torch.from_numpy(d["router_w"]).cuda(),
          "bias": torch.from_numpy(d["bias"]).cuda(), "table": blob_table(blobs, spec.n_experts),
          "shared": torch.from_numpy(shared).cuda()}
    dims = q().make_dims(spec)
    assert q().coli_moe_expert_bytes(dims) == 20_054_016
    ws, idx, w, out = _layer_call(torch, dims, dl, S)
    assert status(ws) == 0, q().coli_moe_last_error()
    assert np.array_equal(idx, o_idx)
    want = oracle.forward(spec, d["x"], o_idx, o_w, [host.get(e) for e in range(spec.n_experts)], shared,
                          parallel=True)
    say("mx glm parity", parity(out, want))
