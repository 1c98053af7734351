"""GPU parity of the whole layer through the C ABI (coli_moe_route,
coli_moe_forward, coli_moe_stage_experts) against the CPU oracle on the same
seeded inputs: bit-exact routing, binary32 outputs within rel-L2 1e-5 and
max-abs 1e-3 x RMS (and, by the layer's fixed operation order, bit-exact)."""
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


@pytest.fixture(params=["multi", "persistent", "grouped"])
def path(request, torch):
    """Runs a test with the multi-launch decode kernels, the persistent ones
    or the grouped matrix-core kernels (each forced at every batch size the
    family takes)."""
    qm = q()
    qm.coli_moe_debug_force_path({"multi": qm.PATH_MULTI, "persistent": qm.PATH_PERSISTENT,
                                  "grouped": qm.PATH_GROUPED}[request.param])
    yield request.param
    qm.coli_moe_debug_force_path(qm.PATH_AUTO)


def _layer(spec, S, seed=0):
    d = synth.tiny_layer(seed=seed, S=S, spec=spec)
    return d


def _run(torch, spec, d, S=None, dev=None):
    from synth.device import upload_layer
    dims = q().make_dims(spec)
    dl = upload_layer(d) if dev is None else dev
    S = d["x"].shape[0] if S is None else S
    ws = workspace(dims, S)
    idx, w = gpu_route(dims, dl, ws)
    out = gpu_forward(dims, dl, idx, w, ws)
    rc = status(ws)
    return dims, dl, ws, idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy(), rc


def _oracle(spec, d):
    out, idx, w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    return out, idx, w


def test_tiny_layer_bitexact(torch, path):
    say(f"tiny layer S=4 int4 [{path}]")
    spec = synth.TINY
    d = _layer(spec, 4)
    _, _, _, idx, w, out, rc = _run(torch, spec, d)
    assert rc == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = _oracle(spec, d)
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8, 9, 17])
def test_tiny_ragged_token_counts(torch, path, S):
    if path == "persistent" and S > 8:
        pytest.skip("the persistent forward takes at most 8 tokens")
    say(f"tiny layer S={S} [{path}]")
    spec = synth.TINY
    d = _layer(spec, S, seed=S)
    _, _, _, idx, w, out, rc = _run(torch, spec, d)
    assert rc == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = _oracle(spec, d)
    assert np.array_equal(idx, o_idx)
    parity(out, o_out)


@pytest.mark.parametrize("spec", [
    dataclasses.replace(synth.TINY, wbits=8),
    dataclasses.replace(synth.TINY, wbits=2),
    dataclasses.replace(synth.TINY, top_k=1, n_shared=0, routed_scaling_factor=1.0),
    dataclasses.replace(synth.TINY, n_experts=40, top_k=6, hidden=512, inter=96),
    dataclasses.replace(synth.TINY, norm_topk_prob=0, routed_scaling_factor=1.5, n_experts=70, top_k=9),
], ids=["int8", "int2", "k1-noshared", "e40-h512-i96", "nonorm-e70-k9"])
def test_tiny_variants(torch, path, spec):
    say(f"tiny variant {spec} [{path}]")
    d = _layer(spec, 5, seed=11)
    _, _, _, idx, w, out, rc = _run(torch, spec, d)
    assert rc == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = _oracle(spec, d)
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)


def test_batch_invariance(torch, path):
    """A token's output bits do not depend on which other tokens share the call."""
    say(f"batch invariance [{path}]")
    from synth.device import upload_layer
    spec = synth.TINY
    d = _layer(spec, 6, seed=21)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, 6)
    idx, w = gpu_route(dims, dl, ws)
    full = gpu_forward(dims, dl, idx, w, ws).cpu().numpy()
    for t in range(6):
        one = dict(dl)
        one["x"] = dl["x"][t:t + 1].contiguous()
        o = gpu_forward(dims, one, idx[t:t + 1].contiguous(), w[t:t + 1].contiguous(), ws).cpu().numpy()
        assert np.array_equal(o[0].view(np.uint32), full[t].view(np.uint32))
    assert status(ws) == 0


def _one_hot_router(torch, logits_rows, K, bias=None):
    """Routes tokens whose logits are given exactly: W_r rows are one-hot and
    x carries the logits (the binary32 logit of a one-hot row is exact)."""
    lg = np.asarray(logits_rows, np.float32)
    S, E = lg.shape
    spec = dataclasses.replace(synth.TINY, n_experts=E, top_k=K, routed_scaling_factor=1.0)
    x = np.zeros((S, spec.hidden), np.float32)
    x[:, :E] = lg
    W = np.zeros((E, spec.hidden), np.float32)
    W[np.arange(E), np.arange(E)] = 1.0
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    dims = q().make_dims(spec)
    dl = {"x": torch.from_numpy(x).cuda(), "router_w": torch.from_numpy(W).cuda(), "bias": torch.from_numpy(b).cuda()}
    ws = workspace(dims, S)
    idx, w = gpu_route(dims, dl, ws)
    return idx.cpu().numpy(), w.cpu().numpy(), status(ws)


def test_router_worked_examples_through_the_abi(torch):
    import json
    import os
    say("router worked examples")
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "router_worked_examples.json")))
    ex = g["tie_break"]
    idx, _, rc = _one_hot_router(torch, [ex["logits"]], ex["top_k"], ex["bias"])
    assert rc == 0
    assert sorted(idx[0].tolist()) == ex["expected_sorted_set"] and idx[0, -1] == ex["expected_last"]
    ex = g["near_tie"]
    lg = np.array(ex["logits"], np.float64)
    nudged = lg.copy()
    nudged[ex["nudge_expert"]] += ex["nudge"]
    idx, _, rc = _one_hot_router(torch, [lg, nudged], ex["top_k"], ex["bias"])
    assert rc == 0
    assert idx[0, -1] == ex["expected_last_before"] and idx[1, -1] == ex["expected_last_after"]
    bad = np.zeros((1, 8), np.float32)
    bad[0, 3] = np.nan
    _, _, rc = _one_hot_router(torch, bad, 5)
    assert rc == q().COLI_ENONFINITE


def test_error_contract(torch, path):
    say(f"error contract [{path}]")
    from synth.device import upload_layer
    qm = q()
    spec = synth.TINY
    d = _layer(spec, 4, seed=5)
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, 4)
    idx, w = gpu_route(dims, dl, ws)
    assert status(ws) == 0
    # non-finite hidden state
    dl2 = dict(dl)
    dl2["x"] = dl["x"].clone()
    dl2["x"][1, 3] = float("nan")
    gpu_forward(dims, dl2, idx, w, ws)
    assert status(ws) == qm.COLI_ENONFINITE
    gpu_route(dims, dl2, ws)
    assert status(ws) == qm.COLI_ENONFINITE
    # routed expert not resident
    table = dl["table"].clone()
    table[int(idx[0, 0])] = 0
    dl3 = dict(dl)
    dl3["table"] = table
    gpu_forward(dims, dl3, idx, w, ws)
    assert status(ws) == qm.COLI_ENOTRESIDENT
    # index out of range, repeated index
    i2 = idx.clone()
    i2[2, 1] = spec.n_experts
    gpu_forward(dims, dl, i2, w, ws)
    assert status(ws) == qm.COLI_EINVAL
    i3 = idx.clone()
    i3[3, 1] = i3[3, 0]
    gpu_forward(dims, dl, i3, w, ws)
    assert status(ws) == qm.COLI_EINVAL
    # status cleared, normal call fine again
    gpu_forward(dims, dl, idx, w, ws)
    assert status(ws) == 0
    # host-side checks
    small = ws[: 1024]
    with pytest.raises(qm.ColiError) as e:
        gpu_forward(dims, dl, idx, w, small)
    assert e.value.code == qm.COLI_EWORKSPACE
    bad = qm.make_dims(spec)
    bad.wbits = 3
    with pytest.raises(qm.ColiError) as e:
        gpu_route(bad, dl, ws)
    assert e.value.code == qm.COLI_EINVAL
    # zero tokens: no-op
    empty = dict(dl)
    empty["x"] = dl["x"][:0]
    o = gpu_forward(dims, empty, idx[:0], w[:0], ws)
    assert o.shape == (0, spec.hidden) and status(ws) == 0


def test_pending_experts_run_after_the_event(torch):
    say("pending mask")
    from synth.device import upload_layer
    spec = synth.TINY
    d = _layer(spec, 4, seed=8)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, 4)
    idx, w = gpu_route(dims, dl, ws)
    ref = gpu_forward(dims, dl, idx, w, ws).cpu().numpy()
    mask = np.zeros(spec.n_experts, np.uint8)
    mask[idx[0].cpu().numpy()] = 1
    ev = torch.cuda.Event()
    ev.record()
    out = gpu_forward(dims, dl, idx, w, ws, pending_mask=mask, pending_ready=ev).cpu().numpy()
    assert status(ws) == 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("S", [1, 2])
def test_nonfinite_router_rows_leave_a_safe_unit_table(torch, S):
    """At least E - K + 1 router rows of NaN: no token has K finite scores,
    so the selection fails and may repeat an expert.  coli_moe_layer (its
    router launch selects and writes the unit table) must report
    COLI_ENONFINITE and leave a table the expert kernels can run; the next,
    valid call on the same workspace is bitwise the oracle's."""
    from synth.device import upload_layer
    say(f"NaN router rows, layer call S={S}")
    spec = synth.TINY
    qm = q()
    d = _layer(spec, S, seed=31)
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    bad = dl["router_w"].clone()
    bad[: spec.n_experts - spec.top_k + 1] = float("nan")
    ws = workspace(dims, S)
    idx = torch.empty((S, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((S, spec.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((S, spec.hidden), dtype=torch.float32, device="cuda")
    qm.coli_moe_layer(dims, dl["x"], bad, dl["bias"], dl["table"], dl["shared"], idx, w, out, ws)
    assert status(ws) == qm.COLI_ENONFINITE
    qm.coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()
    o_out, o_idx, _ = _oracle(spec, d)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    parity(out.cpu().numpy(), o_out)


def test_stage_experts_copies_bytes(torch):
    say("stage experts")
    spec = synth.TINY
    n = 5
    host = [torch.from_numpy(synth.gaussian_expert(2, 0, e, spec)[0]).pin_memory() for e in range(n)]
    dev = [torch.empty(spec.blob_bytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
    s = torch.cuda.Stream()
    ev = torch.cuda.Event()
    q().coli_moe_stage_experts(host, dev, spec.blob_bytes, s, ev)
    ev.synchronize()
    for h, dv in zip(host, dev):
        assert torch.equal(h, dv.cpu())


def _glm_layer_for_tokens(torch, spec, S, seed, x=None, layer=0):
    """GLM-shaped layer with only the experts the tokens route to resident."""
    from synth.device import blob_table
    d = synth.layer_inputs(seed, layer, spec, S)
    if x is not None:
        d["x"] = x
    dims = q().make_dims(spec)
    dl = {"x": torch.from_numpy(d["x"]).cuda(), "router_w": torch.from_numpy(d["router_w"]).cuda(),
          "bias": torch.from_numpy(d["bias"]).cuda()}
    ws = workspace(dims, S)
    idx, w = gpu_route(dims, dl, ws)
    assert status(ws) == 0
    used = sorted(set(idx.cpu().numpy().ravel().tolist()))
    host = {e: synth.expert_blob(seed, layer, e, spec) for e in used}
    shared = synth.expert_blob(seed, layer, spec.n_experts, spec)
    blobs = [torch.from_numpy(host[e]).cuda() if e in host else None for e in range(spec.n_experts)]
    dl["blobs"] = blobs
    dl["table"] = blob_table(blobs, spec.n_experts)
    dl["shared"] = torch.from_numpy(shared).cuda()
    d["blobs"] = [host.get(e) for e in range(spec.n_experts)]
    d["shared"] = shared
    return d, dims, dl, ws, idx, w, used


def test_glm_decode_one_token(torch, path):
    """GLM-5.2-shaped decode layer (H 6144, I 2048, 256 experts top-8 + shared,
    int4, 1 token); the persistent kernels are the launch configuration the
    benchmark times."""
    say(f"glm decode S=1 int4 [{path}]")
    spec = synth.GLM
    d, dims, dl, ws, idx, w, used = _glm_layer_for_tokens(torch, spec, 1, seed=0)
    o_idx, o_w, _, _ = oracle.route(spec, d["x"], d["router_w"], d["bias"])
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))
    out = gpu_forward(dims, dl, idx, w, ws).cpu().numpy()
    assert status(ws) == 0
    want = oracle.forward(spec, d["x"], o_idx, o_w, d["blobs"], d["shared"])
    r = parity(out, want)
    say("glm decode parity", r)


def test_glm_verify_four_tokens_int8(torch, path):
    """Speculative-verify batch: S=4 tokens routed jointly, int8 experts,
    tokens sharing experts (batch-union)."""
    say(f"glm verify S=4 int8 [{path}]")
    spec = synth.GLM_INT8
    x = synth.verify_hidden_states(0, 0, spec, 4)
    d, dims, dl, ws, idx, w, used = _glm_layer_for_tokens(torch, spec, 4, seed=0, x=x)
    say("unique experts", len(used))
    assert len(used) < 32
    o_idx, o_w, _, _ = oracle.route(spec, d["x"], d["router_w"], d["bias"])
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    out = gpu_forward(dims, dl, idx, w, ws).cpu().numpy()
    assert status(ws) == 0
    want = oracle.forward(spec, d["x"], o_idx, o_w, d["blobs"], d["shared"])
    parity(out, want)


def test_paths_agree_bitwise(torch):
    """Multi-launch, persistent and grouped kernels give the same bits (S = 1..8)."""
    from synth.device import upload_layer
    qm = q()
    spec = synth.TINY
    for S in (1, 3, 8):
        say(f"path agreement S={S}")
        d = _layer(spec, S, seed=40 + S)
        dims = qm.make_dims(spec)
        dl = upload_layer(d)
        ws = workspace(dims, S)
        outs = []
        for p in (qm.PATH_MULTI, qm.PATH_PERSISTENT, qm.PATH_GROUPED):
            qm.coli_moe_debug_force_path(p)
            idx, w = gpu_route(dims, dl, ws)
            outs.append((idx.cpu().numpy(), gpu_forward(dims, dl, idx, w, ws).cpu().numpy()))
            assert status(ws) == 0
        qm.coli_moe_debug_force_path(qm.PATH_AUTO)
        for o in outs[1:]:
            assert np.array_equal(outs[0][0], o[0])
            assert np.array_equal(outs[0][1].view(np.uint32), o[1].view(np.uint32))


def gpu_layer(torch, dims, dl, ws):
    S = dl["x"].shape[0]
    idx = torch.full((S, dims.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((S, dims.top_k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, dims.hidden), float("nan"), dtype=torch.float32, device="cuda")
    q().coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out, ws)
    return idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("S", [1, 2, 4, 7, 8, 13])
def test_layer_entry_tiny(torch, path, S):
    """coli_moe_layer (router + experts + combine in one call) against the
    oracle, ragged token counts; above 8 tokens it runs route + forward."""
    from synth.device import upload_layer
    if path == "persistent" and S > 8:
        pytest.skip("the persistent kernel takes at most 8 tokens (forcing it above is an error)")
    say(f"coli_moe_layer tiny S={S} [{path}]")
    spec = synth.TINY
    d = _layer(spec, S, seed=70 + S)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    idx, w, out = gpu_layer(torch, dims, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = _oracle(spec, d)
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)


@pytest.mark.parametrize("spec", [
    dataclasses.replace(synth.TINY, wbits=8),
    dataclasses.replace(synth.TINY, wbits=2, n_shared=0, top_k=3),
    dataclasses.replace(synth.TINY, n_experts=70, top_k=9, hidden=512, inter=96, norm_topk_prob=0),
], ids=["int8", "int2-k3-noshared", "e70-k9-h512-i96-nonorm"])
@pytest.mark.parametrize("S", [2, 5])
def test_layer_entry_variants(torch, path, spec, S):
    """Up to two tokens the router launch also runs the shared expert's
    gate/up tiles; more tokens leave them to the gate/up launch."""
    from synth.device import upload_layer
    say(f"coli_moe_layer variant {spec} S={S} [{path}]")
    d = _layer(spec, S, seed=3)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    idx, w, out = gpu_layer(torch, dims, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = _oracle(spec, d)
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)


def _glm_resident_for_oracle_routing(torch, spec, S, seed, x=None, layer=0):
    """GLM-shaped layer whose resident experts are the ones the oracle routes
    the tokens to (the others are null in the table)."""
    from synth.device import blob_table
    d = synth.layer_inputs(seed, layer, spec, S)
    if x is not None:
        d["x"] = x
    o_idx, o_w, _, _ = oracle.route(spec, d["x"], d["router_w"], d["bias"])
    used = sorted(set(o_idx.ravel().tolist()))
    host = {e: synth.expert_blob(seed, layer, e, spec) for e in used}
    shared = synth.expert_blob(seed, layer, spec.n_experts, spec)
    blobs = [torch.from_numpy(host[e]).cuda() if e in host else None for e in range(spec.n_experts)]
    dl = {"x": torch.from_numpy(d["x"]).cuda(), "router_w": torch.from_numpy(d["router_w"]).cuda(),
          "bias": torch.from_numpy(d["bias"]).cuda(), "blobs": blobs,
          "table": blob_table(blobs, spec.n_experts), "shared": torch.from_numpy(shared).cuda()}
    d["blobs"] = [host.get(e) for e in range(spec.n_experts)]
    d["shared"] = shared
    return d, dl, o_idx, o_w, used


@pytest.mark.parametrize("case", ["decode-s1-int4", "verify-s4-int8"])
def test_layer_entry_glm(torch, path, case):
    """The benchmarked call at its full shape: GLM-5.2-shaped layer through
    coli_moe_layer, every output element against the oracle."""
    say(f"coli_moe_layer glm {case} [{path}]")
    if case == "decode-s1-int4":
        spec, S, x = synth.GLM, 1, None
    else:
        spec, S = synth.GLM_INT8, 4
        x = synth.verify_hidden_states(0, 0, spec, S)
    d, dl, o_idx, o_w, used = _glm_resident_for_oracle_routing(torch, spec, S, seed=0, x=x)
    dims = q().make_dims(spec)
    ws = workspace(dims, S)
    idx, w, out = gpu_layer(torch, dims, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    want = oracle.forward(spec, d["x"], o_idx, o_w, d["blobs"], d["shared"])
    say("glm layer parity", parity(out, want))


def test_layer_entry_repeat_calls_reset_the_grid_barrier(torch):
    """Back-to-back persistent launches on one workspace: each one leaves the
    barrier words at zero for the next (alternating layers and token counts)."""
    from synth.device import upload_layer
    qm = q()
    spec = synth.TINY
    dims = qm.make_dims(spec)
    ws = workspace(dims, 8)
    cases = []
    for i, S in enumerate((3, 8, 1, 6, 2)):
        d = _layer(spec, S, seed=90 + i)
        cases.append((d, upload_layer(d)))
    qm.coli_moe_debug_force_path(qm.PATH_PERSISTENT)
    try:
        for rep in range(3):
            for d, dl in cases:
                say(f"repeat {rep} S={d['x'].shape[0]}")
                idx, w, out = gpu_layer(torch, dims, dl, ws)
                assert status(ws) == 0, qm.coli_moe_last_error()
                o_out, o_idx, _ = _oracle(spec, d)
                assert np.array_equal(idx, o_idx)
                parity(out, o_out)
    finally:
        qm.coli_moe_debug_force_path(qm.PATH_AUTO)


def _layer_any(spec, S, seed):
    """Layer inputs with blobs by size (cdf recipe for large matrices)."""
    d = synth.layer_inputs(seed, 0, spec, S)
    d["blobs"] = [synth.expert_blob(seed, 0, e, spec) for e in range(spec.n_experts)]
    d["shared"] = synth.expert_blob(seed, 0, spec.n_experts, spec) if spec.n_shared else None
    return d


@pytest.mark.parametrize("spec", [
    dataclasses.replace(synth.TINY, n_experts=1024, top_k=32, hidden=256, inter=32),
    dataclasses.replace(synth.TINY, n_experts=8, top_k=2, hidden=16384, inter=64),
    dataclasses.replace(synth.TINY, n_experts=4, top_k=1, hidden=256, inter=16384, wbits=8),
], ids=["e1024-k32", "h16384", "i16384-int8"])
def test_layer_entry_limits(torch, path, spec):
    """The largest dimensions the boundary accepts (1024 experts with top-32,
    hidden 16384, inter 16384) through every kernel family."""
    from synth.device import upload_layer
    S = 3
    say(f"coli_moe_layer limits {spec} [{path}]")
    d = _layer_any(spec, S, seed=17)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    qm = q()
    try:
        idx, w, out = gpu_layer(torch, dims, dl, ws)
    except qm.ColiError as err:
        # the persistent kernel refuses shapes beyond its LDS budget
        assert path == "persistent" and err.code == qm.COLI_EINVAL, str(err)
        return
    assert status(ws) == 0, qm.coli_moe_last_error()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)


def test_grouped_batch_limit(torch):
    """The grouped kernels' pair list lives in LDS: a batch beyond 160 KiB of
    it is refused on the host (no launch), a large one within it runs."""
    from synth.device import upload_layer
    qm = q()
    spec = synth.TINY
    S = 2500
    say(f"grouped large batch S={S}")
    d = synth.tiny_layer(seed=23, S=S, spec=spec)
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    idx, w, out = gpu_layer(torch, dims, dl, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()
    o_out, o_idx, _ = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx, o_idx)
    parity(out, o_out)
    big = dataclasses.replace(spec, n_experts=64, top_k=32)
    Sb = 1400  # (32 + 1) * 1400 pair words > 160 KiB
    dims_b = qm.make_dims(big)
    x = torch.zeros((Sb, big.hidden), dtype=torch.float32, device="cuda")
    wsb = workspace(dims_b, Sb)
    table = torch.zeros(big.n_experts, dtype=torch.int64, device="cuda")
    idx_b = torch.zeros((Sb, big.top_k), dtype=torch.int32, device="cuda")
    w_b = torch.zeros((Sb, big.top_k), dtype=torch.float32, device="cuda")
    o_b = torch.zeros((Sb, big.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(qm.ColiError) as e:
        qm.coli_moe_forward(dims_b, x, idx_b, w_b, table, dl["shared"], o_b, wsb)
    assert e.value.code == qm.COLI_EINVAL


@pytest.mark.parametrize("S", [1, 4, 40])
def test_graph_replay_matches_eager(torch, path, S):
    """The benchmark replays coli_moe_layer calls from a captured HIP graph:
    every replay (with eager work and synchronisations in between) must give
    the eager call's bits, for each kernel family."""
    from synth.device import upload_layer
    if path == "persistent" and S > 8:
        pytest.skip("the persistent kernel takes at most 8 tokens")
    say(f"graph replay S={S} [{path}]")
    qm = q()
    spec = synth.TINY
    d = _layer(spec, S, seed=90 + S)
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    ref_idx, ref_w, ref_out = gpu_layer(torch, dims, dl, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()
    idx = torch.full((S, spec.top_k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((S, spec.top_k), dtype=torch.float32, device="cuda")
    out = torch.zeros((S, spec.hidden), dtype=torch.float32, device="cuda")
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        qm.coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out, ws,
                          stream=cap)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        idx.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref_out.view(np.uint32)), f"replay {rep}"
        # eager work between replays
        gpu_layer(torch, dims, dl, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()


def test_misaligned_pointers_refused(torch):
    """x, router_w, out and shared_blob are read and written 16 bytes at a
    time: a pointer off by 4 bytes is refused on the host (COLI_EINVAL),
    before anything is launched."""
    from synth.device import upload_layer
    qm = q()
    spec = synth.TINY
    d = _layer(spec, 2, seed=9)
    dims = qm.make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, 2)
    S, H = 2, spec.hidden
    xbuf = torch.zeros(S * H + 4, dtype=torch.float32, device="cuda")
    x_off = xbuf[1:1 + S * H].view(S, H)
    x_off.copy_(dl["x"])
    idx = torch.empty((S, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((S, spec.top_k), dtype=torch.float32, device="cuda")
    obuf = torch.zeros(S * H + 4, dtype=torch.float32, device="cuda")
    out_off = obuf[1:1 + S * H].view(S, H)
    out = torch.zeros((S, H), dtype=torch.float32, device="cuda")
    for call in (lambda: qm.coli_moe_route(dims, x_off, dl["router_w"], dl["bias"], idx, w, ws),
                 lambda: qm.coli_moe_layer(dims, x_off, dl["router_w"], dl["bias"], dl["table"], dl["shared"],
                                           idx, w, out, ws),
                 lambda: qm.coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"],
                                           idx, w, out_off, ws)):
        with pytest.raises(qm.ColiError) as err:
            call()
        assert err.value.code == qm.COLI_EINVAL
        assert "aligned" in str(err.value)
    qm.coli_moe_route(dims, dl["x"], dl["router_w"], dl["bias"], idx, w, ws)
    qm.coli_moe_forward(dims, dl["x"], idx, w, dl["table"], dl["shared"], out, ws)
    with pytest.raises(qm.ColiError):
        qm.coli_moe_forward(dims, dl["x"], idx, w, dl["table"], dl["shared"], out_off, ws)
    assert status(ws) == 0
    o_out, _, _ = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    parity(out.cpu().numpy(), o_out)


@pytest.mark.parametrize("S", [4, 12])
def test_repeated_index_across_groups_top10(torch, S):
    """Top-10 routing: the unit table reads each token's indices in groups of
    eight, so a repeat within the second group and a repeat across the two
    groups must both be reported (COLI_EINVAL), by the decode kernels (4
    tokens) and the grouping kernel of the grouped path (12 tokens); the
    unmodified indices give the oracle's layer again."""
    from synth.device import upload_layer
    spec = dataclasses.replace(synth.TINY, n_experts=32, top_k=10)
    d = synth.tiny_layer(seed=77, S=S, spec=spec)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    qm = q()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    idx = torch.from_numpy(o_idx).cuda()
    w = torch.from_numpy(o_w).cuda()
    say(f"repeated top-10 indices, {S} tokens")
    for k_dup, k_src in ((9, 8), (9, 1), (8, 0)):
        bad = idx.clone()
        bad[S - 1, k_dup] = bad[S - 1, k_src]
        gpu_forward(dims, dl, bad, w, ws)
        assert status(ws) == qm.COLI_EINVAL, (k_dup, k_src)
    out = gpu_forward(dims, dl, idx, w, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()
    parity(out.cpu().numpy(), o_out)


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5])
def test_top32_of_256_routing_and_layer(torch, S):
    """The widest selection the boundary admits (top-32 of 256 experts, the
    most the one-workgroup selections of one to four tokens rank) through
    coli_moe_route and coli_moe_layer: indices and weights bitwise equal to
    the oracle's, the layer output too (five tokens take the per-token
    arrival path)."""
    from synth.device import upload_layer
    spec = dataclasses.replace(synth.TINY, n_experts=256, top_k=32, hidden=256, inter=64)
    d = synth.tiny_layer(seed=91 + S, S=S, spec=spec)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    qm = q()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    say(f"top-32 of 256, {S} tokens")
    idx, w = gpu_route(dims, dl, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))
    l_idx, l_w, out = gpu_layer(torch, dims, dl, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()
    assert np.array_equal(l_idx, o_idx)
    assert np.array_equal(l_w.view(np.uint32), o_w.view(np.uint32))
    parity(out, o_out)
    assert np.array_equal(out.view(np.uint32), o_out.view(np.uint32))
