"""GPU check of the expert-staging tier: layers whose experts live in pinned
host memory and are copied into a small per-layer LRU of HBM slots
(coli_moe_stage_experts on a side stream), the forward running resident
experts first and the copied ones after the copy event.  Outputs must equal
the oracle's bitwise, step after step, while slots are evicted and refilled."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import parity, q, say, status, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "no GPU visible"
    return t


@pytest.mark.parametrize("bits", [4, 2])
def test_tiered_steps_match_oracle(torch, bits):
    from quantized_expert_ffn_amd.tier import ExpertTier
    import dataclasses
    spec = dataclasses.replace(synth.TINY, wbits=bits)
    L, SLOTS, STEPS = 3, 3, 6
    say(f"tiered tiny int{bits}: {L} layers, {SLOTS} slots per layer, {STEPS} steps")
    qm = q()
    dims = qm.make_dims(spec)
    E, bb = spec.n_experts, spec.blob_bytes
    layers = [synth.tiny_layer(seed=30 + l, S=STEPS, spec=spec) for l in range(L)]
    host = [[torch.from_numpy(b).pin_memory() for b in d["blobs"]] for d in layers]
    shared = [torch.from_numpy(d["shared"]).cuda() for d in layers]
    W = [torch.from_numpy(d["router_w"]).cuda() for d in layers]
    bias = [torch.from_numpy(d["bias"]).cuda() for d in layers]
    cache = torch.zeros(L * SLOTS * bb, dtype=torch.uint8, device="cuda")
    tier = ExpertTier(L, E, SLOTS, bb, slot_addr=lambda l, s: cache.data_ptr() + (l * SLOTS + s) * bb,
                      host_addr=lambda l, e: host[l][e].data_ptr())
    copy = torch.cuda.Stream()
    ws = workspace(dims, 1)
    idx = torch.empty((1, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, spec.top_k), dtype=torch.float32, device="cuda")
    staged = 0
    for s in range(STEPS):
        for l in range(L):
            x = torch.from_numpy(layers[l]["x"][s:s + 1]).cuda()
            qm.coli_moe_route(dims, x, W[l], bias[l], idx, w, ws)
            chosen = idx.cpu().numpy()[0]
            table, copies = tier.plan(l, chosen)
            ev = None
            if copies:
                ev = torch.cuda.Event()
                copy.wait_stream(torch.cuda.current_stream())
                qm.coli_moe_stage_experts([c[1] for c in copies], [c[2] for c in copies], bb, copy, ev)
                staged += len(copies)
            mask = np.zeros(E, np.uint8)
            for e, _, _ in copies:
                mask[e] = 1
            dtab = torch.tensor(table, dtype=torch.int64, device="cuda")
            out = torch.full((1, spec.hidden), float("nan"), dtype=torch.float32, device="cuda")
            qm.coli_moe_forward(dims, x, idx, w, dtab, shared[l], out, ws,
                                pending_mask=mask if copies else None, pending_ready=ev)
            assert status(ws) == 0, qm.coli_moe_last_error()
            d = layers[l]
            want, o_idx, _ = oracle.layer(spec, d["x"][s:s + 1], d["router_w"], d["bias"], d["blobs"], d["shared"])
            assert np.array_equal(chosen, o_idx[0])
            parity(out.cpu().numpy(), want)
    say("staged", staged, "hits", tier.hits, "misses", tier.misses)
    assert tier.misses == staged and staged > L * SLOTS  # slots were refilled after evictions


@pytest.mark.parametrize("bits", [4])
def test_tiered_lookahead_steps_match_oracle(torch, bits):
    """The staged flow with look-ahead: while layer l computes, the experts
    the next layer's router picks from layer l's hidden state are copied into
    the next layer's slots; at the next layer the predicted experts are hits
    whose copies may still be running (pending until the copy event), the
    others demand copies.  Every output bitwise against the oracle."""
    from quantized_expert_ffn_amd.tier import ExpertTier
    import dataclasses
    spec = dataclasses.replace(synth.TINY, wbits=bits)
    L, SLOTS, STEPS = 3, 4, 6
    say(f"tiered look-ahead tiny int{bits}: {L} layers, {SLOTS} slots per layer, {STEPS} steps")
    qm = q()
    dims = qm.make_dims(spec)
    E, bb = spec.n_experts, spec.blob_bytes
    layers = [synth.tiny_layer(seed=50 + l, S=STEPS, spec=spec) for l in range(L)]
    host = [[torch.from_numpy(b).pin_memory() for b in d["blobs"]] for d in layers]
    shared = [torch.from_numpy(d["shared"]).cuda() for d in layers]
    W = [torch.from_numpy(d["router_w"]).cuda() for d in layers]
    bias = [torch.from_numpy(d["bias"]).cuda() for d in layers]
    cache = torch.zeros(L * SLOTS * bb, dtype=torch.uint8, device="cuda")
    tier = ExpertTier(L, E, SLOTS, bb, slot_addr=lambda l, s: cache.data_ptr() + (l * SLOTS + s) * bb,
                      host_addr=lambda l, e: host[l][e].data_ptr())
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    ws = workspace(dims, 1)
    idx = torch.empty((1, spec.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, spec.top_k), dtype=torch.float32, device="cuda")
    pidx = torch.empty((1, spec.top_k), dtype=torch.int32, device="cuda")
    pw = torch.empty((1, spec.top_k), dtype=torch.float32, device="cuda")
    for s in range(STEPS):
        for l in range(L):
            d = layers[l]
            x = torch.from_numpy(d["x"][s:s + 1]).cuda()
            qm.coli_moe_route(dims, x, W[l], bias[l], idx, w, ws)
            if l + 1 < L:
                qm.coli_moe_route(dims, x, W[l + 1], bias[l + 1], pidx, pw, ws)
            chosen = idx.cpu().numpy()[0]
            table, copies, early = tier.plan_with_ahead(l, chosen)
            ev = None
            mask = None
            if copies or early:
                ev = torch.cuda.Event()
                copy.wait_stream(comp)
                qm.coli_moe_stage_experts([c[1] for c in copies], [c[2] for c in copies], bb, copy, ev)
                mask = np.zeros(E, np.uint8)
                mask[[c[0] for c in copies] + list(early)] = 1
            dtab = torch.tensor(table, dtype=torch.int64, device="cuda")
            out = torch.full((1, spec.hidden), float("nan"), dtype=torch.float32, device="cuda")
            qm.coli_moe_forward(dims, x, idx, w, dtab, shared[l], out, ws, pending_mask=mask, pending_ready=ev)
            if l + 1 < L:
                pc = tier.prefetch(l + 1, pidx.cpu().numpy()[0])
                if pc:
                    # no wait on the compute stream: the next layer's slots are
                    # not read by this layer's forward
                    qm.coli_moe_stage_experts([c[1] for c in pc], [c[2] for c in pc], bb, copy, None)
            assert status(ws) == 0, qm.coli_moe_last_error()
            want, o_idx, _ = oracle.layer(spec, d["x"][s:s + 1], d["router_w"], d["bias"], d["blobs"], d["shared"])
            assert np.array_equal(chosen, o_idx[0])
            parity(out.cpu().numpy(), want)
    torch.cuda.synchronize()
    say("prefetched", tier.prefetched, "used early", tier.prefetch_used, "hits", tier.hits, "misses", tier.misses)
    assert tier.prefetched > 0
