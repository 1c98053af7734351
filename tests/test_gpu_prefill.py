"""GPU parity of the grouped kernels (int8 matrix-core gate/up and down per
32-row tile and tile of up to 32 (token, expert) pairs of one expert), which
serve batches of 9 or more tokens: bit-exact routing against the oracle's
router and binary32 layer outputs bitwise equal to the oracle's.

Inputs follow the batch-union prefill workload: tokens routed with a
Zipf(1.1) skew over expert popularity (Gumbel-top-K through the
pseudo-inverse of the router gate, zero bias)."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import parity, q, say, status, workspace

pytestmark = pytest.mark.gpu

# a mid-size layer the oracle finishes in seconds, with enough tokens per
# popular expert for several tiles and a ragged last one
MID = synth.LayerSpec(hidden=512, inter=256, n_experts=64, top_k=8, n_shared=1, wbits=4)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "no GPU visible"
    return t


def _upload(torch, d):
    from synth.device import blob_table
    spec = d["spec"]
    blobs = [None if b is None else torch.from_numpy(b).cuda() for b in d["blobs"]]
    return {"x": torch.from_numpy(d["x"]).cuda(), "router_w": torch.from_numpy(d["router_w"]).cuda(),
            "bias": torch.from_numpy(d["bias"]).cuda(), "blobs": blobs,
            "table": blob_table(blobs, spec.n_experts),
            "shared": None if d["shared"] is None else torch.from_numpy(d["shared"]).cuda()}


def _zipf_layer(spec, S, seed=0):
    d = synth.layer_inputs(seed, 0, spec, S)
    d["x"] = synth.prefill_hidden_states(seed, 0, spec, S)
    d["bias"] = np.zeros(spec.n_experts, np.float32)
    d["blobs"] = [synth.expert_blob(seed, 0, e, spec) for e in range(spec.n_experts)]
    d["shared"] = synth.expert_blob(seed, 0, spec.n_experts, spec) if spec.n_shared else None
    return d


def _layer_call(torch, spec, dl, ws):
    S = dl["x"].shape[0]
    idx = torch.full((S, spec.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((S, spec.top_k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, spec.hidden), float("nan"), dtype=torch.float32, device="cuda")
    q().coli_moe_layer(q().make_dims(spec), dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"],
                       idx, w, out, ws)
    return idx, w, out


def _histogram(idx, E):
    c = np.bincount(idx.ravel(), minlength=E)
    return {"unique": int((c > 0).sum()), "min": int(c[c > 0].min()), "median": float(np.median(c[c > 0])),
            "max": int(c.max())}


@pytest.mark.parametrize("fmt", ["int4", "int8", "int2", "mxfp4"])
def test_mid_zipf_layer(torch, fmt):
    """coli_moe_layer at 160 tokens (grouped kernels by default; MXFP4
    experts on the FP4 matrix cores): every output element against the
    oracle."""
    bits = 4 if fmt == "mxfp4" else int(fmt[3:])
    spec = dataclasses.replace(MID, wbits=bits, fmt=1 if fmt == "mxfp4" else 0)
    S = 160
    say(f"grouped mid layer S={S} {fmt}")
    d = _zipf_layer(spec, S, seed=bits + (10 if fmt == "mxfp4" else 0))
    dl = _upload(torch, d)
    ws = workspace(q().make_dims(spec), S)
    idx, w, out = _layer_call(torch, spec, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    idx = idx.cpu().numpy()
    h = _histogram(idx, spec.n_experts)
    say("routing", h)
    assert h["max"] > 64  # at least one expert spans three tiles
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))
    say("parity", parity(out.cpu().numpy(), o_out))


def test_tile_boundaries(torch):
    """Units of exactly 32 and 64 pairs, of one pair, and a shared unit of
    97 (three full tiles and a tail of one); routing fixed through one-hot
    router rows (x carries the logits in its first E entries)."""
    say("grouped tile boundaries S=97")
    spec = dataclasses.replace(synth.TINY, n_experts=16, top_k=2)
    S, E = 97, spec.n_experts
    d = synth.tiny_layer(seed=9, S=S, spec=spec)
    lg = np.full((S, E), -4.0, np.float32)
    lg[:64, [0, 1]] = 3.0
    lg[64:96, [2, 3]] = 3.0
    lg[96, [4, 5]] = 3.0
    lg[:, 1] += 0.5  # distinct ranks inside a token
    lg[64:96, 3] += 0.5
    lg[96, 5] += 0.5
    d["x"] = d["x"].copy()
    d["x"][:, :E] = lg
    W = np.zeros((E, spec.hidden), np.float32)
    W[np.arange(E), np.arange(E)] = 1.0
    d["router_w"] = W
    d["bias"] = np.zeros(E, np.float32)
    dl = _upload(torch, d)
    ws = workspace(q().make_dims(spec), S)
    idx, w, out = _layer_call(torch, spec, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    c = np.bincount(idx.cpu().numpy().ravel(), minlength=E)
    assert c[:6].tolist() == [64, 64, 32, 32, 1, 1]
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    parity(out.cpu().numpy(), o_out)


def test_pending_experts_grouped(torch):
    """Grouped kernels with a pending mask: the whole forward waits for the
    event, and the result equals the unmasked call."""
    say("grouped pending mask S=20")
    from tests.gpu_util import gpu_forward, gpu_route
    spec = synth.TINY
    d = synth.tiny_layer(seed=12, S=20, spec=spec)
    dl = _upload(torch, d)
    dims = q().make_dims(spec)
    ws = workspace(dims, 20)
    idx, w = gpu_route(dims, dl, ws)
    ref = gpu_forward(dims, dl, idx, w, ws).cpu().numpy()
    mask = np.zeros(spec.n_experts, np.uint8)
    mask[idx[0].cpu().numpy()] = 1
    ev = torch.cuda.Event()
    ev.record()
    out = gpu_forward(dims, dl, idx, w, ws, pending_mask=mask, pending_ready=ev).cpu().numpy()
    assert status(ws) == 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    o_out, _, _ = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    parity(out, o_out)


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_glm_prefill_2048_zipf(torch, fmt):
    """The batch-union prefill workload at its full size: GLM-5.2-shaped
    layer (H 6144, I 2048, 256 experts top-8 + shared, int4 or MXFP4), 2048
    tokens with Zipf(1.1) expert popularity, through coli_moe_layer as the
    benchmark calls it.  Routing of all tokens against the oracle's router,
    and every output row bitwise against the oracle's forward (the
    multi-threaded build of the oracle, over chunks of tokens; it gives the
    same bits as the single-threaded one)."""
    spec, S = (synth.GLM_MX if fmt == "mxfp4" else synth.GLM), 2048
    say(f"glm prefill S={S} {fmt}: generating inputs")
    d = synth.layer_inputs(0, 0, spec, S)
    d["x"] = synth.prefill_hidden_states(0, 0, spec, S)
    d["bias"] = np.zeros(spec.n_experts, np.float32)
    E, bb = spec.n_experts, spec.blob_bytes
    host = np.empty((E + 1) * bb, np.uint8)
    fill = synth.mx_cdf_expert_into if fmt == "mxfp4" else synth.cdf_expert_into
    for e in range(E + 1):
        fill(host.ctypes.data + e * bb, 0, 0, e, spec)
    dev = torch.from_numpy(host).cuda()
    table = torch.tensor([dev.data_ptr() + e * bb for e in range(E)], dtype=torch.int64, device="cuda")
    dl = {"x": torch.from_numpy(d["x"]).cuda(), "router_w": torch.from_numpy(d["router_w"]).cuda(),
          "bias": torch.from_numpy(d["bias"]).cuda(), "table": table, "shared": dev.data_ptr() + E * bb}
    ws = workspace(q().make_dims(spec), S)
    say("glm prefill: layer call")
    idx, w, out = _layer_call(torch, spec, dl, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    idx = idx.cpu().numpy()
    w = w.cpu().numpy()
    out = out.cpu().numpy()
    del dev, dl, ws, table
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(out))
    h = _histogram(idx, E)
    say("routing", h)
    assert h["unique"] == E and h["max"] > 1000
    nthr = oracle.threads()
    say(f"glm prefill: oracle routing of all tokens ({nthr} threads)")
    o_idx, o_w, _, _ = oracle.route(spec, d["x"], d["router_w"], d["bias"], parallel=True)
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(w.view(np.uint32), o_w.view(np.uint32))
    blobs = [host[e * bb:(e + 1) * bb] for e in range(E)]
    shared = host[E * bb:(E + 1) * bb]
    CH = 128
    n_diff = 0
    for t0 in range(0, S, CH):
        t1 = min(S, t0 + CH)
        want = oracle.forward(spec, d["x"][t0:t1], o_idx[t0:t1], o_w[t0:t1], blobs, shared, parallel=True)
        st = parity(out[t0:t1], want, bitwise=False)
        n_diff += st["bit_diffs"]
        say(f"glm prefill: tokens {t0}..{t1 - 1} against the oracle: rel-L2 {st['rel_l2']:.2e}, "
            f"{st['bit_diffs']} elements differ in bits")
    assert n_diff == 0, f"{n_diff} of {S * spec.hidden} output elements differ in bits"
