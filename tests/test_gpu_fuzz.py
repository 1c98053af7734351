"""Seeded shape sweep: layers of many small shapes (odd expert counts, top-k
from 1 to 10, one-block intermediates, every code width, group scales, with
and without the shared expert and the renormalisation) through
coli_moe_layer and through coli_moe_route + coli_moe_forward, each against
the oracle: routing bit-exact, outputs within the layer tolerance and
bitwise equal."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import gpu_forward, gpu_route, parity, q, say, status, workspace

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(i):
    """Dimensions of case i, drawn from a generator seeded by i (every draw
    is one check_dims admits)."""
    rng = np.random.default_rng(9000 + i)
    bits = int(rng.choice([8, 4, 2]))
    big_e = rng.random() < 0.3
    E = int(rng.integers(257, 301)) if big_e else int(rng.integers(1, 65))
    K = int(rng.integers(1, min(E, 10) + 1))
    H = int(rng.choice([256, 512] if big_e else [256, 512, 768, 1024]))
    I = int(rng.choice([32, 64, 96, 128] if big_e else [32, 64, 96, 160, 256]))
    group = 0
    if bits == 4 and rng.random() < 0.4:
        group = int(rng.choice([g for g in (32, 64) if H % g == 0 and I % g == 0]))
    spec = dataclasses.replace(synth.TINY, hidden=H, inter=I, n_experts=E, top_k=K,
                               n_shared=int(rng.integers(0, 2)), wbits=bits, group=group,
                               norm_topk_prob=int(rng.integers(0, 2)),
                               routed_scaling_factor=float(np.float32(rng.choice([1.0, 2.5, 0.75]))))
    S = int(rng.choice([1, 2, 3, 6, 9, 12]))
    return spec, S


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "no GPU visible"
    return t


@pytest.mark.parametrize("i", range(N_CASES))
def test_shape_sweep(torch, i):
    from synth.device import upload_layer
    spec, S = _case(i)
    say(f"sweep case {i}: S={S} {spec}")
    d = synth.tiny_layer(seed=100 + i, S=S, spec=spec)
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    dims = q().make_dims(spec)
    dl = upload_layer(d)

    ws = workspace(dims, S)
    idx = torch.full((S, spec.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((S, spec.top_k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((S, spec.hidden), float("nan"), dtype=torch.float32, device="cuda")
    q().coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out, ws)
    assert status(ws) == 0, q().coli_moe_last_error()
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))
    parity(out.cpu().numpy(), o_out)

    ws2 = workspace(dims, S)
    idx2, w2 = gpu_route(dims, dl, ws2)
    out2 = gpu_forward(dims, dl, idx2, w2, ws2)
    assert status(ws2) == 0, q().coli_moe_last_error()
    assert np.array_equal(idx2.cpu().numpy(), o_idx)
    parity(out2.cpu().numpy(), o_out)
