"""A failure path forced from the host, with every kernel ending normally.

The router launch of one to four tokens selects in one workgroup that
waits, bounded, for the logits its other workgroups publish.  coli_moe_debug_route_wait
makes that wait look for a tag no workgroup writes, with a short bound, so
it always gives up.  The contract for that case (a failure is reported,
never hidden behind a fallback: colibrì README v1.0, "Experimental resident
CUDA backend"): the status is COLI_EHIP with a timed-out message, the unit
table holds the shared expert alone, so the output is exactly the shared
expert's (0 + y_shared, the combine's chain with no routed term), and the
next call with the normal wait is bitwise the oracle's layer again."""
import dataclasses

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


def _call(torch, dims, dl, ws):
    S = dl["x"].shape[0]
    idx = torch.empty((S, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((S, dims.top_k), dtype=torch.float32, device="cuda")
    out = torch.full((S, dims.hidden), float("nan"), dtype=torch.float32, device="cuda")
    q().coli_moe_layer(dims, dl["x"], dl["router_w"], dl["bias"], dl["table"], dl["shared"], idx, w, out, ws)
    return idx, w, out


@pytest.mark.parametrize("fmt,S", [("int4", 1), ("int8", 1), ("mxfp4", 1), ("int4", 2), ("int8", 4), ("mxfp4", 3)])
def test_router_wait_gives_up_routes_the_shared_expert_alone(torch, fmt, S):
    from synth.device import upload_layer
    spec = {"int4": synth.TINY, "int8": dataclasses.replace(synth.TINY, wbits=8), "mxfp4": synth.TINY_MX}[fmt]
    d = synth.tiny_layer(seed=31, S=S, spec=spec)
    dims = q().make_dims(spec)
    dl = upload_layer(d)
    ws = workspace(dims, S)
    qm = q()
    say(f"router wait forced to give up ({fmt}, {S} tokens)")
    qm.coli_moe_debug_route_wait(64, 1)
    try:
        _, _, out = _call(torch, dims, dl, ws)
        rc = status(ws)
    finally:
        qm.coli_moe_debug_route_wait(0, 0)
    assert rc == qm.COLI_EHIP and "timed out" in qm.coli_moe_last_error()
    got = out.cpu().numpy()
    for t in range(S):
        qx, dx = oracle.q8_0(d["x"][t])
        y = oracle.expert(d["shared"], spec.hidden, spec.inter, spec.wbits, qx, dx, spec.group, spec.fmt)["y"]
        want = (np.float32(0.0) + y).astype(np.float32)
        assert np.array_equal(got[t].view(np.uint32), want.view(np.uint32)), t
    say(f"router wait restored ({fmt}, {S} tokens)")
    idx, w, out = _call(torch, dims, dl, ws)
    assert status(ws) == 0, qm.coli_moe_last_error()
    o_out, o_idx, o_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))
    parity(out.cpu().numpy(), o_out)
