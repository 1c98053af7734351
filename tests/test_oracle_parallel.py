"""The oracle's two builds of one source: the single-threaded library and
the OpenMP one, whose loops over independent tokens run on several threads.
Routing and layer outputs must be the same bits, whatever the thread count,
so that the multi-threaded build can check large batches (the full-size
prefill test) and time the all-core CPU baseline."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth


def _same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


@pytest.mark.parametrize("spec", [
    synth.TINY,
    dataclasses.replace(synth.TINY, wbits=8),
    dataclasses.replace(synth.TINY, wbits=2, n_shared=0),
    synth.TINY_GS64,
    dataclasses.replace(synth.TINY, hidden=768, inter=96, n_experts=40, top_k=6, norm_topk_prob=0),
], ids=["int4", "int8", "int2-noshared", "gs64", "h768-i96-e40-k6"])
def test_parallel_build_is_bitwise_the_same(spec):
    S = 29
    d = synth.tiny_layer(seed=77, S=S, spec=spec)
    want_out, want_idx, want_w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"])
    for n in (8, 3):
        assert oracle.threads(n) == n
        out, idx, w = oracle.layer(spec, d["x"], d["router_w"], d["bias"], d["blobs"], d["shared"], parallel=True)
        assert np.array_equal(idx, want_idx)
        assert _same_bits(w, want_w)
        assert _same_bits(out, want_out)


def test_single_threaded_build_reports_one_thread():
    assert oracle.lib().oq_threads(4) == 1


def test_parallel_build_keeps_the_error_contract():
    """An invalid routing is refused by both builds with the same code."""
    spec = synth.TINY
    d = synth.tiny_layer(seed=3, S=6, spec=spec)
    idx = np.tile(np.arange(spec.top_k, dtype=np.int32), (6, 1))
    idx[4, 1] = idx[4, 0]   # an expert repeated within a token
    w = np.full((6, spec.top_k), 0.5, np.float32)
    for par in (False, True):
        with pytest.raises(oracle.OracleError) as e:
            oracle.forward(spec, d["x"], idx, w, d["blobs"], d["shared"], parallel=par)
        assert e.value.rc == oracle.EINVAL
    x = d["x"].copy()
    x[5, 7] = np.nan
    for par in (False, True):
        with pytest.raises(oracle.OracleError) as e:
            oracle.route(spec, x, d["router_w"], d["bias"], parallel=par)
        assert e.value.rc == oracle.ENONFINITE
