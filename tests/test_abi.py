"""The C-ABI library loads on a machine without a GPU and exports every
function include/coli_moe.h declares; host-side argument checks answer
without touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli_moe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coli_moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "coli_moe_hip_build", os.path.join(ROOT, "quantized_expert_ffn_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    if not os.path.exists(b.LIB):
        b.build()
    return ctypes.CDLL(b.LIB)


def test_header_declares_the_three_entry_points():
    names = _declared()
    for n in ("coli_moe_route", "coli_moe_forward", "coli_moe_stage_experts"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_the_header():
    import quantized_expert_ffn_amd as q
    assert sorted(q.EXPORTS) == _declared()
    for n in _declared():
        assert callable(getattr(q, n))


def test_sizes_and_dim_checks_without_a_device():
    import quantized_expert_ffn_amd as q
    import synth
    assert q.coli_moe_expert_bytes(q.make_dims(synth.GLM)) == 18915328
    assert q.coli_moe_expert_bytes(q.make_dims(synth.TINY)) == 51200
    for spec in (synth.GLM, synth.GLM_INT8, synth.GLM_INT2, synth.TINY):
        assert q.coli_moe_expert_bytes(q.make_dims(spec)) == synth.blob_layout(spec.hidden, spec.inter, spec.wbits)["total"]
    assert q.coli_moe_workspace_bytes(q.make_dims(synth.GLM), 4) > 0
    bad = q.make_dims(synth.TINY)
    bad.hidden = 200
    assert q.coli_moe_expert_bytes(bad) == 0
    assert "hidden" in q.coli_moe_last_error()
    bad = q.make_dims(synth.TINY)
    bad.top_k = 0
    assert q.coli_moe_workspace_bytes(bad, 4) == 0
