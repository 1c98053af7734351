"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the CPU-side code.

Three drivers under tests/sanitize/ are built with the sanitizers and run:
  * the CPU oracle (oracle/moe_oracle.c), every entry point and error path,
    with OpenMP threads;
  * the input generator's C helper (synth/gen.c), every blob recipe;
  * the HIP library's host code (every source, device code as shipped, host
    code instrumented): size queries, argument checks, messages and mode
    switches, up to the device query (no kernel is launched).
A sanitizer report makes the driver exit non-zero (-fno-sanitize-recover).
Builds are cached under tests/sanitize/_build, keyed by the sources' text.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(SAN_DIR, "_build")
GCC_SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"]
# host-side instrumentation only: the device code is built as shipped
HIP_SAN = ["-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="3")


def _hipbuild():
    spec = importlib.util.spec_from_file_location(
        "coli_moe_hip_build_san", os.path.join(ROOT, "quantized_expert_ffn_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _stamp(paths, extra):
    h = hashlib.sha256(" ".join(extra).encode())
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _cached(name, inputs, flags, make):
    """Runs make(out_path) unless a build of the same inputs and flags exists."""
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "%s-%s" % (name, _stamp(inputs, flags)))
    if not os.path.exists(exe):
        make(exe + ".tmp")
        os.replace(exe + ".tmp", exe)
    return exe


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s failed:\n%s\n%s" % (what, " ".join(cmd), r.stderr[-4000:])


def _check(exe, ok_line):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, "sanitized run failed (rc %d):\n%s\n%s" % (r.returncode, r.stdout[-2000:],
                                                                         r.stderr[-6000:])
    assert ok_line in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def _gcc():
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    return gcc


def test_asan_catches_a_planted_overflow():
    """The toolchain's sanitizer really reports: a one-byte heap overflow
    written for this check must fail its run."""
    gcc = _gcc()
    os.makedirs(OUT, exist_ok=True)
    src = os.path.join(OUT, "planted.c")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\nint main(void){volatile char *p = malloc(16); p[16] = 1;"
                " int r = p[0]; free((void *)p); return r;}\n")
    exe = os.path.join(OUT, "planted")
    _run([gcc, *GCC_SAN, src, "-o", exe], "gcc")
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=60)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr or "insufficient space" in r.stderr


def test_oracle_under_sanitizers():
    gcc = _gcc()
    srcs = [os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(SAN_DIR, "oracle_driver.c")]
    exe = _cached("oracle", srcs, GCC_SAN, lambda out: _run([gcc, *GCC_SAN, *srcs, "-o", out, "-lm"], "gcc"))
    _check(exe, "oracle sanitizer run ok")


def test_input_generator_under_sanitizers():
    gcc = _gcc()
    srcs = [os.path.join(ROOT, "synth", "gen.c"), os.path.join(SAN_DIR, "gen_driver.c")]
    exe = _cached("gen", srcs, GCC_SAN, lambda out: _run([gcc, *GCC_SAN, *srcs, "-o", out], "gcc"))
    _check(exe, "generator sanitizer run ok")


def test_library_host_code_under_sanitizers():
    hb = _hipbuild()
    if not os.path.exists(hb.HIPCC):
        pytest.skip("hipcc not found")
    csrc = [os.path.join(hb.CSRC, s) for s in hb.SOURCES]
    headers = sorted(os.path.join(hb.CSRC, h) for h in os.listdir(hb.CSRC) if h.endswith(".h"))
    driver = os.path.join(SAN_DIR, "host_driver.cpp")
    api_h = os.path.join(ROOT, "include", "coli_moe.h")
    flags = [*hb.FLAGS, *HIP_SAN]

    def make(out):
        objdir = out + ".objs"
        os.makedirs(objdir, exist_ok=True)

        def one(src):
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            extra = hb.EXTRA.get(os.path.basename(src), [])
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            _run([hb.HIPCC, *flags, *extra, *lang, "-c", src, "-o", obj], "hipcc")
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            objs = list(ex.map(one, csrc + [driver]))
        _run([hb.HIPCC, "--offload-arch=gfx950", *HIP_SAN, *objs, "-o", out], "link")
        shutil.rmtree(objdir, ignore_errors=True)

    exe = _cached("host", csrc + headers + [driver, api_h], flags, make)
    _check(exe, "host sanitizer run ok")
