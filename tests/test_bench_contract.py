"""bench.py's command-line contract on a machine without a GPU: more than one
GPU is refused with a message (the layer runs on one GPU), and the options
parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_options_parse():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--group-size", "--steps", "--warmup", "--tier-bits"):
        assert opt in r.stdout
