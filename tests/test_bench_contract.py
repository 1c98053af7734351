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


def test_graph_plan_times_exactly_the_requested_steps():
    """Timed steps are whole replays of one graph, exactly --steps of them;
    warmup is exactly --warmup steps and includes a replay of the graph
    whenever it is not empty; several replays give the spread."""
    sys.path.insert(0, ROOT)
    import bench
    for K in (1, 2, 5, 7, 20, 50, 64, 200, 2400, 97):
        for W in (0, 1, 3, 5, 10, 20, 240):
            for cap in (10, 240):
                G, reps, reps_w, eager = bench.graph_plan(K, W, cap)
                assert 1 <= G <= cap and G * reps == K
                assert reps_w * G + eager == W
                if W > 0:
                    assert reps_w >= 1
                if K >= 5:
                    assert reps >= 5
