"""bench.py's command-line contract, checked without a GPU: it runs on one GPU
only, so --gpus above 1 exits with a message (status 2) before touching a
device, and the argument parser lists every workload."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "4")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 4" in r.stderr


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("prefill", "decode", "rdc", "dense", "dense16k", "prefill_bwd", "decode_bwd"):
        assert w in r.stdout
