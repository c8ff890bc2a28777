"""bench.py's host-side contract: one GPU only, with a message for any other count."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_workload_switches():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--workload", "--recipe", "--output-cast", "--layernorm", "--gemm-accum", "--no-graph", "--gemm-data",
                 "--copy-reference"):
        assert flag in r.stdout
