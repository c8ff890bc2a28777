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
                 "--copy-reference", "--steps-per-graph"):
        assert flag in r.stdout


def test_steps_per_graph_divides_the_timed_steps():
    """The timed region replays whole graphs: the steps per graph is the largest divisor of --steps not above
    the request, so exactly --steps steps are timed."""
    import bench
    assert [bench.steps_per_graph(k, 10) for k in (1, 2, 3, 7, 12, 20, 50, 97, 100)] == [1, 2, 3, 7, 6, 10, 10, 1, 10]
    assert bench.steps_per_graph(20, 1) == 1 and bench.steps_per_graph(20, 0) == 1
    for k in range(1, 60):
        for want in range(1, 15):
            d = bench.steps_per_graph(k, want)
            assert k % d == 0 and 1 <= d <= max(1, want)


def test_source_digest_ignores_comments_and_whitespace_only():
    """The counters' digest follows the GEMM code, not its comments: stripping keeps code and string literals."""
    import bench
    a = bench.code_text('int f() { return 1; } // one\n/* block */\nconst char* s = "// kept";')
    b = bench.code_text('int  f()  {\n  return 1;\n}\nconst char* s = "// kept";   // trailing')
    assert a == b == 'int f() { return 1; } const char* s = "// kept";'
    assert bench.code_text("x = 1;") != bench.code_text("x = 2;")
    assert len(bench.source_digest()) == 16
