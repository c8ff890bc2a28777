"""The GEMM's tile plan and persistent walk, checked on the CPU by tests/plan/plan_check.cpp, which is built
from the kernel header itself: every output cell covered by exactly one tile for the workloads' shapes and 300
random shapes on several CU counts, and every tile id taken by exactly one workgroup, each keeping to its XCD."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_tile_plan_covers_every_output_once_and_walk_takes_every_tile_once(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "fp8_mixed_precision_cast_amd", "csrc")]
    exe = str(tmp_path / "plan_check")
    cmd = [HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", *inc, "-x", "hip",
           os.path.join(ROOT, "tests", "plan", "plan_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
