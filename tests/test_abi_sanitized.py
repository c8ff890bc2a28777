"""The C-ABI front end (argument validation and dispatch in csrc/api.hip) built with host address and
undefined-behaviour sanitizers, the kernel launchers replaced by host stubs, and driven through every
entry point by tests/sanitize/abi_driver.cpp on the CPU. A sanitizer report (out-of-bounds access,
signed overflow in a size check, misaligned load, ...) or an unexpected status fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-side sanitizers only: device code is never instrumented
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all".split()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_c_abi_front_end_under_host_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "fp8_mixed_precision_cast_amd", "csrc")]
    common = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "--offload-arch=gfx950"]
    objs = []
    for src, lang in ((os.path.join(ROOT, "fp8_mixed_precision_cast_amd", "csrc", "api.hip"), "hip"),
                      (os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "hip"),
                      (os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "hip")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, *common, *SAN, *inc, "-x", lang, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([HIPCC, *common, *SAN, *objs, "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES=os.environ.get(
                   "HIP_VISIBLE_DEVICES", ""))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert r.returncode == 0, out
    assert "0 failures" in r.stdout
