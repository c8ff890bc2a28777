"""Builds libfp8mp.so (the HIP kernels and the C-ABI) in-tree for gfx950.

    python -m fp8_mixed_precision_cast_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8mp.so")
BUILD = os.path.join(ROOT, "_build")

# gemm_exact_a4/a5 (the FP32-accumulation GEMM's instantiations, the longest
# to compile) come first so that they start at once
SOURCES = ["gemm_exact_a4.hip", "gemm_exact_a5.hip", "gemm_fast.hip", "gemm.hip", "api.hip", "cast.hip",
           "scale_update.hip", "layernorm.hip", "reduce.hip", "adam.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # FP arithmetic is written out exactly as meant: no contraction into FMAs,
    # IEEE division (the HIP default), no flushing of subnormals (the default).
    "-ffp-contract=off",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(jobs: int = 6, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        out = _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=6)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
