"""Build libsvdq.so in-tree: HIP kernels for gfx950 with hipcc, host code with g++.

Usage: ``python -m rank_bit_residual_amd.build`` (always rebuilds).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsvdq.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # keep the compiler from forming packed-FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# per-file extra flags: the quantisation kernels keep every rounding step as written
HIP_SOURCES = {
    "k_act.hip": ["-ffp-contract=off"],
    "k_gemm.hip": [],
    "k_gemm_mx.hip": [],
    "k_gemm_decode.hip": [],
    "k_gemm_int.hip": [],
    "k_calib.hip": [],
    "k_svd.hip": [],
    "k_ceiling.hip": [],
    "capi.hip": [],
}
CXX = os.environ.get("CXX", "g++")
CXX_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-fopenmp"]
CXX_SOURCES = {
    "host_svd.cpp": ["-mavx2", "-mfma"],
    "host_prep.cpp": ["-ffp-contract=off"],
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l and "unknown target feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, extra in CXX_SOURCES.items():
        obj = os.path.join(BUILD, src + ".o")
        out = _run([CXX, *CXX_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    for src, extra in HIP_SOURCES.items():
        obj = os.path.join(BUILD, src + ".o")
        out = _run([HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp, "-lgomp"])
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
