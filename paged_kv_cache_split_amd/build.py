"""Build libkvc.so in-tree with hipcc for gfx950.

Usage: python paged_kv_cache_split_amd/build.py   (runs without importing the package,
whose import needs the built library)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libkvc.so")
SOURCES = [os.path.join(CSRC, "kvc_host.cpp"), os.path.join(CSRC, "kvc_sched.cpp"),
           os.path.join(CSRC, "kvc_kernels.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 instructions anywhere (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE float32 division: the fp8 scale rule divides and must round exactly
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # matrix-core accumulators in ordinary VGPRs (no AGPR copies around the
    # online-softmax rescale)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # single-lane atomics stay single-lane: the wave-wide rewrite reads the
    # result right after issuing it, which would stall the decode's ticket
    # request that is meant to overlap the chunk's last blocks
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libkvc")
    return path


def build_library(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
