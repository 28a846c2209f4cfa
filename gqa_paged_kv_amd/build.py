"""Build libgqa.so (gfx950) in-tree with hipcc.

Usage: python -m gqa_paged_kv_amd.build   (or gqa_paged_kv_amd.build.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgqa.so")
ARCH = "gfx950"

HIP_SOURCES = ["api.hip", "decode.hip", "decode_balanced.hip", "aux_kernels.hip", "prefill.hip",
               "ceiling.hip"]
CPP_SOURCES = ["validate.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # never emit packed-fp32 VALU ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgqa")


def build(verbose: bool = False) -> str:
    """Compile every source and link libgqa.so next to this file; returns its path."""
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in HIP_SOURCES + CPP_SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        if src.endswith(".cpp"):
            cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", path, "-o", obj]
        else:
            cmd = [hipcc, *HIPCC_FLAGS, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
