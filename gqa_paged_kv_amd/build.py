"""Build libgqa.so (gfx950) in-tree with hipcc, and libgqa_debug.so: the same kernels with
the entry points compiled with GQA_DEBUG (page ids checked on the host before every launch).

Usage: python -m gqa_paged_kv_amd.build            (or gqa_paged_kv_amd.build.build())
       python -m gqa_paged_kv_amd.build --valu-scores
           also builds libgqa_valu_scores.so, whose balanced bf16 decode computes the scores
           on the vector ALU instead of the matrix core (for side-by-side measurements:
           bench.py --lib gqa_paged_kv_amd/libgqa_valu_scores.so)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgqa.so")
DEBUG_LIB = os.path.join(HERE, "libgqa_debug.so")
VALU_SCORES_LIB = os.path.join(HERE, "libgqa_valu_scores.so")
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


def build(verbose: bool = False, valu_scores: bool = False) -> str:
    """Compile every source and link libgqa.so (and libgqa_debug.so; with valu_scores also
    libgqa_valu_scores.so) next to this file; returns the path of libgqa.so."""
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds, objs = [], []
    for src in HIP_SOURCES + CPP_SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        if src.endswith(".cpp"):
            cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", path, "-o", obj]
        else:
            cmd = [hipcc, *HIPCC_FLAGS, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        cmds.append(cmd)
        objs.append(obj)
    # the entry points once more with the debug page-id checks
    dbg_obj = os.path.join(objdir, "api.hip.debug.o")
    cmds.append([hipcc, *HIPCC_FLAGS, "-DGQA_DEBUG", "-c", os.path.join(CSRC, "api.hip"), "-o",
                 dbg_obj])
    valu_obj = os.path.join(objdir, "decode_balanced.hip.valu.o")
    if valu_scores:
        cmds.append([hipcc, *HIPCC_FLAGS, "-DGQA_DECODE_VALU_SCORES=1", "-c",
                     os.path.join(CSRC, "decode_balanced.hip"), "-o", valu_obj])
    # one compiler process per source, at most as many as the host has cores (and 8)
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as pool:
        for r in list(pool.map(lambda c: subprocess.run(c), cmds)):
            if r.returncode != 0:
                raise subprocess.CalledProcessError(r.returncode, r.args)
    api_obj = os.path.join(objdir, "api.hip.o")
    bal_obj = os.path.join(objdir, "decode_balanced.hip.o")
    libs = [(LIB, objs), (DEBUG_LIB, [dbg_obj if o == api_obj else o for o in objs])]
    if valu_scores:
        libs.append((VALU_SCORES_LIB, [valu_obj if o == bal_obj else o for o in objs]))
    for lib, lib_objs in libs:
        tmp = lib + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *lib_objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, valu_scores="--valu-scores" in sys.argv))
