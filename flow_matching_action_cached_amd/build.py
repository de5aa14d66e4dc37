"""Build libphyai.so (HIP kernels for gfx950 + the C-ABI runtime) in-tree.

Usage: python -m flow_matching_action_cached_amd.build   (or call build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libphyai.so")

SOURCES = [os.path.join(CSRC, n)
           for n in ("loop.hip", "gemv.hip", "attention.hip", "update.hip", "loop_persistent.hip", "gemm_tiled.hip",
                     "tables.hip", "runtime.cpp")]
HEADERS = [os.path.join(CSRC, n) for n in ("common.h", "kernels.h", "epilogue.h", "launch.h", "persistent.h")] + \
    [os.path.join(INCLUDE, "phyai.h")]

# Packed-fp32 VALU forms are kept out of every code object (they are not needed here and
# the build stays on plain fp32 instructions).
GPU_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # leading scalar kernel arguments are preloaded into SGPRs at wave launch
             "-mllvm", "-amdgpu-kernarg-preload-count=8"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, phase_trace: bool = False) -> str:
    """Compile every source for gfx950 and link libphyai.so next to this file.

    phase_trace=True builds libphyai_trace.so instead: the same library with per-wave phase
    timestamps recorded by the kernels (exported readers phyai_phase_trace_gemv, _attn and
    _update, and phyai_persist_trace for the persistent loop)."""
    cc = hipcc()
    objs = []
    objdir = os.path.join(PKG, "_build_trace" if phase_trace else "_build")
    lib = LIB.replace("libphyai.so", "libphyai_trace.so") if phase_trace else LIB
    extra = ["-DPHYAI_PHASE_TRACE"] if phase_trace else []
    os.makedirs(objdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *GPU_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        objs.append(obj)
    tmp = lib + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_trace="--phase-trace" in sys.argv))
