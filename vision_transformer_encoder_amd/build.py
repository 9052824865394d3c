"""Build ``libvitblk.so`` in-tree for gfx950 with hipcc.

Usage: ``python -m vision_transformer_encoder_amd.build`` (or ``build()``).
Every call recompiles every source; objects go to ``_build/`` next to the
package and the library to ``vision_transformer_encoder_amd/libvitblk.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libvitblk.so")

ARCH = os.environ.get("VITBLK_OFFLOAD_ARCH", "gfx950")
HIP_SOURCES = ["api.hip", "layernorm.hip", "gemm.hip", "gemm_f32.hip", "attention.hip", "attention_f32.hip",
               "attention_resident.hip", "patch.hip", "generic.hip", "pack.hip",
               "backward.hip", "wgrad.hip", "attention_bwd.hip"]
HOST_SOURCES = ["validate.cpp"]

# Packed-fp32 instructions are disabled for all device code; a variable read
# before it is set (e.g. a local initialised from itself) is an error.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Werror=uninitialized", "-Werror=sometimes-uninitialized",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvitblk.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    if verbose and r.stdout.strip():
        print(r.stdout, flush=True)
    return r.stdout


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link the shared library; return its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    incs = [f"-I{INCLUDE}", f"-I{CSRC}"]
    steps = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        steps.append([hipcc, *HIP_FLAGS, *incs, "-c", os.path.join(CSRC, src), "-o", obj])
    cxx = shutil.which("g++") or shutil.which("c++")
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        steps.append([cxx, *HOST_FLAGS, *incs, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(steps), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
