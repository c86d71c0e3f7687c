"""Build libtreeattn.so in-tree for gfx950.

HIP sources go through hipcc (--offload-arch=gfx950); the host-only C++
sources go through g++ with the HIP headers.  Objects land in ``_build/``
next to this file, the library in this package directory.  Packed-fp32 VALU
forms are disabled for all device code.

    python -m prefix_tree_attention_amd.build [-j N] [--verbose]
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
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libtreeattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["meta.hip", "fwd_bf16.hip", "bwd_bf16.hip", "attn_f32.hip", "logprob.hip", "rope.hip", "noalloc.hip", "dfs.hip"]
CXX_SOURCES = ["capi.cpp", "status.cpp", "pack.cpp", "dfs.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC]
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-ffast-math", "-fno-finite-math-only", "-munsafe-fp-atomics",
             "-mllvm", "-amdgpu-mfma-vgpr-form"]
CXX_FLAGS = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append([HIPCC, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in CXX_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        cmds.append(["g++", *COMMON, *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    shutil.move(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-j", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.j, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
