"""Builds libpagedkv.so in-tree for gfx950.

Host-only C++ (the block manager, error plumbing) is compiled with g++;
the HIP sources with hipcc for gfx950; hipcc links the shared library.

    python paged_kv_cache_421_amd/build.py [--verbose]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedkv.so")
ARCH = os.environ.get("PAGEDKV_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CXX = shutil.which("g++") or "g++"

# Packed fp32 instructions are disabled for all device code.  MFMA results
# are kept in VGPRs (the accumulator registers are left for spills): the
# kernels rescale their accumulators with ordinary vector arithmetic, which
# cannot read accumulator registers, so the default placement copies every
# accumulator out and back on each tile.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
             "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)          # host pass warns; harmless
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for name in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, name)
        obj = os.path.join(BUILD, name + ".o")
        if name.endswith(".cpp"):
            jobs.append([CXX, *CXX_FLAGS, "-c", src, "-o", obj])
        elif name.endswith(".hip"):
            jobs.append([HIPCC, *HIP_FLAGS, "-c", src, "-o", obj])
        else:
            continue
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
