"""Builds libpagedkv.so in-tree for gfx950, and libpagedkv_debug.so, the
same sources with PA_DEBUG defined (values inside device arrays -- block ids,
slots, lengths, copy pairs -- are checked on the host before any launch).

Host-only C++ (the block manager, error plumbing) is compiled with g++;
the HIP sources with hipcc for gfx950; hipcc links the shared libraries.

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
DEBUG_LIB = os.path.join(PKG, "libpagedkv_debug.so")
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


def _variant(out_dir, extra):
    """Compile commands and object files of one build variant."""
    os.makedirs(out_dir, exist_ok=True)
    jobs, objs = [], []
    for name in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, name)
        obj = os.path.join(out_dir, name + ".o")
        if name.endswith(".cpp"):
            jobs.append([CXX, *CXX_FLAGS, *extra, "-c", src, "-o", obj])
        elif name.endswith(".hip"):
            jobs.append([HIPCC, *HIP_FLAGS, *extra, "-c", src, "-o", obj])
        else:
            continue
        objs.append(obj)
    return jobs, objs


# Host-only part (block manager, error messages) under AddressSanitizer and
# UndefinedBehaviorSanitizer, for the block-manager tests; g++ only.
HOST_SAN_LIB = os.path.join(BUILD, "sanitize", "libpagedkv_host_asan.so")
HOST_SAN_SOURCES = ["block_manager.cpp", "status.cpp"]


def build_host_sanitized(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(HOST_SAN_LIB), exist_ok=True)
    tmp = HOST_SAN_LIB + ".tmp"
    _run([CXX, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", INCLUDE, "-I", CSRC,
          *[os.path.join(CSRC, n) for n in HOST_SAN_SOURCES], "-o", tmp], verbose)
    os.replace(tmp, HOST_SAN_LIB)
    return HOST_SAN_LIB


def build(verbose: bool = False) -> str:
    rel_jobs, rel_objs = _variant(BUILD, [])
    dbg_jobs, dbg_objs = _variant(os.path.join(BUILD, "debug"), ["-DPA_DEBUG"])
    jobs = rel_jobs + dbg_jobs
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    for lib, objs in ((LIB, rel_objs), (DEBUG_LIB, dbg_objs)):
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, lib)
    build_host_sanitized(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
