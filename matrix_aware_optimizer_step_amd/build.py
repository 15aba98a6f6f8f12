"""Compile libmuon355.so in-tree for gfx950 with hipcc.

Every call recompiles.  The library lands next to this file, where the
binding loads it from.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmuon355.so")
SOURCES = ["abi.cpp", "elementwise.hip", "ns_gemm.hip", "adamw.hip", "soap.hip", "scratch.hip"]
ARCH = "gfx950"

# Packed fp32 ALU ops are disabled in all device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]
# Per-source additions.  The GEMM kernel's epilogue loops carry
# "#pragma unroll"; with the parameter update folded into the last step the
# loop over the two staged halves outgrows LLVM's default size limit for a
# pragma unroll, and a loop left rolled indexes the accumulators dynamically
# (they go to scratch memory).  A larger limit keeps every instantiation
# unrolled and the others unchanged.
EXTRA = {"ns_gemm.hip": ["-mllvm", "-pragma-unroll-threshold=65536"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmuon355")


def _compile(hipcc: str, src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err)
    return obj


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
