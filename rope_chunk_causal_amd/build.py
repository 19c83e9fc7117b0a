"""Build librcc.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m rope_chunk_causal_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librcc.so")
SOURCES = ["rcc_abi.cpp", "rope3d.hip", "attn.hip", "attn_d128.hip", "attn_sparse.hip",
           "qkv_rope.hip"]
# The fast attention kernels never rely on NaN semantics (masking uses
# -inf); without NaN honouring fmaxf needs no quieting of its operands.
FILE_FLAGS = {"attn_d128.hip": ["-fno-honor-nans"], "attn_sparse.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from emitting packed fp32 VALU ops.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source and link librcc.so; returns the library path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), "-x", "hip", *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
