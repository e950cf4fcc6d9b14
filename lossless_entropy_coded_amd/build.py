"""Build libwc.so (host encoder + planner + gfx950 kernels) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libwc.so")
SOURCES = ["decode.hip", "decode_lanes.hip", "gemv.hip", "noalloc.hip", "stream.hip", "plan.cpp", "encode.cpp"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # packed-fp32 instructions stay off in every HIP build of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no unaligned LDS/global accesses: the decode kernel's byte stores must not
    # be merged into unaligned dword LDS stores, which stall on CDNA4
    "-Xclang", "-target-feature", "-Xclang", "-unaligned-access-mode",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build_library(verbose: bool = False) -> str:
    """Compile every source into lossless_entropy_coded_amd/libwc.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp, "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
    sys.exit(0)
