"""Build the HIP library ``libhisparse.so`` in-tree for gfx950.

    python -m decode_memory_tiering_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "hisparse.hip")
LIB = os.path.join(PKG, "libhisparse.so")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 instructions are kept out of every kernel; the path has no
# floating point, and the flag makes sure none is generated.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def build(out: str = LIB, extra: tuple = (), verbose: bool = False) -> str:
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-I", INCLUDE, SRC, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
