"""Build libgca.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgca.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are switched off for all device code.  No NaN is ever
# produced on the path (masked scores and empty maxima are -inf, which stays
# honoured), so fmax needs no NaN-quieting of its operands.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fno-honor-nans",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return [os.path.join(CSRC, "gca_kernels.hip"), os.path.join(CSRC, "gca_runtime.cpp")]


def build(verbose: bool = False) -> str:
    """Compile every source into libgca.so; always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, "-fPIC", "-shared", "-I", os.path.join(ROOT, "include"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libgca.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
