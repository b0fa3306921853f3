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


def build(verbose: bool = False, defines=(), name: str = "libgca.so") -> str:
    """Compile every source into libgca.so (or `name`, in the package
    directory, with extra -D `defines`: the kernels' compile-time variants);
    always recompiles."""
    lib = os.path.join(PKG, name)
    tmp = lib + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, *[f"-D{d}" for d in defines], "-fPIC", "-shared",
           "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libgca.so")
    os.replace(tmp, lib)
    return lib


PROBE_SRC = os.path.join(CSRC, "issue_rate_probe.hip")
PROBE = os.path.join(PKG, "issue_rate_probe")


def build_probe(verbose: bool = False) -> str:
    """Compile the VALU/MFMA issue-rate probe (a diagnostic executable)."""
    tmp = PROBE + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build the issue-rate probe")
    os.replace(tmp, PROBE)
    return PROBE


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra define, e.g. GCA_SOFT_EXP=4")
    ap.add_argument("--name", default="libgca.so", help="library file name in the package directory")
    ap.add_argument("--probe", action="store_true", help="build the issue-rate probe executable instead")
    a = ap.parse_args()
    print(build_probe(verbose=True) if a.probe else build(verbose=True, defines=a.defines, name=a.name))
