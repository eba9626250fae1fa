"""Compile the HIP library (libhqq.so) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libhqq.so")
# The same library with a minimal staging pool (one batch plus four slots): the tests run it
# so that the solver's rare pool-full paths (a lane exchanging its group in place) execute.
STRESS_LIB = os.path.join(PKG, "libhqq_stress.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                                   # fma only where written
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _compile(out: str, extra, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)


def build(verbose: bool = False, stress: bool = True) -> str:
    _compile(LIB, [], verbose)
    if stress:
        _compile(STRESS_LIB, ["-DHQQ_STRESS_SLOTS=4"], verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
