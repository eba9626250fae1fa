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
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                                   # fma only where written
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _objects(jobs, verbose: bool) -> None:
    """Compiles (source, object, extra flags) jobs in parallel, each to a temporary file
    renamed into place when it succeeds."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    procs = []
    for src, obj, extra in jobs:
        cmd = [hipcc, *HIPCC_FLAGS, *extra, "-c", "-I", os.path.join(ROOT, "include"),
               "-I", os.path.join(PKG, "csrc"), "-o", obj + ".tmp", src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), obj))
    failed = [obj for p, obj in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, "hipcc", f"failed: {failed}")
    for _, obj in procs:
        os.replace(obj + ".tmp", obj)


def _link(out: str, objs, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, stress: bool = True) -> str:
    """Every source to an object in parallel (the stress library recompiles only the solver,
    the one file its macro changes), then one link per library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    obj = lambda src, tag="": os.path.join(objdir, os.path.basename(src)[:-4] + tag + ".o")
    jobs = [(src, obj(src), []) for src in sources()]
    stream_src = os.path.join(PKG, "csrc", "hqq_stream.hip")
    if stress:
        jobs.append((stream_src, obj(stream_src, "_stress"), ["-DHQQ_STRESS_SLOTS=4"]))
    _objects(jobs, verbose)
    _link(LIB, [obj(src) for src in sources()], verbose)
    if stress:
        _link(STRESS_LIB, [obj(src, "_stress") if src == stream_src else obj(src)
                           for src in sources()], verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
