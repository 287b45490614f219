"""Build the HIP library ``libfqm.so`` in-tree for gfx950 with hipcc.

Every source under ``csrc/`` is compiled and linked into one shared object
next to this file; the benchmark's reference kernel under ``bench_kernels/``
goes into ``libfqm_bench.so`` beside it.  Packed-FP32 instruction selection is disabled for the
device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfqm.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


BENCH_LIB = os.path.join(HERE, "libfqm_bench.so")


def bench_sources():
    return sorted(glob.glob(os.path.join(HERE, "bench_kernels", "*.hip")))


def build(verbose: bool = False) -> str:
    """Build libfqm.so (the library) and libfqm_bench.so (the benchmark's
    streaming-read reference kernel)."""
    _hipcc_shared(LIB, sources(), verbose)
    _hipcc_shared(BENCH_LIB, bench_sources(), verbose)
    return LIB


def _hipcc_shared(lib: str, srcs, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           "-o", tmp] + list(srcs)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
