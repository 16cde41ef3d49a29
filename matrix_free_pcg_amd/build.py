"""Build the HIP library (libmfpcg.so) for gfx950 with hipcc.

The library is a plain shared object with a C ABI (include/mfpcg.h); the
Python binding loads it with ctypes.  Building writes
``matrix_free_pcg_amd/lib/libmfpcg.so`` in the source tree, and
``lib/libmfprobe.so``, the streaming-bandwidth probe that bench.py
--stream-probe runs (a measurement tool, not part of the solver).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmfpcg.so")
SOURCES = [os.path.join(CSRC, "mfpcg.hip")]
PROBE_SRC = os.path.join(CSRC, "stream_probe.hip")
PROBE_LIB = os.path.join(LIBDIR, "libmfprobe.so")
DEPENDS = SOURCES + [os.path.join(CSRC, "kernels.hpp"), os.path.join(INCLUDE, "mfpcg.h")]

ARCH = os.environ.get("MFPCG_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # never emit packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found (ROCm is required to build libmfpcg.so)")


def _compile(sources, out, verbose, extra):
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    """Compile the library into LIB and the probe into PROBE_LIB (always recompiles)."""
    os.makedirs(LIBDIR, exist_ok=True)
    _compile(SOURCES, LIB, verbose, extra)
    _compile([PROBE_SRC], PROBE_LIB, verbose, extra)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPENDS)


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    print(LIB)
