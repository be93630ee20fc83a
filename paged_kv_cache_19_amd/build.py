"""Build libpa.so (the HIP kernels and the C ABI) in-tree for gfx950.

``python -m paged_kv_cache_19_amd.build`` compiles every source under
``csrc/`` with hipcc into ``paged_kv_cache_19_amd/libpa.so``.  No GPU is
needed: hipcc cross-compiles for gfx950.
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
LIB = os.path.join(PKG, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["pa_kernels.hip", "pa_api.cpp", "pa_sched.cpp", "pa_noalloc.hip"]

# Packed fp32 instructions are kept out of every kernel: hipcc must not
# generate v_pk_{add,mul,fma}_f32 from ordinary float code on this target.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def build(verbose: bool = False) -> str:
    """Compile libpa.so; return its path.  Always recompiles."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}", *DEVICE_FLAGS,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


PROBE_SOURCE = os.path.join(CSRC, "probe", "pa_probe.hip")
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile libpa_probe.so, the read-ceiling probe bench.py times beside
    the attention call (not part of libpa's ABI).  Always recompiles."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC", "-Wall",
           *DEVICE_FLAGS, PROBE_SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
