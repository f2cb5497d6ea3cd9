"""Build ``persistent_runtime_amd/liblf.so`` (gfx950) with hipcc, in-tree.

Every HIP source is compiled with packed-fp32 instructions disabled
(``-target-feature -packed-fp32-ops``): ordinary float code only.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblf.so")
TRACE_LIB = os.path.join(HERE, "liblf_trace.so")   # LF_TRACE build: per-phase timestamps of one token
SOURCES = [os.path.join(CSRC, "lf_api.cpp"), os.path.join(CSRC, "lf_kernel.hip")]
ARCH = os.environ.get("LF_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def command(out: str, trace: bool = False) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument"] + (["-DLF_TRACE"] if trace else []) + [
            "-I", os.path.join(ROOT, "include"), "-x", "hip"] + SOURCES + ["-o", out]


def build(verbose: bool = False, trace: bool = False) -> str:
    """Compile the library; with ``trace`` the LF_TRACE variant (liblf_trace.so),
    which a process loads instead with LF_LIB (see phase_trace.py)."""
    lib = TRACE_LIB if trace else LIB
    tmp = lib + ".tmp"
    cmd = command(tmp, trace)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, trace="--trace" in sys.argv[1:])
    sys.exit(0)
