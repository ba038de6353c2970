"""Build the HIP library in place: ``libultraep.so`` next to this file.

One hipcc invocation compiles every source under ``csrc/`` for gfx950.
Packed-fp32 instruction selection is switched off for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libultraep.so")
SOURCES = ["ultraep_kernels.hip", "ultraep_combine.hip", "ultraep_weights.hip", "ultraep_abi.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libultraep.so")


def command(out: str = LIB) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
