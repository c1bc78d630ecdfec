"""Compile the HIP sources of this package into ``libttt_mem.so`` for gfx950.

Usage: ``python -m test_neural_memory_amd.build`` (or ``build()`` from Python).
The library is written next to this file so that it travels with the source
tree; nothing is installed anywhere else.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", name) for name in ("ttt_mem_linear.hip", "ttt_mem_deep.hip", "ttt_mem_decode.hip", "ttt_mem_linear_bwd.hip")]
LIB = os.path.join(PKG, "libttt_mem.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Keep packed-FP32 VALU instructions out of the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libttt_mem.so")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libttt_mem.so``; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
