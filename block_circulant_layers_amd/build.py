"""Build librdfft.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m block_circulant_layers_amd.build

Steps: generate csrc/twiddles.inc from float64 math, then one hipcc call.
Packed FP32 instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "librdfft.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = True) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    subprocess.run(
        [sys.executable, os.path.join(CSRC, "gen_twiddles.py"), os.path.join(CSRC, "twiddles.inc")], check=True
    )
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "rdfft_lib.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
