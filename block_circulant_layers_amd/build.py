"""Build librdfft.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m block_circulant_layers_amd.build

Steps: generate csrc/twiddles.inc from float64 math, then one hipcc call for
librdfft.so and one for libstreamprobe.so (the in-place streaming pass that
bench.py measures the transforms against).  Packed FP32 instructions are
disabled for all device code.

kernel_resources() reads back, from the built library's own gfx950 code
object, the register and scratch figures the compiler recorded for every
kernel (the AMDGPU code-object metadata note).
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "librdfft.so")
# the in-place streaming pass bench.py measures the transforms against
PROBE_LIB = os.path.join(LIBDIR, "libstreamprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LLVM_BIN = os.environ.get("RDFFT_LLVM_BIN", "/opt/rocm/llvm/bin")
OFFLOAD_TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

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
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, os.path.join(CSRC, "stream_probe.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_LIB)
    return LIB


def kernel_resources(lib: str = LIB) -> dict:
    """Per-kernel metadata of the gfx950 code object inside ``lib`` (a library
    built here): {mangled name: {"private_segment_fixed_size", "vgpr_count",
    "agpr_count", "sgpr_count", "vgpr_spill_count", "sgpr_spill_count",
    "group_segment_fixed_size", "uses_dynamic_stack"}}.  The code object is
    taken out of the library's offload bundle and its metadata note read as
    YAML."""
    import yaml

    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin.bin")
        co = os.path.join(tmp, "gfx950.co")
        subprocess.run([os.path.join(LLVM_BIN, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", lib,
                        os.path.join(tmp, "stripped.so")], check=True, capture_output=True)
        subprocess.run([os.path.join(LLVM_BIN, "clang-offload-bundler"), "--unbundle", "--type=o",
                        f"--targets={OFFLOAD_TARGET}", f"--input={fat}", f"--output={co}"],
                       check=True, capture_output=True)
        notes = subprocess.run([os.path.join(LLVM_BIN, "llvm-readelf"), "--notes", co], check=True,
                               capture_output=True, text=True).stdout
    start = notes.index("---")
    end = notes.index("\n...", start)
    meta = yaml.safe_load(notes[start:end])
    keys = ("private_segment_fixed_size", "vgpr_count", "agpr_count", "sgpr_count", "vgpr_spill_count",
            "sgpr_spill_count", "group_segment_fixed_size", "uses_dynamic_stack")
    out = {}
    for k in meta["amdhsa.kernels"]:
        out[k[".name"]] = {key: k.get("." + key) for key in keys}
    return out


if __name__ == "__main__":
    build()
