"""Host builds of the library for the CPU checks (test infrastructure).

run_abi.cpp includes rdfft_lib.hip, so one host compile carries the C ABI,
its dispatch logic and every kernel template, against the CPU stand-in of
hip/hip_runtime.h in this folder.  Three builds:
  tsan  ThreadSanitizer: the LDS schedule checker (one host thread per GPU
        thread, barriers as pthread barriers; see hip/hip_runtime.h);
  asan  AddressSanitizer + UndefinedBehaviorSanitizer on the host code: the
        argument checks and launch arithmetic;
  bank  bank_model.cpp: the LDS bank model of the exchange layouts.
A build is redone when any source is newer than its executable.
"""

from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "block_circulant_layers_amd", "csrc")
BUILD = os.path.join(HERE, "_build")
CXX = os.environ.get("RDFFT_HOST_CXX", "/opt/rocm/llvm/bin/clang++")

FLAGS = {
    "tsan": ["-O1", "-g", "-fsanitize=thread"],
    # -O0: the optimised sanitizer build of every kernel template takes minutes
    "asan": ["-O0", "-g1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
    "bank": ["-O1"],
}
MAIN = {"tsan": "run_abi.cpp", "asan": "run_abi.cpp", "bank": "bank_model.cpp"}


def sources():
    return ([os.path.join(HERE, "run_abi.cpp"), os.path.join(HERE, "bank_model.cpp"), os.path.join(HERE, "hip", "hip_runtime.h"),
             os.path.join(ROOT, "include", "rdfft.h")]
            + glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(CSRC, "*.hip"))
            + [os.path.join(CSRC, "twiddles.inc")])


def build(kind: str) -> str:
    exe = os.path.join(BUILD, f"run_abi_{kind}" if kind != "bank" else "bank_model")
    twiddles = os.path.join(CSRC, "twiddles.inc")
    if not os.path.exists(twiddles):
        subprocess.run(["python3", os.path.join(CSRC, "gen_twiddles.py"), twiddles], check=True)
    if os.path.exists(exe) and os.path.getmtime(exe) >= max(os.path.getmtime(s) for s in sources()):
        return exe
    os.makedirs(BUILD, exist_ok=True)
    tmp = exe + ".tmp"
    cmd = [CXX, "-std=c++20", *FLAGS[kind], "-Wno-pass-failed", "-Wno-unused-command-line-argument",
           "-I", HERE, "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(HERE, MAIN[kind]),
           "-o", tmp, "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, exe)
    return exe
