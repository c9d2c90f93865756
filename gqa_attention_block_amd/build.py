"""Build libgqa.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python gqa_attention_block_amd/build.py`` (runs without importing the
package, which would load the library being rebuilt) or ``build_library()``.
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
LIB_NAME = "libgqa.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["gqa_kernels.hip", "gqa_head.hip", "gqa_noalloc.hip", "gqa_host.cpp"]

# Packed fp32 (v_pk_*_f32) is switched off for all device code; the host
# pass warns that it does not know the feature, which is harmless.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core accumulators in ordinary VGPRs: the attention rescales its
    # accumulators with VALU multiplies, and with the AGPR form the compiler
    # copied all 64 of them between the two register files on every tile.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libgqa")
    return path


def build_library(verbose: bool = False, extra_flags=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
