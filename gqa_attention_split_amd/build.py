"""Build the HIP library (gfx950) in-tree: gqa_attention_split_amd/libmga_gqa.so.

Usage: python -m gqa_attention_split_amd.build [--verbose] [--resource-usage]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libmga_gqa.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = [os.path.join(CSRC, "gqa_kernels.hip"), os.path.join(CSRC, "mga_api.cpp"),
           os.path.join(CSRC, "mga_device.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU forms are turned off for every device compile.
# MFMA results go to VGPRs (the scores feed VALU exp directly, no AGPR reads).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form", "-Wall"]


def build(verbose: bool = False, resource_usage: bool = False, extra=None) -> str:
    cmd = [HIPCC, *DEVICE_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"),
           "-o", LIB_PATH + ".tmp", *SOURCES]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if extra:
        cmd[1:1] = list(extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv, resource_usage="--resource-usage" in sys.argv)
