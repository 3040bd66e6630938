"""Build the gfx950 shared library libmoe_gate.so in-tree with hipcc.

    python -m combine_moe_gate_amd._build

hipcc cross-compiles for gfx950 without a GPU present. The same build compiles
tests/c_abi_check, a C++ program that drives the library through its C ABI alone.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmoe_gate.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("api.hip", "gate.hip", "layout.hip", "rows.hip", "gemm.hip", "gemm_bwd.hip")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("internal.h", "moe_device.h", "gemm_common.h")] + [
    os.path.join(ROOT, "include", "moe_gate.h")]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # products and sums are rounded separately, as the combine definition states
    "-ffp-contract=off",
    # keep float32 subnormals (the host reference keeps them)
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 arithmetic (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmoe_gate.so")
    return path


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi_check.cpp")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c_abi_check")


def build_c_check(verbose: bool = False) -> str:
    """Compile the C++ program that drives the library through its C ABI alone (a GPU
    test runs it). It links LIB_PATH, found next to the binary through its run path."""
    cmd = [hipcc(), "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), C_CHECK_SRC,
           "-L", HERE, "-lmoe_gate", "-Wl,-rpath,$ORIGIN/../combine_moe_gate_amd", "-o", C_CHECK_BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    return C_CHECK_BIN


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles). Returns the path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    build_c_check(verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
