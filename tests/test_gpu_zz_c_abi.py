"""The library driven from C++ through its C ABI alone (tests/c_abi_check.cpp): hipMalloc'd
buffers, one HIP stream, no Python or PyTorch in the process. The program calls every
entry point (gate, layout and its options, dispatch, replay, combine, the backward passes,
the variants, the grouped expert GEMM and its gradients), checks the results against
properties and closed forms (see its header), plus the host-side argument checks, and exits
0 when all hold.
It is compiled with the library by the package build."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_program_through_the_abi():
    assert os.path.exists(BIN), f"{BIN} is missing: build first (python -m combine_moe_gate_amd._build)"
    print("CASE c_abi_check", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=100)
    print(res.stdout[-2000:], flush=True)
    assert res.returncode == 0, f"exit {res.returncode}\n{res.stdout[-2000:]}\n{res.stderr[-4000:]}"
    assert "c_abi_check: ok" in res.stdout
