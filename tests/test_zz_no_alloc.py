"""The layout entry point that allocates nothing, through the C ABI.

moe_dispatch_layout_static_scratch keeps the layout's tile tables in a static device
array of the library instead of the caller's workspace, which then holds only the
handle's arrays. Its handle must equal moe_dispatch_layout_ex's bit for bit (counts,
kept, offsets, dst, src, routing copy, checksum, flags) and serve every later call
alike, on consecutive calls of decreasing size (the array keeps the last call's
contents, which no later call may depend on).
"""
import ctypes

import numpy as np
import pytest
import torch

import combine_moe_gate_amd as M
import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def align(n):
    return (n + 255) // 256 * 256


def handle_bytes(s, e, k, rows):
    """The handle's share of a layout workspace, as the header states it."""
    return (2 * align(4 * e) + align(4 * (e + 1)) + 2 * align(4 * s * k) + align(4 * rows)
            + align(8) + align(4))


def static_layout(idx, e, cap, route_major=False, pad=1, ws_bytes=None):
    s, k = idx.shape
    rows = e * cap if cap > 0 else s * k + e * (pad - 1)
    need = handle_bytes(s, e, k, rows)
    ws = torch.empty(need if ws_bytes is None else ws_bytes, dtype=torch.uint8, device="cuda")
    st = M.LayoutStruct()
    opts = M.LayoutOptions(int(route_major), pad)
    status = M.lib().moe_dispatch_layout_static_scratch(
        ctypes.c_void_p(idx.data_ptr()), s, e, k, cap, ctypes.byref(opts), ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), ctypes.byref(st), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return status, M.Layout(st, ws)


def assert_same_layout(Ls, Lr, what):
    assert Ls.rows == Lr.rows, what
    for f in ("counts", "kept", "offsets", "dst", "src", "route_idx"):
        assert torch.equal(getattr(Ls, f), getattr(Lr, f)), f"{what}: {f}"
    assert M.moe_layout_read(Ls) == M.moe_layout_read(Lr), f"{what}: flags / checksum"


def routing(name=None, s=None, e=None, k=None, seed=0):
    if name is not None:
        inp = W.make_inputs(name)
        return torch.from_numpy(oracle.gate_topk(inp.logits, inp.workload.k)[0]).cuda()
    rng = np.random.default_rng(seed)
    return torch.from_numpy(W.random_idx(rng, s, e, k)).cuda()


# consecutive calls, each smaller than the one before: more than 256 tiles (the tile table
# scanned by its own launch), many tiles with the Zipf routing, fewer tiles with a capacity
# drop, route-major priority, padded segments, and one tile (where the build uses no
# tables at all)
CALLS = [
    ("s=70000 e=64 k=2 dropless, 274 tiles", dict(s=70000, e=64, k=2, seed=6), 64, 0, False, 1),
    ("zipf_skew_h4096 routing, dropless", dict(name="zipf_skew_h4096"), 128, 0, False, 1),
    ("s=3000 e=64 k=4 capacity 150", dict(s=3000, e=64, k=4, seed=1), 64, 150, False, 1),
    ("s=900 e=32 k=2 capacity 40 route-major", dict(s=900, e=32, k=2, seed=2), 32, 40, True, 1),
    ("s=700 e=40 k=3 pad 8", dict(s=700, e=40, k=3, seed=3), 40, 0, False, 8),
    ("s=100 e=8 k=2 one tile", dict(s=100, e=8, k=2, seed=4), 8, 0, False, 1),
]


def test_static_scratch_layout_equals_the_workspace_layout_on_consecutive_calls():
    for what, spec, e, cap, rm, pad in CALLS:
        print("CASE static scratch", what, flush=True)
        idx = routing(**spec)
        status, Ls = static_layout(idx, e, cap, rm, pad)
        assert status == M.MOE_OK, (what, M.lib().moe_last_error().decode())
        Lr = M.moe_dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
        assert_same_layout(Ls, Lr, what)
        # the handle serves the row calls like any other
        m = 64
        x = torch.randn((idx.shape[0], m), device="cuda").to(torch.bfloat16)
        assert torch.equal(M.moe_dispatch(Ls, x).view(torch.int16), M.moe_dispatch(Lr, x).view(torch.int16)), what
        torch.cuda.synchronize()


def test_static_scratch_layout_refuses_what_does_not_fit():
    print("CASE static scratch refusals", flush=True)
    idx = routing(s=1000, e=16, k=2, seed=5)
    need = handle_bytes(1000, 16, 2, 2000)
    status, L = static_layout(idx, 16, 0, ws_bytes=need - 1)
    assert status == 3 and L.struct.magic == 0  # MOE_ERR_WORKSPACE, nothing filled
    # tile tables beyond the static array: 1024 experts x 784 tiles x 4 bytes > 2 MiB
    big = torch.zeros((200000, 1), dtype=torch.int32, device="cuda")
    status, L = static_layout(big, 1024, 0)
    assert status == 2 and L.struct.magic == 0  # MOE_ERR_UNSUPPORTED
    assert "static scratch" in M.lib().moe_last_error().decode()
    torch.cuda.synchronize()
