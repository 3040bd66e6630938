"""The C-ABI library loads, exports every symbol include/moe_gate.h declares, and
rejects bad arguments on the host before enqueuing anything (no GPU needed)."""
import ctypes
import os
import re

import pytest
import torch

import combine_moe_gate_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_gate.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        from combine_moe_gate_amd import _build
        _build.build()
    return M.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), f"{name} declared but not exported"
    assert set(names) == set(M.EXPORTS)


def test_abi_version_and_status_names(lib):
    header = open(os.path.join(os.path.dirname(__file__), "..", "include", "moe_gate.h")).read()
    declared = int(re.search(r"#define MOE_ABI_VERSION (\d+)", header).group(1))
    assert lib.moe_abi_version() == declared == M.ABI_VERSION == 6
    for code, name in M.STATUS_NAMES.items():
        assert lib.moe_status_string(code).decode() == name
    assert lib.moe_status_string(99).decode() == "MOE_STATUS_UNKNOWN"


def test_layout_struct_matches_header_size():
    # magic, 6 ints, rows, 10 pointers, size_t
    assert ctypes.sizeof(M.LayoutStruct) == 8 + 24 + 8 + 10 * 8 + 8
    assert ctypes.sizeof(M.LayoutOptions) == 8


def test_workspace_bytes(lib):
    wb = M.workspace_bytes
    for args in [(256, 8, 2, 80), (8192, 128, 8, 0), (16384, 64, 4, 1024), (0, 4, 2, 3), (1, 1, 1, 0)]:
        n = wb(*args)
        assert n > 0 and n % 256 == 0
    s, e, k = 8192, 128, 8
    assert wb(s, e, k, 0) >= 4 * (2 * s * k + s * k)  # dst + route copy + src
    assert wb(2 * s, e, k, 0) > wb(s, e, k, 0)
    # invalid or unsupported sizes give 0
    assert wb(-1, 8, 2, 0) == 0
    assert wb(10, 8, 9, 0) == 0
    assert wb(10, 2000, 2, 0) == 0
    assert wb(10, 64, 17, 0) == 0
    assert wb(2**30, 128, 8, 0) == 0  # s*k over 2**31
    # options: route-major tiles cover s*k items, padding adds e*(P-1) rows
    assert wb(1000, 64, 4, 0, route_major=True) > wb(1000, 64, 4, 0)
    assert wb(1000, 64, 4, 0, pad_multiple=128) >= wb(1000, 64, 4, 0) + 4 * 64 * 127
    assert wb(1000, 64, 4, 10, pad_multiple=2) == 0  # padding is dropless-only
    assert wb(1000, 64, 4, 0, pad_multiple=0) == 0


# The calls below carry fake device addresses that must be rejected before any
# kernel is enqueued. On a machine with a GPU they are skipped, so that a bug in the
# checks could never launch a kernel on a fake address.
no_gpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                 reason="fake-pointer validation tests run only without a GPU")

FAKE = ctypes.c_void_p(1 << 20)


@no_gpu_only
def test_gate_argument_checks(lib):
    out = ctypes.c_void_p(1 << 21)
    assert lib.moe_gate_topk(FAKE, 4, 8, 9, out, out, None) == 1  # k > e
    assert "k must be in" in lib.moe_last_error().decode()
    assert lib.moe_gate_topk(FAKE, 4, 2048, 2, out, out, None) == 2  # e too large
    assert lib.moe_gate_topk(FAKE, 4, 64, 17, out, out, None) == 2  # k too large
    assert lib.moe_gate_topk(None, 4, 8, 2, out, out, None) == 1  # NULL logits
    assert lib.moe_gate_topk(FAKE, -1, 8, 2, out, out, None) == 1
    assert lib.moe_gate_topk_backward(FAKE, FAKE, None, 4, 8, 2, out, None) == 1


@no_gpu_only
def test_layout_argument_checks(lib):
    st = M.LayoutStruct()
    need = M.workspace_bytes(100, 8, 2, 0)
    assert lib.moe_dispatch_layout(FAKE, 100, 8, 2, 0, FAKE, need - 1, ctypes.byref(st), None) == 3
    assert "workspace" in lib.moe_last_error().decode()
    assert lib.moe_dispatch_layout(FAKE, 100, 8, 2, 0, ctypes.c_void_p((1 << 20) + 8), need,
                                   ctypes.byref(st), None) == 5
    assert lib.moe_dispatch_layout(FAKE, 100, 8, 2, 0, None, need, ctypes.byref(st), None) == 1
    assert lib.moe_dispatch_layout(FAKE, 100, 8, 2, 0, FAKE, need, None, None) == 1
    assert lib.moe_dispatch_layout(None, 100, 8, 2, 0, FAKE, need, ctypes.byref(st), None) == 1
    assert st.magic == 0  # nothing was filled
    bad = M.LayoutOptions(0, 4)
    assert lib.moe_dispatch_layout_ex(FAKE, 100, 8, 2, 5, ctypes.byref(bad), FAKE, need,
                                      ctypes.byref(st), None) == 1  # padding with a capacity
    bad = M.LayoutOptions(2, 1)
    assert lib.moe_dispatch_layout_ex(FAKE, 100, 8, 2, 0, ctypes.byref(bad), FAKE, need,
                                      ctypes.byref(st), None) == 1
    assert st.magic == 0


@no_gpu_only
def test_static_scratch_layout_argument_checks(lib):
    """The layout that keeps its tile tables in the library's static array needs only the
    handle's share of a workspace, and refuses sizes whose tables exceed the array, both
    before touching the device."""
    st = M.LayoutStruct()

    def handle_bytes(s, e, k, rows):
        a = lambda n: (n + 255) // 256 * 256
        return 2 * a(4 * e) + a(4 * (e + 1)) + 2 * a(4 * s * k) + a(4 * rows) + a(8) + a(4)

    need = handle_bytes(100, 8, 2, 200)
    assert need < M.workspace_bytes(100, 8, 2, 0)
    f = lib.moe_dispatch_layout_static_scratch
    assert f(FAKE, 100, 8, 2, 0, None, FAKE, need - 1, ctypes.byref(st), None) == 3
    assert "workspace" in lib.moe_last_error().decode()
    assert f(FAKE, 200000, 1024, 1, 0, None, FAKE, 1 << 30, ctypes.byref(st), None) == 2
    assert "static scratch" in lib.moe_last_error().decode()
    assert f(FAKE, 100, 8, 9, 0, None, FAKE, need, ctypes.byref(st), None) == 1  # k > e
    assert f(FAKE, 100, 8, 2, 0, None, None, need, ctypes.byref(st), None) == 1
    assert st.magic == 0


@no_gpu_only
def test_row_calls_reject_foreign_or_bad_handles(lib):
    st = M.LayoutStruct()  # never filled by moe_dispatch_layout
    out = ctypes.c_void_p(1 << 21)
    assert lib.moe_dispatch(ctypes.byref(st), FAKE, 64, 1, out, None) == 4
    assert lib.moe_combine(ctypes.byref(st), FAKE, FAKE, 64, 1, out, None) == 4
    assert lib.moe_combine_backward(ctypes.byref(st), FAKE, FAKE, FAKE, 64, 1, out, out, None) == 4
    assert lib.moe_dispatch_backward(ctypes.byref(st), FAKE, 64, 1, out, None) == 4
    assert lib.moe_dispatch_replay(ctypes.byref(st), None, FAKE, 64, 1, out, None) == 4
    assert lib.moe_layout_read(ctypes.byref(st), None, None, None) == 4
    assert lib.moe_dispatch(None, FAKE, 64, 1, out, None) == 1


@no_gpu_only
def test_row_calls_check_alignment_and_dtype(lib):
    # a handle that looks valid to the host checks, over a fake workspace
    s, e, k = 40, 8, 2
    ws = 1 << 24
    need = M.workspace_bytes(s, e, k, 0)
    st = _fake_handle(s, e, k, 0, ws, need)
    out = ctypes.c_void_p(1 << 22)
    assert lib.moe_dispatch(ctypes.byref(st), FAKE, 3, 1, out, None) == 5  # 6-byte rows
    assert lib.moe_dispatch(ctypes.byref(st), ctypes.c_void_p((1 << 20) + 4), 64, 1, out, None) == 5
    assert lib.moe_dispatch(ctypes.byref(st), FAKE, 64, 7, out, None) == 1  # unknown dtype
    assert lib.moe_dispatch(ctypes.byref(st), FAKE, 0, 1, out, None) == 1  # m = 0
    assert lib.moe_dispatch_weighted(ctypes.byref(st), FAKE, None, 64, 1, out, None) == 1  # NULL weights
    assert lib.moe_renormalize_kept(ctypes.byref(st), FAKE, FAKE, None) == 1  # in place
    assert lib.moe_dispatch_weighted_backward(ctypes.byref(st), FAKE, FAKE, FAKE, 64, 1, out, None, None) == 1
    st.rows = st.rows + 1
    assert lib.moe_dispatch(ctypes.byref(st), FAKE, 64, 1, out, None) == 4


@no_gpu_only
def test_expert_gemm_argument_checks(lib):
    s, e, k = 40, 8, 2
    ws = 1 << 24
    st = _fake_handle(s, e, k, 0, ws, M.workspace_bytes(s, e, k, 0))
    h = ctypes.byref(st)
    a, w, out = FAKE, ctypes.c_void_p(1 << 26), ctypes.c_void_p(1 << 28)
    assert lib.moe_expert_gemm(h, a, 1, w, 64, 64, 0, None, out, None) == 2  # float32: no MFMA path
    assert "bf16 and f16" in lib.moe_last_error().decode()
    assert lib.moe_expert_gemm(h, a, 2, w, 64, 64, 1, None, out, None) == 1  # gather must be 0/1
    assert lib.moe_expert_gemm(h, a, 1, w, 12, 64, 1, None, out, None) == 5  # 24-byte input rows
    assert lib.moe_expert_gemm(h, a, 1, w, 64, 4, 1, None, out, None) == 5  # 8-byte output rows
    assert lib.moe_expert_gemm(h, a, 1, None, 64, 64, 1, None, out, None) == 1  # NULL weights
    assert lib.moe_expert_gemm(h, a, 1, ctypes.c_void_p((1 << 26) + 8), 64, 64, 1, None, out, None) == 5
    assert lib.moe_expert_gemm(h, a, 1, w, 64, 64, 1, None, None, None) == 1  # NULL out
    # a and out overlapping (out starts inside x's 40 rows of 128 bytes)
    assert lib.moe_expert_gemm(h, a, 1, w, 64, 64, 1, None, ctypes.c_void_p((1 << 20) + 1024), None) == 1
    assert "overlap" in lib.moe_last_error().decode()
    st2 = M.LayoutStruct()  # never filled by moe_dispatch_layout
    assert lib.moe_expert_gemm(ctypes.byref(st2), a, 1, w, 64, 64, 1, None, out, None) == 4


@no_gpu_only
def test_binding_refuses_a_library_of_another_abi_version(monkeypatch):
    """A library built for other signatures is refused at load, before any call."""
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "ABI_VERSION", M.ABI_VERSION + 1)
    with pytest.raises(RuntimeError, match="ABI version"):
        M.lib()


@no_gpu_only
def test_expert_gemm_gradient_argument_checks(lib):
    s, e, k = 40, 8, 2
    ws = 1 << 24
    st = _fake_handle(s, e, k, 0, ws, M.workspace_bytes(s, e, k, 0))
    h = ctypes.byref(st)
    a, g, w, out = FAKE, ctypes.c_void_p(1 << 26), ctypes.c_void_p(1 << 27), ctypes.c_void_p(1 << 28)
    # weight gradient
    assert lib.moe_expert_gemm_wgrad(h, a, 1, g, 64, 64, 0, 0, out, None) == 2  # float32 operands
    assert lib.moe_expert_gemm_wgrad(h, a, 1, g, 64, 64, 1, 2, out, None) == 2  # f16 grad_w of bf16
    assert lib.moe_expert_gemm_wgrad(h, a, 3, g, 64, 64, 1, 0, out, None) == 1  # gather flag
    assert lib.moe_expert_gemm_wgrad(h, a, 1, g, 12, 64, 1, 0, out, None) == 5  # 24-byte rows
    assert lib.moe_expert_gemm_wgrad(h, a, 1, None, 64, 64, 1, 0, out, None) == 1  # NULL grad_out
    assert lib.moe_expert_gemm_wgrad(h, a, 1, g, 64, 64, 1, 0, None, None) == 1  # NULL grad_w
    assert lib.moe_expert_gemm_wgrad(h, a, 1, g, 64, 64, 1, 0, ctypes.c_void_p((1 << 28) + 4), None) == 5
    assert lib.moe_expert_gemm_wgrad(h, a, 1, g, 64, 64, 1, 0, ctypes.c_void_p((1 << 26) + 256), None) == 1
    assert "overlap" in lib.moe_last_error().decode()
    # input-row gradient
    assert lib.moe_expert_gemm_dgrad(h, g, w, 64, 64, 0, out, None) == 2
    assert lib.moe_expert_gemm_dgrad(h, g, w, 64, 4, 1, out, None) == 5  # 8-byte grad_out rows
    assert lib.moe_expert_gemm_dgrad(h, g, None, 64, 64, 1, out, None) == 1
    assert lib.moe_expert_gemm_dgrad(h, g, w, 64, 64, 1, ctypes.c_void_p((1 << 26) + 512), None) == 1
    assert "overlap" in lib.moe_last_error().decode()
    st2 = M.LayoutStruct()
    assert lib.moe_expert_gemm_dgrad(ctypes.byref(st2), g, w, 64, 64, 1, out, None) == 4
    assert lib.moe_expert_gemm_wgrad(ctypes.byref(st2), a, 1, g, 64, 64, 1, 0, out, None) == 4


def _fake_handle(s, e, k, capacity, ws, need):
    """Reproduce what moe_dispatch_layout fills in, without running it (256-byte carving)."""
    def take(cur, n):
        cur = (cur + 255) // 256 * 256
        return cur, cur + n
    rows = e * capacity if capacity > 0 else s * k
    ntiles = (s + 255) // 256
    cur = 0
    offs = {}
    for name, n in [("counts", 4 * e), ("kept", 4 * e), ("offsets", 4 * (e + 1)), ("dst", 4 * s * k),
                    ("src", 4 * rows), ("route_idx", 4 * s * k), ("checksum", 8), ("flags", 4),
                    ("scratch", 4 * ntiles * e)]:
        at, cur = take(cur, n)
        offs[name] = at
    st = M.LayoutStruct()
    st.magic = 0x4D4F454C41594F54
    st.s, st.e, st.k, st.capacity, st.rows = s, e, k, capacity, rows
    st.route_major, st.pad_multiple = 0, 1
    for name, at in offs.items():
        setattr(st, name, ws + at)
    st.workspace = ws
    st.workspace_bytes = need
    return st


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(4, 8)
    with pytest.raises((ValueError, RuntimeError)):
        M.moe_gate_topk(x, 2)


# ----------------------------------------------------------------------------
# the binding checks tensors against the layout before any pointer reaches the library
# (the C ABI gets bare pointers and could not tell a short or mistyped buffer)


def fake_layout(s=6, e=4, k=2, rows=12):
    st = M.LayoutStruct()
    st.s, st.e, st.k, st.rows = s, e, k, rows
    return M.Layout(st, torch.empty(0, dtype=torch.uint8))


@pytest.fixture
def no_library(monkeypatch):
    def refuse():
        raise AssertionError("the library was called with arguments the binding should have refused")
    monkeypatch.setattr(M, "lib", refuse)


BAD_CALLS = [
    # (call, message fragment): shapes against the layout s=6, e=4, k=2, rows=12, m=8
    (lambda L: M.moe_dispatch(L, torch.zeros(5, 8)), "x must have shape [6, *]"),
    (lambda L: M.moe_dispatch(L, torch.zeros(6, 8, dtype=torch.int32)), "x must be"),
    (lambda L: M.moe_dispatch(L, torch.zeros(6, 8), out=torch.zeros(11, 8)), "out must have shape [12, 8]"),
    (lambda L: M.moe_dispatch(L, torch.zeros(6, 8), out=torch.zeros(12, 8, dtype=torch.float16)), "out must be"),
    (lambda L: M.moe_dispatch_replay(L, torch.zeros(6, 8), torch.zeros(6, 3, dtype=torch.int32)), "idx must have"),
    (lambda L: M.moe_dispatch_replay(L, torch.zeros(6, 8), torch.zeros(6, 2, dtype=torch.int64)), "idx must be"),
    (lambda L: M.moe_combine(L, torch.zeros(11, 8), torch.zeros(6, 2)), "expert_out must have shape [12, *]"),
    (lambda L: M.moe_combine(L, torch.zeros(12, 8), torch.zeros(6, 2, dtype=torch.bfloat16)), "w must be"),
    (lambda L: M.moe_combine(L, torch.zeros(12, 8), torch.zeros(5, 2)), "w must have shape [6, 2]"),
    (lambda L: M.moe_combine(L, torch.zeros(12, 8), None, out=torch.zeros(6, 4)), "out must have shape [6, 8]"),
    (lambda L: M.moe_combine_backward(L, torch.zeros(6, 8), torch.zeros(12, 8), None), "w is required"),
    (lambda L: M.moe_combine_backward(L, torch.zeros(6, 8), torch.zeros(12, 4), torch.zeros(6, 2)),
     "expert_out must have shape [12, 8]"),
    (lambda L: M.moe_combine_backward(L, torch.zeros(6, 8), torch.zeros(12, 8, dtype=torch.float16),
                                      torch.zeros(6, 2)), "expert_out must be"),
    (lambda L: M.moe_combine_backward(L, torch.zeros(6, 8), torch.zeros(12, 8), torch.zeros(6, 2),
                                      grad_w=torch.zeros(6, 2, dtype=torch.float64)), "grad_w must be"),
    (lambda L: M.moe_dispatch_backward(L, torch.zeros(6, 8)), "grad_out must have shape [12, *]"),
    (lambda L: M.moe_dispatch_weighted(L, torch.zeros(6, 8), torch.zeros(6, 1)), "w must have shape [6, 2]"),
    (lambda L: M.moe_dispatch_weighted_backward(L, torch.zeros(12, 8), torch.zeros(6, 8), torch.zeros(6, 2),
                                                grad_x=torch.zeros(6, 9)), "grad_x must have shape [6, 8]"),
    (lambda L: M.moe_renormalize_kept(L, torch.zeros(6, 3)), "w must have shape [6, 2]"),
    (lambda L: M.moe_renormalize_kept_backward(L, torch.zeros(6, 2), torch.zeros(6, 2, dtype=torch.float16)),
     "grad_out must be"),
    (lambda L: M.moe_expert_gemm(L, torch.zeros(12, 8, dtype=torch.bfloat16),
                                 torch.zeros(4, 16, 8, dtype=torch.bfloat16)), "a must have shape [6, *]"),
    (lambda L: M.moe_expert_gemm(L, torch.zeros(6, 8, dtype=torch.bfloat16),
                                 torch.zeros(3, 16, 8, dtype=torch.bfloat16)), "weights must have shape [4, *, 8]"),
    (lambda L: M.moe_expert_gemm(L, torch.zeros(6, 8, dtype=torch.bfloat16),
                                 torch.zeros(4, 16, 8, dtype=torch.float16)), "weights must be"),
    (lambda L: M.moe_expert_gemm_wgrad(L, torch.zeros(6, 8, dtype=torch.bfloat16),
                                       torch.zeros(12, 16, dtype=torch.bfloat16), out=torch.zeros(4, 16, 9)),
     "out must have shape [4, 16, 8]"),
    (lambda L: M.moe_expert_gemm_dgrad(L, torch.zeros(12, 16, dtype=torch.bfloat16),
                                       torch.zeros(4, 15, 8, dtype=torch.bfloat16)), "weights must have shape [4, 16, *]"),
]


@pytest.mark.parametrize("case", range(len(BAD_CALLS)))
def test_binding_refuses_mismatched_tensors_before_the_library(case, no_library):
    call, fragment = BAD_CALLS[case]
    with pytest.raises(ValueError) as err:
        call(fake_layout())
    assert fragment in str(err.value)


def test_binding_refuses_wrong_gate_and_layout_arguments(no_library):
    with pytest.raises(ValueError, match="logits must be"):
        M.moe_gate_topk(torch.zeros(4, 8, dtype=torch.float16), 2)
    with pytest.raises(ValueError, match=r"idx_out must have shape \[4, 2\]"):
        M.moe_gate_topk(torch.zeros(4, 8), 2, idx_out=torch.zeros(4, 3, dtype=torch.int32))
    with pytest.raises(ValueError, match="grad_w must be"):
        M.moe_gate_topk_backward(torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2),
                                 torch.zeros(4, 2, dtype=torch.float64), 8)
    with pytest.raises(ValueError, match="expert ids must be"):
        M.moe_dispatch_layout(torch.zeros(4, 2, dtype=torch.int64), 8)
    with pytest.raises(ValueError, match="workspace must be"):
        M.moe_dispatch_layout(torch.zeros(4, 2, dtype=torch.int32), 8, workspace=torch.zeros(64))


def test_binding_refuses_well_shaped_cpu_tensors(no_library):
    """Right shapes and types on the host still stop before the library: no CPU path."""
    with pytest.raises(ValueError, match="on the GPU"):
        M.moe_dispatch(fake_layout(), torch.zeros(6, 8))
    with pytest.raises(ValueError, match="on the GPU"):
        M.moe_combine(fake_layout(), torch.zeros(12, 8), torch.zeros(6, 2))
