"""MI355X-native MoE gate / dispatch / combine: thin Python binding over libmoe_gate.so.

Every step of the path runs in the library's HIP kernels; this module only
marshals arguments. PyTorch provides device memory and the current stream. The
function names are those of the C ABI in include/moe_gate.h:

    idx, w  = moe_gate_topk(logits, k)
    layout  = moe_dispatch_layout(idx, e, capacity)        # capacity <= 0: dropless
    buf     = moe_dispatch(layout, x)                      # [layout.rows, m]
    buf     = moe_dispatch_replay(layout, x, idx=None)     # recompute from a saved layout
    y       = moe_combine(layout, buf_or_expert_out, w)    # [s, m]
    gE, gw  = moe_combine_backward(layout, grad_y, expert_out, w)
    gx      = moe_dispatch_backward(layout, grad_out)
    gl      = moe_gate_topk_backward(idx, w, gw, e)
    flags, checksum = moe_layout_read(layout)              # synchronises; tests/debug

There is no CPU fallback: without the built library, or without a GPU, every
call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gate.so")

MOE_OK = 0
STATUS_NAMES = {
    0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
    4: "MOE_ERR_HANDLE_MISMATCH", 5: "MOE_ERR_MISALIGNED", 6: "MOE_ERR_HIP",
}
MOE_F32, MOE_BF16, MOE_F16 = 0, 1, 2
FLAG_EXPERT_OUT_OF_RANGE = 1
FLAG_DUPLICATE_EXPERT = 2
FLAG_REPLAY_MISMATCH = 4
MAX_EXPERTS = 1024
MAX_TOPK = 16

_DTYPE_CODE = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.float16: MOE_F16}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class LayoutStruct(ctypes.Structure):
    """Mirror of moe_layout_t."""
    _fields_ = [
        ("magic", ctypes.c_uint64),
        ("s", ctypes.c_int32), ("e", ctypes.c_int32), ("k", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("route_major", ctypes.c_int32), ("pad_multiple", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("counts", ctypes.c_void_p), ("kept", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
        ("dst", ctypes.c_void_p), ("src", ctypes.c_void_p), ("route_idx", ctypes.c_void_p),
        ("checksum", ctypes.c_void_p), ("flags", ctypes.c_void_p), ("scratch", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class LayoutOptions(ctypes.Structure):
    """Mirror of moe_layout_options_t."""
    _fields_ = [("route_major", ctypes.c_int32), ("pad_multiple", ctypes.c_int32)]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGNATURES = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_layout_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "moe_layout_workspace_bytes_ex": (ctypes.c_size_t, [_I, _I, _I, _I, ctypes.POINTER(LayoutOptions)]),
    "moe_dispatch_layout_ex": (ctypes.c_int, [_P, _I, _I, _I, _I, ctypes.POINTER(LayoutOptions), _P,
                                              ctypes.c_size_t, ctypes.POINTER(LayoutStruct), _P]),
    "moe_dispatch_weighted": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _I, ctypes.c_int, _P, _P]),
    "moe_dispatch_weighted_backward": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _P, _I,
                                                      ctypes.c_int, _P, _P, _P]),
    "moe_expert_gemm": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _I, _P, _I, _I, ctypes.c_int,
                                       _P, _P, _P]),
    "moe_expert_gemm_wgrad": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _I, _P, _I, _I,
                                             ctypes.c_int, ctypes.c_int, _P, _P]),
    "moe_expert_gemm_dgrad": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _I, _I, ctypes.c_int,
                                             _P, _P]),
    "moe_renormalize_kept": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _P]),
    "moe_renormalize_kept_backward": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _P, _P]),
    "moe_gate_topk": (ctypes.c_int, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_gate_topk_backward": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_dispatch_layout": (ctypes.c_int, [_P, _I, _I, _I, _I, _P, ctypes.c_size_t,
                                           ctypes.POINTER(LayoutStruct), _P]),
    "moe_dispatch": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _I, ctypes.c_int, _P, _P]),
    "moe_dispatch_replay": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _I, ctypes.c_int,
                                           _P, _P]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _I, ctypes.c_int, _P, _P]),
    "moe_combine_backward": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _P, _I,
                                            ctypes.c_int, _P, _P, _P]),
    "moe_dispatch_backward": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _I, ctypes.c_int,
                                             _P, _P]),
    "moe_layout_read": (ctypes.c_int, [ctypes.POINTER(LayoutStruct), _P, _P, _P]),
    "moe_dispatch_layout_static_scratch": (ctypes.c_int, [_P, _I, _I, _I, _I, ctypes.POINTER(LayoutOptions), _P,
                                                          ctypes.c_size_t, ctypes.POINTER(LayoutStruct), _P]),
}
EXPORTS = tuple(_SIGNATURES)


ABI_VERSION = 6  # MOE_ABI_VERSION of include/moe_gate.h that _SIGNATURES follows


def lib() -> ctypes.CDLL:
    """Load libmoe_gate.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m combine_moe_gate_amd._build)")
        handle = ctypes.CDLL(LIB_PATH)
        handle.moe_abi_version.restype = ctypes.c_int
        handle.moe_abi_version.argtypes = []
        built = handle.moe_abi_version()
        if built != ABI_VERSION:  # the signatures below would not match the library's
            raise RuntimeError(f"{LIB_PATH} implements ABI version {built}, this binding expects "
                               f"{ABI_VERSION}: rebuild it (python -m combine_moe_gate_amd._build)")
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


if hasattr(torch._C, "_cuda_getCurrentRawStream"):
    def _stream(t: torch.Tensor):
        """The current HIP stream of t's device, as the library takes it (void*)."""
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(t.get_device()))
else:  # older torch: the public (slower) route
    def _stream(t: torch.Tensor):
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require_gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU (no CPU fallback exists)")
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _expect(t, name: str, shape, dtype=None):
    """Check a tensor argument before any pointer reaches the library: its shape (None
    matches any size in that place) and element type (one, or a tuple of allowed ones).
    The C ABI receives bare pointers and cannot tell a short or mistyped buffer from a
    right one."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    got = t.shape
    ok = len(got) == len(shape)
    if ok:
        for g, want in zip(got, shape):
            if want is not None and g != want:
                ok = False
                break
    if not ok:
        want = "[" + ", ".join("*" if d is None else str(d) for d in shape) + "]"
        raise ValueError(f"{name} must have shape {want}, got {list(got)}")
    if dtype is not None and t.dtype is not dtype and (type(dtype) is not tuple or t.dtype not in dtype):
        allowed = dtype if type(dtype) is tuple else (dtype,)
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in allowed)}, got {t.dtype}")


_ROW_DTYPES = tuple(_DTYPE_CODE)


def _same_device(layout, *tensors):
    """Every tensor on the layout's device (its workspace's), contiguous."""
    _require_gpu(*tensors)
    dev = layout.workspace.device
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError(f"tensor on {t.device}, the layout lives on {dev}")


def workspace_bytes(s: int, e: int, k: int, capacity: int, route_major: bool = False,
                    pad_multiple: int = 1) -> int:
    opts = LayoutOptions(int(route_major), pad_multiple)
    return int(lib().moe_layout_workspace_bytes_ex(s, e, k, capacity, ctypes.byref(opts)))


class Layout:
    """A dispatch layout: the C handle plus the device workspace backing it.

    `rows` is a host int. The array properties are device tensors viewing the
    workspace (read-only by convention).
    """

    def __init__(self, struct: LayoutStruct, workspace: torch.Tensor):
        self.struct = struct
        self.workspace = workspace

    @property
    def s(self): return self.struct.s
    @property
    def e(self): return self.struct.e
    @property
    def k(self): return self.struct.k
    @property
    def capacity(self): return self.struct.capacity
    @property
    def rows(self): return int(self.struct.rows)
    @property
    def route_major(self): return bool(self.struct.route_major)
    @property
    def pad_multiple(self): return int(self.struct.pad_multiple)

    def _view(self, ptr, n, dtype=torch.int32):
        off = ptr - self.workspace.data_ptr()
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype)

    @property
    def counts(self): return self._view(self.struct.counts, self.e)
    @property
    def kept(self): return self._view(self.struct.kept, self.e)
    @property
    def offsets(self): return self._view(self.struct.offsets, self.e + 1)
    @property
    def dst(self): return self._view(self.struct.dst, self.s * self.k).view(self.s, self.k)
    @property
    def src(self): return self._view(self.struct.src, self.rows)
    @property
    def route_idx(self): return self._view(self.struct.route_idx, self.s * self.k).view(self.s, self.k)

    def byref(self):
        return ctypes.byref(self.struct)


def moe_gate_topk(logits: torch.Tensor, k: int, idx_out=None, w_out=None):
    _expect(logits, "logits", (None, None), torch.float32)
    s, e = logits.shape
    _expect(idx_out, "idx_out", (s, k), torch.int32)
    _expect(w_out, "w_out", (s, k), torch.float32)
    _require_gpu(logits, idx_out, w_out)
    idx = idx_out if idx_out is not None else torch.empty((s, k), dtype=torch.int32, device=logits.device)
    w = w_out if w_out is not None else torch.empty((s, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_gate_topk(_ptr(logits), s, e, k, _ptr(idx), _ptr(w), _stream(logits)))
    return idx, w


def moe_gate_topk_backward(idx: torch.Tensor, w: torch.Tensor, grad_w: torch.Tensor, e: int, out=None):
    _expect(idx, "idx", (None, None), torch.int32)
    s, k = idx.shape
    _expect(w, "w", (s, k), torch.float32)
    _expect(grad_w, "grad_w", (s, k), torch.float32)
    _expect(out, "out", (s, e), torch.float32)
    _require_gpu(idx, w, grad_w, out)
    gl = out if out is not None else torch.empty((s, e), dtype=torch.float32, device=idx.device)
    _check(lib().moe_gate_topk_backward(_ptr(idx), _ptr(w), _ptr(grad_w), s, e, k, _ptr(gl), _stream(idx)))
    return gl


def moe_dispatch_layout(idx: torch.Tensor, e: int, capacity: int = 0, workspace=None,
                        route_major: bool = False, pad_multiple: int = 1) -> Layout:
    _expect(idx, "expert ids", (None, None), torch.int32)
    _expect(workspace, "workspace", (None,), torch.uint8)
    _require_gpu(idx, workspace)
    s, k = idx.shape
    opts = LayoutOptions(int(route_major), pad_multiple)
    nbytes = workspace_bytes(s, e, k, capacity, route_major, pad_multiple)
    if nbytes == 0:
        # let the library name the problem
        _check(lib().moe_dispatch_layout_ex(_ptr(idx), s, e, k, capacity, ctypes.byref(opts),
                                            ctypes.c_void_p(0), 0, ctypes.byref(LayoutStruct()),
                                            _stream(idx)))
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=idx.device)
    elif workspace.device != idx.device:
        raise ValueError(f"workspace on {workspace.device}, the expert ids on {idx.device}")
    st = LayoutStruct()
    _check(lib().moe_dispatch_layout_ex(_ptr(idx), s, e, k, capacity, ctypes.byref(opts),
                                        _ptr(workspace), workspace.numel(), ctypes.byref(st),
                                        _stream(idx)))
    return Layout(st, workspace)


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPE_CODE[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported element type {t.dtype}") from None


def moe_dispatch(layout: Layout, x: torch.Tensor, out=None):
    _expect(x, "x", (layout.s, None), _ROW_DTYPES)
    m = x.shape[1]
    _expect(out, "out", (layout.rows, m), x.dtype)
    _same_device(layout, x, out)
    out = out if out is not None else torch.empty((layout.rows, m), dtype=x.dtype, device=x.device)
    _check(lib().moe_dispatch(layout.byref(), _ptr(x), m, _dtype_code(x), _ptr(out), _stream(x)))
    return out


def moe_dispatch_replay(layout: Layout, x: torch.Tensor, idx=None, out=None):
    _expect(x, "x", (layout.s, None), _ROW_DTYPES)
    m = x.shape[1]
    _expect(idx, "idx", (layout.s, layout.k), torch.int32)
    _expect(out, "out", (layout.rows, m), x.dtype)
    _same_device(layout, x, idx, out)
    out = out if out is not None else torch.empty((layout.rows, m), dtype=x.dtype, device=x.device)
    _check(lib().moe_dispatch_replay(layout.byref(), _ptr(idx), _ptr(x), m, _dtype_code(x),
                                     _ptr(out), _stream(x)))
    return out


def moe_combine(layout: Layout, expert_out: torch.Tensor, w, out=None):
    """Weighted combine; w=None gives the unweighted sum (after moe_dispatch_weighted)."""
    _expect(expert_out, "expert_out", (layout.rows, None), _ROW_DTYPES)
    m = expert_out.shape[1]
    _expect(w, "w", (layout.s, layout.k), torch.float32)
    _expect(out, "out", (layout.s, m), expert_out.dtype)
    _same_device(layout, expert_out, w, out)
    y = out if out is not None else torch.empty((layout.s, m), dtype=expert_out.dtype, device=expert_out.device)
    _check(lib().moe_combine(layout.byref(), _ptr(expert_out), _ptr(w), m, _dtype_code(expert_out),
                             _ptr(y), _stream(expert_out)))
    return y


def moe_combine_backward(layout: Layout, grad_y: torch.Tensor, expert_out: torch.Tensor,
                         w: torch.Tensor, grad_expert_out=None, grad_w=None):
    _expect(grad_y, "grad_y", (layout.s, None), _ROW_DTYPES)
    m = grad_y.shape[1]
    _expect(expert_out, "expert_out", (layout.rows, m), grad_y.dtype)
    if w is None:
        raise ValueError("w is required (the combine's route weights)")
    _expect(w, "w", (layout.s, layout.k), torch.float32)
    _expect(grad_expert_out, "grad_expert_out", (layout.rows, m), grad_y.dtype)
    _expect(grad_w, "grad_w", (layout.s, layout.k), torch.float32)
    _same_device(layout, grad_y, expert_out, w, grad_expert_out, grad_w)
    gE = grad_expert_out if grad_expert_out is not None else torch.empty(
        (layout.rows, m), dtype=grad_y.dtype, device=grad_y.device)
    gw = grad_w if grad_w is not None else torch.empty((layout.s, layout.k), dtype=torch.float32,
                                                      device=grad_y.device)
    _check(lib().moe_combine_backward(layout.byref(), _ptr(grad_y), _ptr(expert_out), _ptr(w), m,
                                      _dtype_code(grad_y), _ptr(gE), _ptr(gw), _stream(grad_y)))
    return gE, gw


def moe_dispatch_backward(layout: Layout, grad_out: torch.Tensor, out=None):
    _expect(grad_out, "grad_out", (layout.rows, None), _ROW_DTYPES)
    m = grad_out.shape[1]
    _expect(out, "out", (layout.s, m), grad_out.dtype)
    _same_device(layout, grad_out, out)
    gx = out if out is not None else torch.empty((layout.s, m), dtype=grad_out.dtype, device=grad_out.device)
    _check(lib().moe_dispatch_backward(layout.byref(), _ptr(grad_out), m, _dtype_code(grad_out),
                                       _ptr(gx), _stream(grad_out)))
    return gx


def moe_dispatch_weighted(layout: Layout, x: torch.Tensor, w: torch.Tensor, out=None):
    _expect(x, "x", (layout.s, None), _ROW_DTYPES)
    m = x.shape[1]
    if w is None:
        raise ValueError("w is required (the route weights applied at dispatch)")
    _expect(w, "w", (layout.s, layout.k), torch.float32)
    _expect(out, "out", (layout.rows, m), x.dtype)
    _same_device(layout, x, w, out)
    out = out if out is not None else torch.empty((layout.rows, m), dtype=x.dtype, device=x.device)
    _check(lib().moe_dispatch_weighted(layout.byref(), _ptr(x), _ptr(w), m, _dtype_code(x), _ptr(out),
                                       _stream(x)))
    return out


def moe_dispatch_weighted_backward(layout: Layout, grad_out: torch.Tensor, x: torch.Tensor,
                                   w: torch.Tensor, grad_x=None, grad_w=None):
    _expect(x, "x", (layout.s, None), _ROW_DTYPES)
    m = x.shape[1]
    _expect(grad_out, "grad_out", (layout.rows, m), x.dtype)
    if w is None:
        raise ValueError("w is required (the route weights applied at dispatch)")
    _expect(w, "w", (layout.s, layout.k), torch.float32)
    _expect(grad_x, "grad_x", (layout.s, m), x.dtype)
    _expect(grad_w, "grad_w", (layout.s, layout.k), torch.float32)
    _same_device(layout, grad_out, x, w, grad_x, grad_w)
    gx = grad_x if grad_x is not None else torch.empty_like(x)
    gw = grad_w if grad_w is not None else torch.empty((layout.s, layout.k), dtype=torch.float32,
                                                      device=x.device)
    _check(lib().moe_dispatch_weighted_backward(layout.byref(), _ptr(grad_out), _ptr(x), _ptr(w), m,
                                                _dtype_code(x), _ptr(gx), _ptr(gw), _stream(x)))
    return gx, gw


def moe_expert_gemm(layout: Layout, a: torch.Tensor, weights: torch.Tensor, gather: bool = True,
                    w: torch.Tensor | None = None, out=None):
    """Grouped expert GEMM over the layout's segments: out[r] = A(r) @ weights[x]^T.

    a is the token rows x [s, m] when gather (the dispatch fused into the GEMM's operand
    loads), else a dispatched buffer [rows, m]; weights [e, n, m]; w [s, k] float32 scales
    each row by its route's weight, or None. Returns out [rows, n].
    """
    _expect(a, "a", (layout.s if gather else layout.rows, None), _ROW_DTYPES)
    m = a.shape[1]
    _expect(weights, "weights", (layout.e, None, m), a.dtype)
    n = weights.shape[1]
    _expect(w, "w", (layout.s, layout.k), torch.float32)
    _expect(out, "out", (layout.rows, n), a.dtype)
    _same_device(layout, a, weights, w, out)
    out = out if out is not None else torch.empty((layout.rows, n), dtype=a.dtype, device=a.device)
    _check(lib().moe_expert_gemm(layout.byref(), _ptr(a), int(bool(gather)), _ptr(weights), m, n,
                                 _dtype_code(a), _ptr(w), _ptr(out), _stream(a)))
    return out


def moe_expert_gemm_wgrad(layout: Layout, a: torch.Tensor, grad_out: torch.Tensor,
                          gather: bool = True, out=None, out_dtype=torch.float32):
    """Weight gradient of moe_expert_gemm: grad_w[x] = sum over expert x's rows r of
    outer(grad_out[r], A(r)), [e, n, m] (zeros for experts with no rows), accumulated in
    float32 and stored as float32 or rounded once to a's dtype (out_dtype, or out's dtype
    when out is given).

    a is x [s, m] when gather (rows gathered through the layout), else a dispatched
    buffer [rows, m]; grad_out [rows, n] in a's dtype.
    """
    _expect(a, "a", (layout.s if gather else layout.rows, None), _ROW_DTYPES)
    m = a.shape[1]
    _expect(grad_out, "grad_out", (layout.rows, None), a.dtype)
    n = grad_out.shape[1]
    _expect(out, "out", (layout.e, n, m), (torch.float32, a.dtype))
    _same_device(layout, a, grad_out, out)
    if out is None:
        if out_dtype not in (torch.float32, a.dtype):
            raise ValueError(f"out_dtype must be float32 or {a.dtype}, got {out_dtype}")
        out = torch.empty((layout.e, n, m), dtype=out_dtype, device=a.device)
    _check(lib().moe_expert_gemm_wgrad(layout.byref(), _ptr(a), int(bool(gather)), _ptr(grad_out), m, n,
                                       _dtype_code(a), _dtype_code(out), _ptr(out), _stream(a)))
    return out


def moe_expert_gemm_dgrad(layout: Layout, grad_out: torch.Tensor, weights: torch.Tensor, out=None):
    """Input-row gradient of moe_expert_gemm: grad_a[r] = grad_out[r] @ weights[x] for the
    placed rows of expert x, [rows, m] (zero rows where no route is placed). The token
    gradient of the gathered forward is moe_dispatch_backward(layout, grad_a)."""
    _expect(grad_out, "grad_out", (layout.rows, None), _ROW_DTYPES)
    n = grad_out.shape[1]
    _expect(weights, "weights", (layout.e, n, None), grad_out.dtype)
    m = weights.shape[2]
    _expect(out, "out", (layout.rows, m), grad_out.dtype)
    _same_device(layout, grad_out, weights, out)
    out = out if out is not None else torch.empty((layout.rows, m), dtype=grad_out.dtype, device=grad_out.device)
    _check(lib().moe_expert_gemm_dgrad(layout.byref(), _ptr(grad_out), _ptr(weights), m, n,
                                       _dtype_code(grad_out), _ptr(out), _stream(grad_out)))
    return out


def moe_renormalize_kept(layout: Layout, w: torch.Tensor, out=None):
    _expect(w, "w", (layout.s, layout.k), torch.float32)
    _expect(out, "out", (layout.s, layout.k), torch.float32)
    _same_device(layout, w, out)
    w_out = out if out is not None else torch.empty_like(w)
    _check(lib().moe_renormalize_kept(layout.byref(), _ptr(w), _ptr(w_out), _stream(w)))
    return w_out


def moe_renormalize_kept_backward(layout: Layout, w: torch.Tensor, grad_out: torch.Tensor, out=None):
    _expect(w, "w", (layout.s, layout.k), torch.float32)
    _expect(grad_out, "grad_out", (layout.s, layout.k), torch.float32)
    _expect(out, "out", (layout.s, layout.k), torch.float32)
    _same_device(layout, w, grad_out, out)
    gw = out if out is not None else torch.empty_like(w)
    _check(lib().moe_renormalize_kept_backward(layout.byref(), _ptr(w), _ptr(grad_out), _ptr(gw),
                                               _stream(w)))
    return gw


def moe_layout_read(layout: Layout):
    flags = ctypes.c_int32(0)
    checksum = ctypes.c_uint64(0)
    _check(lib().moe_layout_read(layout.byref(), ctypes.byref(flags), ctypes.byref(checksum),
                                 _stream(layout.workspace)))
    return int(flags.value), int(checksum.value)


__all__ = [
    "moe_gate_topk", "moe_gate_topk_backward", "moe_dispatch_layout", "moe_dispatch",
    "moe_dispatch_replay", "moe_combine", "moe_combine_backward", "moe_dispatch_backward",
    "moe_layout_read", "moe_dispatch_weighted", "moe_dispatch_weighted_backward",
    "moe_renormalize_kept", "moe_renormalize_kept_backward", "moe_expert_gemm", "moe_expert_gemm_wgrad", "moe_expert_gemm_dgrad", "workspace_bytes", "Layout",
    "LayoutOptions", "MoeError", "lib", "EXPORTS",
]
