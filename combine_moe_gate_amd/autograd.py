"""PyTorch autograd over the MoE gate / dispatch / combine library, and an
activation-checkpoint layout recorder.

Every forward and backward step calls the library's HIP kernels; these classes
only wire them into autograd:

    idx, w  = route(logits, k, rec)               # w carries a gradient to the logits
    buf, L  = dispatch(x, idx, e, capacity, rec)  # buf [L.rows, m]; grad -> x
    y       = combine(expert_out, w, L)           # grads -> expert_out and w

Dispatch and combine are each other's adjoint, so the backward of one runs the
other's kernel on the layout the forward built (DeepSpeed PR "Add an opt-in
DeepEP transport for the AutoEP expert all-to-all", first commit). The routing
weights are an autograd output of the gate and an input of the combine, so the
router receives their gradient (same page, review-fix commit).

LayoutRecorder follows NeMo Automodel PR "perf(moe): reuse the DeepEP dispatch
layout on activation-checkpoint recompute", section 1 and its "How" part: one
recorder per checkpointed call. The forward logs, in call order, each gate's
routing (expert ids and weights) and each dispatch's layout; only this routing
metadata is kept, never the dispatched rows. The recompute consumes the log in
the same order: the gate hands back the recorded routing instead of running
top-k again (the router is bypassed, and the weights' gradient still reaches the
logits through the recorded selection), and the dispatch replays the recorded
layout without rebuilding it. The replayed layout therefore always meets the
routing it was built from. A layout replayed for routing that did not come from
the recorder's gate is verified on the GPU against the recorded routing, and the
backward of that dispatch raises if they differ: a mis-route fails loudly
instead of silently. A recompute that outruns its log builds afresh.
"""
from __future__ import annotations

import torch
import torch.utils.checkpoint

from . import (FLAG_REPLAY_MISMATCH, Layout, moe_combine, moe_combine_backward, moe_dispatch,
               moe_dispatch_backward, moe_dispatch_layout, moe_dispatch_replay,
               moe_dispatch_weighted, moe_dispatch_weighted_backward, moe_expert_gemm,
               moe_expert_gemm_dgrad, moe_expert_gemm_wgrad, moe_gate_topk,
               moe_gate_topk_backward, moe_layout_read, moe_renormalize_kept,
               moe_renormalize_kept_backward)


class _Gate(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, k):
        idx, w = moe_gate_topk(logits.contiguous(), k)
        ctx.save_for_backward(idx, w)
        ctx.e = logits.shape[1]
        ctx.mark_non_differentiable(idx)
        return idx, w

    @staticmethod
    def backward(ctx, _g_idx, g_w):
        idx, w = ctx.saved_tensors
        if g_w is None:
            return None, None
        return moe_gate_topk_backward(idx, w, g_w.float().contiguous(), ctx.e), None


class _GateReplay(torch.autograd.Function):
    """The gate on a recompute, pinned to the forward's record: the recorded weights come
    back as they are (top-k is not run again on the recomputed logits), and their
    gradient reaches the logits through the recorded selection (the gate backward needs
    only the ids and weights)."""

    @staticmethod
    def forward(ctx, logits, idx, w):
        ctx.save_for_backward(idx, w)
        ctx.e = logits.shape[1]
        return w.clone()

    @staticmethod
    def backward(ctx, g_w):
        idx, w = ctx.saved_tensors
        return moe_gate_topk_backward(idx, w, g_w.float().contiguous(), ctx.e), None, None


def _raise_on_replay_mismatch(layout: Layout) -> None:
    """Raise if a replay of `layout` was handed routing that differs from the recorded one.

    Inside a backward pass (where a checkpoint's recompute runs) the check is queued to
    run when that pass ends, costing one synchronisation per backward; outside one it
    runs at once."""

    def check():
        flags, _ = moe_layout_read(layout)  # synchronises
        if flags & FLAG_REPLAY_MISMATCH:
            raise RuntimeError("a checkpoint recompute replayed a dispatch layout for routing that "
                               "differs from the forward's (route through the recorder to pin it)")

    try:
        torch.autograd.Variable._execution_engine.queue_callback(check)
    except RuntimeError:  # not inside a backward pass
        check()


class _Dispatch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, layout, verify_idx):
        ctx.layout = layout
        if verify_idx is not None:
            out = moe_dispatch_replay(layout, x.contiguous(), verify_idx)
            _raise_on_replay_mismatch(layout)
            return out
        return moe_dispatch(layout, x.contiguous())

    @staticmethod
    def backward(ctx, g_buf):
        return moe_dispatch_backward(ctx.layout, g_buf.contiguous()), None, None


class _DispatchWeighted(torch.autograd.Function):
    """Weights applied before the experts: out[dst] = w * x."""

    @staticmethod
    def forward(ctx, x, w, layout):
        x = x.contiguous()
        w = w.contiguous()
        ctx.layout = layout
        ctx.save_for_backward(x, w)
        return moe_dispatch_weighted(layout, x, w)

    @staticmethod
    def backward(ctx, g_buf):
        x, w = ctx.saved_tensors
        g_x, g_w = moe_dispatch_weighted_backward(ctx.layout, g_buf.contiguous(), x, w)
        return g_x, g_w, None


class _Combine(torch.autograd.Function):
    @staticmethod
    def forward(ctx, expert_out, w, layout):
        expert_out = expert_out.contiguous()
        w = w.contiguous()
        ctx.layout = layout
        ctx.save_for_backward(expert_out, w)
        return moe_combine(layout, expert_out, w)

    @staticmethod
    def backward(ctx, g_y):
        expert_out, w = ctx.saved_tensors
        g_e, g_w = moe_combine_backward(ctx.layout, g_y.contiguous(), expert_out, w)
        return g_e, g_w, None


class _Sum(torch.autograd.Function):
    """Unweighted combine (after a weighted dispatch); its gradient is a plain dispatch."""

    @staticmethod
    def forward(ctx, expert_out, layout):
        ctx.layout = layout
        return moe_combine(layout, expert_out.contiguous(), None)

    @staticmethod
    def backward(ctx, g_y):
        return moe_dispatch(ctx.layout, g_y.contiguous()), None


class _Renormalize(torch.autograd.Function):
    @staticmethod
    def forward(ctx, w, layout):
        w = w.contiguous()
        ctx.layout = layout
        ctx.save_for_backward(w)
        return moe_renormalize_kept(layout, w)

    @staticmethod
    def backward(ctx, g):
        (w,) = ctx.saved_tensors
        return moe_renormalize_kept_backward(ctx.layout, w, g.float().contiguous()), None


class _ExpertLinear(torch.autograd.Function):
    """One linear projection per expert over the layout's rows, gathered from x."""

    @staticmethod
    def forward(ctx, x, weights, layout):
        x = x.contiguous()
        weights = weights.contiguous()
        ctx.layout = layout
        ctx.save_for_backward(x, weights)
        return moe_expert_gemm(layout, x, weights, gather=True)

    @staticmethod
    def backward(ctx, g_h):
        x, weights = ctx.saved_tensors
        g_h = g_h.contiguous()
        g_x = g_w = None
        if ctx.needs_input_grad[0]:  # input rows, then each token's routes summed
            g_x = moe_dispatch_backward(ctx.layout, moe_expert_gemm_dgrad(ctx.layout, g_h, weights))
        if ctx.needs_input_grad[1]:  # float32 sums, rounded once to the parameter's dtype in the kernel
            g_w = moe_expert_gemm_wgrad(ctx.layout, x, g_h, gather=True, out_dtype=weights.dtype)
        return g_x, g_w, None


class LayoutRecorder:
    """Routing and layouts of one checkpointed call, recorded on its forward, replayed on
    its recompute.

    Enter it (``with rec:``) around each pass of the checkpointed function. The first
    pass records; every later pass replays from the start of the log. `verify` (on by
    default) checks a replayed layout against the routing the recompute hands it when
    that routing did not come from this recorder's gate; the dispatch's backward then
    raises on a mismatch.
    """

    def __init__(self, verify: bool = True):
        self.verify = verify
        self.log: list[tuple[Layout, tuple]] = []
        self.routes: list[tuple[torch.Tensor, torch.Tensor, int, int]] = []
        self.passes = 0
        self._cursor = 0
        self._route_cursor = 0
        self._recording = True
        self.layouts_built = 0
        self.replays = 0
        self.fallbacks = 0
        self.routes_replayed = 0
        self.route_fallbacks = 0
        self._replayed: list[Layout] = []

    def __enter__(self):
        self._recording = self.passes == 0
        self._cursor = 0
        self._route_cursor = 0
        return self

    def __exit__(self, *exc):
        self.passes += 1
        return False

    def route_for(self, logits: torch.Tensor, k: int):
        """Top-k ids and weights: computed and logged on the forward, the logged ones on a
        recompute (with the weights' gradient routed to the recomputed logits)."""
        s, e = logits.shape
        if self._recording:
            idx, w = _Gate.apply(logits, k)
            self.routes.append((idx, w.detach(), e, k))
            return idx, w
        if self._route_cursor < len(self.routes):
            idx, w, e_rec, k_rec = self.routes[self._route_cursor]
            self._route_cursor += 1
            if (s, e, k) != (idx.shape[0], e_rec, k_rec):
                raise RuntimeError(f"recompute asked to route {(s, e, k)}, the forward recorded "
                                   f"{(idx.shape[0], e_rec, k_rec)}")
            self.routes_replayed += 1
            return idx, _GateReplay.apply(logits, idx, w)
        self.route_fallbacks += 1  # the recompute outran its log: route afresh
        return _Gate.apply(logits, k)

    def _pinned(self, idx: torch.Tensor) -> bool:
        """Whether idx is routing this recorder's gate logged (and so the routing the
        recorded layouts were built from)."""
        return any(idx is r[0] for r in self.routes)

    def layout_for(self, idx: torch.Tensor, e: int, capacity: int, **options):
        """The layout to dispatch with, and the routing to verify a replay against."""
        key = (tuple(idx.shape), e, capacity, tuple(sorted(options.items())))
        if self._recording:
            layout = moe_dispatch_layout(idx, e, capacity, **options)
            self.layouts_built += 1
            self.log.append((layout, key))
            return layout, None
        if self._cursor < len(self.log):
            layout, rec_key = self.log[self._cursor]
            self._cursor += 1
            if rec_key != key:
                raise RuntimeError(f"recompute asked for a layout of {key}, the forward recorded {rec_key}")
            self.replays += 1
            self._replayed.append(layout)
            verify = self.verify and not self._pinned(idx)
            return layout, (idx.contiguous() if verify else None)
        self.fallbacks += 1  # the recompute outran its log: build the layout afresh
        layout = moe_dispatch_layout(idx, e, capacity, **options)
        self.layouts_built += 1
        return layout, None

    def check(self) -> None:
        """Raise if any verified replay was handed routing that differs (synchronises)."""
        for layout in self._replayed:
            flags, _ = moe_layout_read(layout)
            if flags & FLAG_REPLAY_MISMATCH:
                raise RuntimeError("a recompute replayed a layout with routing that differs from the forward's")


def route(logits: torch.Tensor, k: int, recorder: LayoutRecorder | None = None):
    """Top-k expert ids (no gradient) and renormalised weights (gradient to the logits);
    with a recorder, logged on the forward and handed back unchanged on the recompute."""
    if recorder is not None:
        return recorder.route_for(logits, k)
    return _Gate.apply(logits, k)


def layout(idx: torch.Tensor, e: int, capacity: int = 0, recorder: LayoutRecorder | None = None,
           route_major: bool = False, pad_multiple: int = 1):
    """The dispatch layout (recorded or replayed through `recorder` if given)."""
    options = dict(route_major=route_major, pad_multiple=pad_multiple)
    if recorder is not None:
        return recorder.layout_for(idx, e, capacity, **options)
    return moe_dispatch_layout(idx, e, capacity, **options), None


def dispatch(x: torch.Tensor, idx: torch.Tensor, e: int, capacity: int = 0,
             recorder: LayoutRecorder | None = None, w: torch.Tensor | None = None,
             route_major: bool = False, pad_multiple: int = 1):
    """Permute token rows into the expert-grouped buffer. Returns (buffer, layout).

    With w given, the weights are applied here, before the experts (the combine is
    then combine(expert_out, None, layout)); a recorder's routing verification
    covers the plain dispatch only.
    """
    L, verify_idx = layout(idx, e, capacity, recorder, route_major, pad_multiple)
    if w is not None:
        return _DispatchWeighted.apply(x, w, L), L
    return _Dispatch.apply(x, L, verify_idx), L


def dispatch_on(x: torch.Tensor, layout: Layout, w: torch.Tensor | None = None):
    """Dispatch on a layout built earlier (e.g. one whose weights were renormalised)."""
    if w is not None:
        return _DispatchWeighted.apply(x, w, layout)
    return _Dispatch.apply(x, layout, None)


def combine(expert_out: torch.Tensor, w: torch.Tensor | None, layout: Layout):
    """Route-ordered float32 sum of each token's expert rows, weighted unless w is None."""
    if w is None:
        return _Sum.apply(expert_out, layout)
    return _Combine.apply(expert_out, w, layout)


def expert_linear(x: torch.Tensor, weights: torch.Tensor, layout: Layout):
    """Each placed row r of expert x: x[src[r]] @ weights[x]^T, the dispatch fused into the
    grouped GEMM's operand loads (forward, input-row gradient and weight gradient all run
    on the layout). weights [e, n, m]; returns [rows, n] for combine()."""
    return _ExpertLinear.apply(x, weights, layout)


def renormalize(w: torch.Tensor, layout: Layout):
    """Weights renormalised over each token's kept routes (after the capacity drop)."""
    return _Renormalize.apply(w, layout)


def checkpoint(fn, *args, verify: bool = True, **kwargs):
    """torch.utils.checkpoint of fn(recorder, *args), with layouts replayed on recompute."""
    rec = LayoutRecorder(verify=verify)

    def run(*a):
        with rec:
            return fn(rec, *a)

    out = torch.utils.checkpoint.checkpoint(run, *args, use_reentrant=False, **kwargs)
    return out, rec


__all__ = ["route", "layout", "dispatch", "dispatch_on", "combine", "renormalize", "expert_linear", "checkpoint",
           "LayoutRecorder"]
