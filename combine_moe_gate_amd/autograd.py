"""PyTorch autograd over the MoE gate / dispatch / combine library, and an
activation-checkpoint layout recorder.

Every forward and backward step calls the library's HIP kernels; these classes
only wire them into autograd:

    idx, w  = route(logits, k)                    # w carries a gradient to the logits
    buf, L  = dispatch(x, idx, e, capacity, rec)  # buf [L.rows, m]; grad -> x
    y       = combine(expert_out, w, L)           # grads -> expert_out and w

The gradient of a combine is a dispatch and the gradient of a dispatch is a
combine, both on the forward's layout (DeepSpeed PR "Add an opt-in DeepEP
transport for the AutoEP expert all-to-all", first commit). The routing
weights are an autograd output of the gate and an input of the combine, so
their gradient reaches the router (same page, review-fix commit: returning no
gradient for them silently stopped the gate from learning).

LayoutRecorder follows NeMo Automodel PR "perf(moe): reuse the DeepEP dispatch
layout on activation-checkpoint recompute", section 1 and its "How" part: one
recorder per checkpointed call; the forward logs each dispatch's layout (and
its routing) in call order; the recompute consumes them in the same order and
replays the dispatch without rebuilding the layout; a recompute that outruns
its log falls back to a full layout; the dispatched rows themselves are not
kept, only routing metadata. With verify=True a replay compares the routing it
is handed with the recorded one on the GPU, and check() raises if any differed
(fail loudly rather than mis-route silently).
"""
from __future__ import annotations

import torch
import torch.utils.checkpoint

from . import (FLAG_REPLAY_MISMATCH, Layout, moe_combine, moe_combine_backward, moe_dispatch,
               moe_dispatch_backward, moe_dispatch_layout, moe_dispatch_replay, moe_gate_topk,
               moe_gate_topk_backward, moe_layout_read)


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


class _Dispatch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, layout, verify_idx):
        ctx.layout = layout
        if verify_idx is not None:
            return moe_dispatch_replay(layout, x.contiguous(), verify_idx)
        return moe_dispatch(layout, x.contiguous())

    @staticmethod
    def backward(ctx, g_buf):
        return moe_dispatch_backward(ctx.layout, g_buf.contiguous()), None, None


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


class LayoutRecorder:
    """Layouts of one checkpointed call, recorded on its forward, replayed on its recompute.

    Enter it (``with rec:``) around each pass of the checkpointed function. The
    first pass records; every later pass replays from the start of the log.
    """

    def __init__(self, verify: bool = False):
        self.verify = verify
        self.log: list[tuple[Layout, tuple]] = []
        self.passes = 0
        self._cursor = 0
        self._recording = True
        self.layouts_built = 0
        self.replays = 0
        self.fallbacks = 0
        self._replayed: list[Layout] = []

    def __enter__(self):
        self._recording = self.passes == 0
        self._cursor = 0
        return self

    def __exit__(self, *exc):
        self.passes += 1
        return False

    def layout_for(self, idx: torch.Tensor, e: int, capacity: int):
        """The layout to dispatch with, and the routing to verify a replay against."""
        key = (tuple(idx.shape), e, capacity)
        if self._recording:
            layout = moe_dispatch_layout(idx, e, capacity)
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
            return layout, (idx.contiguous() if self.verify else None)
        self.fallbacks += 1  # the recompute outran its log: build the layout afresh
        layout = moe_dispatch_layout(idx, e, capacity)
        self.layouts_built += 1
        return layout, None

    def check(self) -> None:
        """Raise if any verified replay was handed routing that differs (synchronises)."""
        for layout in self._replayed:
            flags, _ = moe_layout_read(layout)
            if flags & FLAG_REPLAY_MISMATCH:
                raise RuntimeError("a recompute replayed a layout with routing that differs from the forward's")


def route(logits: torch.Tensor, k: int):
    """Top-k expert ids (no gradient) and renormalised weights (gradient to the logits)."""
    return _Gate.apply(logits, k)


def dispatch(x: torch.Tensor, idx: torch.Tensor, e: int, capacity: int = 0,
             recorder: LayoutRecorder | None = None):
    """Permute token rows into the expert-grouped buffer. Returns (buffer, layout)."""
    if recorder is not None:
        layout, verify_idx = recorder.layout_for(idx, e, capacity)
    else:
        layout, verify_idx = moe_dispatch_layout(idx, e, capacity), None
    return _Dispatch.apply(x, layout, verify_idx), layout


def combine(expert_out: torch.Tensor, w: torch.Tensor, layout: Layout):
    """Weighted, route-ordered float32 sum of each token's expert rows."""
    return _Combine.apply(expert_out, w, layout)


def checkpoint(fn, *args, verify: bool = False, **kwargs):
    """torch.utils.checkpoint of fn(recorder, *args), with layouts replayed on recompute."""
    rec = LayoutRecorder(verify=verify)

    def run(*a):
        with rec:
            return fn(rec, *a)

    out = torch.utils.checkpoint.checkpoint(run, *args, use_reentrant=False, **kwargs)
    return out, rec


__all__ = ["route", "dispatch", "combine", "checkpoint", "LayoutRecorder"]
