"""Loop oracle: the plain definitions of the path, one element at a time in Python.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests and the
benchmark's CPU-baseline leg, never by the product path.

A second CPU reference, written as explicit loops over tokens, routes and row
elements in the order the steps are defined, with no vectorisation and no numpy
routine standing in for a step (numpy only holds the arrays and rounds single
values to float32/float16). It is the slow baseline the benchmark times on the
tiny workload, and a brute-force pin of the vectorised oracle in `oracle.moe`: the
tests run both on small batches and require the same ids, layouts and buffers,
the same float32 sums, and weights and dot products within one float32 ulp (the
two sum float64 values in different orders). It takes the same readings as
`oracle.moe` and covers the default path (token-order slots, no pad multiple).

Steps, cited by page title and section:
  gate      DeepSpeed PR "MoE dispatch: fix silent Tutel + TP corruption, speed up
            native and Tutel paths", part 1 (the top-k columns name the selected
            experts); softmax, top-k, renormalise over the k (the workloads' order).
  layout    same page, review comment on fast_cumsum_sub_one: a route's slot is the
            number of earlier tokens that chose its expert; part 2: routes at or past
            the capacity are dropped; DeepSpeed PR "Add an opt-in DeepEP transport for
            the AutoEP expert all-to-all", review thread on the prefix sum: dropless
            segments start at the exclusive prefix sum of the counts.
  dispatch  DeepSpeed PR 8195 part 3; PR 8213 first commit (a token is copied to
            each of its experts).
  combine   PR 8195 part 3 (float32 accumulation); PR 8213 review thread on combine
            weights (the weights are applied in the combine).
  backward  PR 8213 first commit (combine's gradient is a weighted dispatch, the
            dispatch's gradient an unweighted combine) and review-fix commit (the
            weights' gradient, and through the gate, the logits').
"""
from __future__ import annotations

import math
import struct

import numpy as np

_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def _f32(v: float) -> float:
    """v rounded to the nearest float32 (ties to even), as a Python float."""
    return float(np.float32(v))


def widen(v, dtype: str) -> float:
    """One stored element as its exact value."""
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(v) << 16))[0]
    return float(v)


def narrow(v: float, dtype: str):
    """A float32 value rounded to nearest even in the element type (stored form)."""
    if dtype == "f32":
        return np.float32(v)
    if dtype == "f16":
        return np.float16(np.float32(v))
    bits = struct.unpack("<I", struct.pack("<f", v))[0]
    if (bits & 0x7F800000) == 0x7F800000 and (bits & 0x007FFFFF):  # NaN stays NaN
        return np.uint16((bits >> 16) | 0x0040)
    low = bits & 0xFFFF
    keep = bits >> 16
    if low > 0x8000 or (low == 0x8000 and (keep & 1)):  # round half to even
        keep += 1
    return np.uint16(keep & 0xFFFF)


def gate_topk(logits: np.ndarray, k: int):
    """Per token: the k largest logits (ties to the lower expert id), and the softmax
    over all e logits renormalised over the selection, in float64, rounded to float32."""
    s, e = logits.shape
    idx = np.zeros((s, k), np.int32)
    w = np.zeros((s, k), np.float32)
    for t in range(s):
        row = [float(v) for v in logits[t]]
        order = sorted(range(e), key=lambda i: (-row[i], i))  # -0.0 == +0.0 here
        top = max(row)
        p = [math.exp(v - top) for v in row]
        total = 0.0
        for v in p:
            total += v
        sel = [p[order[j]] / total for j in range(k)]
        sel_total = 0.0
        for v in sel:
            sel_total += v
        for j in range(k):
            idx[t, j] = order[j]
            w[t, j] = np.float32(sel[j] / sel_total)
    return idx, w


class LoopLayout:
    """The layout as plain lists: counts, kept, offsets, dst[t][j], src[r]."""

    def __init__(self, s, e, k, capacity, rows, counts, kept, offsets, dst, src, flags, checksum):
        self.s, self.e, self.k, self.capacity, self.rows = s, e, k, capacity, rows
        self.counts, self.kept, self.offsets = counts, kept, offsets
        self.dst, self.src, self.flags, self.checksum = dst, src, flags, checksum


def dispatch_layout(idx: np.ndarray, e: int, capacity: int) -> LoopLayout:
    """Walk the routes in token order, j = 0..k-1 within a token: a valid route to
    expert x takes slot seen[x] and increments it. Invalid routes (expert outside
    [0, e), or one an earlier route of the token named) are flagged and skipped."""
    s, k = idx.shape
    seen = [0] * e
    slot = [[-1] * k for _ in range(s)]
    flags = 0
    checksum = 0
    for t in range(s):
        for j in range(k):
            x = int(idx[t, j])
            checksum = (checksum + (x + 1) * (t * k + j + 1)) % (1 << 64)
            if not 0 <= x < e:
                flags |= 1
                continue
            if any(int(idx[t, q]) == x for q in range(j)):
                flags |= 2
                continue
            slot[t][j] = seen[x]
            seen[x] += 1
    counts = list(seen)
    if capacity > 0:
        rows = e * capacity
        kept = [min(c, capacity) for c in counts]
        offsets = [x * capacity for x in range(e + 1)]
    else:
        rows = s * k
        kept = list(counts)
        offsets = [0] * (e + 1)
        for x in range(e):
            offsets[x + 1] = offsets[x] + counts[x]
    dst = [[-1] * k for _ in range(s)]
    src = [-1] * rows
    for t in range(s):
        for j in range(k):
            if slot[t][j] < 0:
                continue
            x = int(idx[t, j])
            if capacity > 0 and slot[t][j] >= capacity:
                continue  # dropped
            d = offsets[x] + slot[t][j]
            dst[t][j] = d
            src[d] = t
    return LoopLayout(s, e, k, max(capacity, 0), rows, counts, kept, offsets, dst, src, flags, checksum)


def dispatch(L: LoopLayout, x: np.ndarray) -> np.ndarray:
    """out[dst[t][j]] = x[t], element by element; rows no route fills stay zero."""
    m = x.shape[1]
    out = np.zeros((L.rows, m), dtype=x.dtype)
    for t in range(L.s):
        for j in range(L.k):
            d = L.dst[t][j]
            if d >= 0:
                for i in range(m):
                    out[d, i] = x[t, i]
    return out


def _route_sum(L: LoopLayout, rows_in: np.ndarray, w, dtype: str) -> np.ndarray:
    """y[t][i] = sum over placed routes j in order of w[t][j] * rows_in[dst[t][j]][i],
    each product and each sum rounded to float32, then once to the element type."""
    m = rows_in.shape[1]
    y = np.zeros((L.s, m), dtype=_NP[dtype])
    for t in range(L.s):
        acc = [0.0] * m
        for j in range(L.k):
            d = L.dst[t][j]
            if d < 0:
                continue
            wj = float(np.float32(w[t, j])) if w is not None else None
            for i in range(m):
                v = widen(rows_in[d, i], dtype)
                term = _f32(wj * v) if wj is not None else v
                acc[i] = _f32(acc[i] + term)
        for i in range(m):
            y[t, i] = narrow(acc[i], dtype)
    return y


def combine(L: LoopLayout, expert_out: np.ndarray, w: np.ndarray, dtype: str) -> np.ndarray:
    return _route_sum(L, expert_out, w, dtype)


def combine_backward(L: LoopLayout, grad_y: np.ndarray, expert_out: np.ndarray, w: np.ndarray,
                     dtype: str):
    """grad_E[dst[t][j]][i] = w[t][j] * grad_y[t][i] (float32 product, narrowed); rows no
    route points at are zero. grad_w[t][j] = sum_i grad_y[t][i] * E[dst[t][j]][i], summed
    exactly (math.fsum) and rounded to float32; 0 for a dropped route."""
    m = grad_y.shape[1]
    gE = np.zeros((L.rows, m), dtype=_NP[dtype])
    gw = np.zeros((L.s, L.k), np.float32)
    for t in range(L.s):
        for j in range(L.k):
            d = L.dst[t][j]
            if d < 0:
                continue
            wj = float(np.float32(w[t, j]))
            terms = []
            for i in range(m):
                g = widen(grad_y[t, i], dtype)
                gE[d, i] = narrow(_f32(wj * g), dtype)
                terms.append(g * widen(expert_out[d, i], dtype))  # exact in float64
            gw[t, j] = np.float32(math.fsum(terms))
    return gE, gw


def dispatch_backward(L: LoopLayout, grad_out: np.ndarray, dtype: str) -> np.ndarray:
    """grad_x[t] = sum over placed routes, in order, of grad_out[dst[t][j]] (float32)."""
    return _route_sum(L, grad_out, None, dtype)


def gate_topk_backward(idx: np.ndarray, w: np.ndarray, grad_w: np.ndarray, e: int) -> np.ndarray:
    """grad_logits[t][idx[t][j]] = w_j (g_j - sum_q w_q g_q) in float64, rounded once;
    zero for every unselected expert."""
    s, k = idx.shape
    gl = np.zeros((s, e), np.float32)
    for t in range(s):
        ws = [float(np.float32(w[t, j])) for j in range(k)]
        gs = [float(np.float32(grad_w[t, j])) for j in range(k)]
        dot = 0.0
        for j in range(k):
            dot += ws[j] * gs[j]
        acc = {}
        for j in range(k):
            x = int(idx[t, j])
            if 0 <= x < e:
                acc[x] = acc.get(x, 0.0) + ws[j] * (gs[j] - dot)
        for x, v in acc.items():
            gl[t, x] = np.float32(v)
    return gl


def layout_arrays(L: LoopLayout) -> dict:
    """The layout as int32 arrays, for comparison with other implementations."""
    return {"counts": np.array(L.counts, np.int32), "kept": np.array(L.kept, np.int32),
            "offsets": np.array(L.offsets, np.int32), "dst": np.array(L.dst, np.int32).reshape(L.s, L.k),
            "src": np.array(L.src, np.int32)}
