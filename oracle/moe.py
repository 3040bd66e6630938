"""Reference semantics of the MoE gate / dispatch / combine path, on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path.

Every function is the plain definition written out with numpy, in the order the
pages give the steps. Library primitives used as single steps: a stable argsort
(top-k selection), np.exp, np.cumsum (the cumsum-minus-one slot), fancy-index
gathers. There is no blocking, fusion or reordering.

Element types: "f32" -> float32 arrays, "f16" -> float16 arrays, "bf16" -> uint16
arrays of bfloat16 bit patterns. Low-precision values are widened to float32
exactly; results are narrowed with round-to-nearest-even.

Readings where the pages are silent (each one is also listed in the design notes):
  * Top-k selects on the logits, largest first, ties to the lower expert id
    (softmax is monotone, so this is the exact-softmax order without exp
    rounding ties). +0.0 and -0.0 compare equal.
  * Weights: softmax over all e logits in float64, then the k selected
    probabilities renormalised to sum to one, rounded once to float32.
  * Slots: token order over the union of a token's k routes; capacity drop
    applies after renormalisation, and kept weights are not renormalised again.
  * A route whose expert id is outside [0, e), or repeats an earlier route of
    the same token, is invalid: it is flagged, not counted and never placed.
  * Combine and both backward gathers accumulate in float32 in route order
    j = 0..k-1, skipping dropped routes, with separate multiply and add (no
    fused multiply-add), and round once to the output type.
  * The per-route weight gradient is a dot product over m formed in float64 and
    rounded once to float32.
  * Routing checksum: sum over routes of (idx + 1) * (t*k + j + 1) modulo 2**64,
    with idx read as a signed 32-bit integer. The checksum compared in the
    checkpoint-recompute page has no published definition; this one is ours.
  * Grouped expert GEMM: one projection per expert, weights [e, n, m]; its sums
    are exact (float64) and rounded once to the element type (forward, input-row
    gradient) or to float32 (weight gradient), the latter optionally rounded once
    more, to nearest even, to the element type.

Parity status: every function here is pinned by the `not gpu` tests (brute
force on tiny inputs, the dense one-hot einsum the index path replaced, closed
forms, finite differences and adjoint identities; the grouped expert GEMM and its
two gradients by loops, scaled identities, the forward/backward adjoint identities
and exact integer derivatives, the weight gradient kept in the element type by
ties-to-even sums). Parity unpinned: the routing checksum's definition. The pages
print no definition for it, so it is our own, pinned to that definition only by a
hand-worked fixture.
"""
from __future__ import annotations

import dataclasses

import numpy as np

FLAG_EXPERT_OUT_OF_RANGE = 1
FLAG_DUPLICATE_EXPERT = 2
FLAG_REPLAY_MISMATCH = 4


# ----------------------------------------------------------------------------
# element types


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float32 (exact for all three element types)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "f16":
        assert a.dtype == np.float16
        return a.astype(np.float32)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def from_f32(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Narrow float32 values to the element type, round to nearest even."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f32":
        return a32.copy()
    if dtype == "f16":
        return a32.astype(np.float16)
    if dtype == "bf16":
        u = a32.view(np.uint32)
        odd = (u >> np.uint32(16)) & np.uint32(1)
        r = ((u + np.uint32(0x7FFF) + odd) >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(a32)
        if nan.any():
            sign = ((u[nan] >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16)
            r[nan] = sign | np.uint16(0x7FC0)
        return r
    raise ValueError(dtype)


def zeros(shape, dtype: str) -> np.ndarray:
    return np.zeros(shape, dtype={"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype])


# ----------------------------------------------------------------------------
# step 1: top-k gate


def gate_weights_f64(logits64: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Renormalised top-k weights in float64.

    Softmax over all e experts, then the selected k probabilities divided by
    their sum ([DS-8195] part 1: the gate returns per-route gate values for the
    selected experts; the softmax-then-renormalise order is the workload's).
    """
    z = logits64 - logits64.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def gate_topk(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-k expert ids and renormalised weights per token.

    logits: [s, e] float32. Returns idx [s, k] int32 (largest logit first, ties
    to the lower expert id) and w [s, k] float32.
    [DS-8195] part 1: the top-k columns name the selected experts, and routing
    metadata is handed on as contiguous int32 per-route values.
    """
    l32 = np.asarray(logits, dtype=np.float32)
    s, e = l32.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= k <= e")
    if s == 0:
        return np.zeros((0, k), np.int32), np.zeros((0, k), np.float32)
    l64 = l32.astype(np.float64)
    idx = np.argsort(-l64, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = gate_weights_f64(l64, idx).astype(np.float32)
    return idx, w


def gate_topk_backward(idx: np.ndarray, w: np.ndarray, grad_w: np.ndarray, e: int) -> np.ndarray:
    """Gradient of the renormalised top-k weights with respect to the logits.

    The renormalised weights equal a softmax over the k selected logits (the
    full-softmax denominator cancels), so for selected expert i_j:
        grad_logits[i_j] = w_j * (grad_w_j - sum_q w_q * grad_w_q)
    and every unselected logit gets exactly zero. Formed in float64, rounded once
    to float32. Routes with an out-of-range id are left out of the scatter.
    [DS-8213] review-fix commit: the weights must carry a gradient back to the
    router gate.
    """
    s, k = idx.shape
    w64 = np.asarray(w, np.float32).astype(np.float64)
    g64 = np.asarray(grad_w, np.float32).astype(np.float64)
    dot = (w64 * g64).sum(axis=1, keepdims=True)
    contrib = w64 * (g64 - dot)
    gl = np.zeros((s, e), np.float64)
    rows = np.arange(s)
    for j in range(k):
        col = idx[:, j].astype(np.int64)
        ok = (col >= 0) & (col < e)
        np.add.at(gl, (rows[ok], col[ok]), contrib[ok, j])
    return gl.astype(np.float32)


# ----------------------------------------------------------------------------
# step 2: dispatch layout


@dataclasses.dataclass
class Layout:
    s: int
    e: int
    k: int
    capacity: int  # <= 0: dropless
    rows: int
    idx: np.ndarray  # [s, k] int32, the routing the layout was built from
    counts: np.ndarray  # [e] int32, valid routes per expert before any drop
    kept: np.ndarray  # [e] int32, routes placed per expert
    offsets: np.ndarray  # [e+1] int32, first buffer row of each expert's segment
    dst: np.ndarray  # [s, k] int32, buffer row of each route, -1 if not placed
    src: np.ndarray  # [rows] int32, token of each buffer row, -1 for padding
    flags: int
    checksum: int


def routing_checksum(idx: np.ndarray) -> int:
    """sum over routes of (idx+1) * (t*k + j + 1), modulo 2**64 (our definition)."""
    s, k = idx.shape
    a = (idx.astype(np.int64).reshape(-1) + 1).astype(np.uint64)
    b = np.arange(1, s * k + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return int(np.sum(a * b, dtype=np.uint64))


def route_validity(idx: np.ndarray, e: int) -> tuple[np.ndarray, int]:
    """Which routes are placeable, and the flag bits for the ones that are not."""
    s, k = idx.shape
    in_range = (idx >= 0) & (idx < e)
    dup = np.zeros((s, k), dtype=bool)
    for j in range(k):
        for jp in range(j):
            dup[:, j] |= idx[:, j] == idx[:, jp]
    dup &= in_range
    flags = 0
    if (~in_range).any():
        flags |= FLAG_EXPERT_OUT_OF_RANGE
    if dup.any():
        flags |= FLAG_DUPLICATE_EXPERT
    return in_range & ~dup, flags


def dispatch_layout(idx: np.ndarray, e: int, capacity: int, route_major: bool = False,
                    pad_multiple: int = 1) -> Layout:
    """Per-expert counts, token-order slots, capacity drop and the row maps.

    [DS-8195] review comment on fast_cumsum_sub_one: a route's slot in its
    expert is the column cumsum of the token x expert mask minus one, so slots
    follow token order. [DS-8195] parts 2 and 3: with a capacity c the buffer
    is [e, c, m] and routes whose slot is >= c are dropped; tokens then move
    through their capacity slots. [DS-8213] first commit and the review on
    trimming rows by the prefix sum: without a capacity the buffer holds the
    s*k routes grouped by expert, each expert's segment starting at the
    exclusive prefix sum of the per-expert counts.

    route_major: slots are handed to every token's first route, then every
    token's second route, and so on (the per-route masks mask1, mask2, ... of
    the same review comment, each cumsum offset by the counts of the earlier
    routes: first choices win capacity before second choices).
    pad_multiple (dropless only): each expert's segment is rounded up to a
    multiple of rows, as a grouped GEMM with fixed row tiles wants; the buffer
    then has s*k + e*(pad_multiple-1) rows and the unused ones are padding
    (NeMo Automodel PR on layout reuse, section 1: a pad multiple fixed at
    construction).
    """
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    s, k = idx.shape
    if pad_multiple < 1 or (pad_multiple > 1 and capacity > 0):
        raise ValueError("pad_multiple must be >= 1, and 1 with a capacity")
    valid, flags = route_validity(idx, e)
    tt, jj = np.nonzero(valid)
    xx = idx[tt, jj].astype(np.int64)

    slot = np.full((s, k), -1, dtype=np.int64)
    if not route_major:
        mask = np.zeros((s, e), dtype=np.int64)
        mask[tt, xx] = 1
        locations = np.cumsum(mask, axis=0) - 1  # cumsum-minus-one, token order
        slot[tt, jj] = locations[tt, xx]
        counts = mask.sum(axis=0).astype(np.int64)
    else:
        earlier = np.zeros(e, dtype=np.int64)  # routes of earlier columns per expert
        for j in range(k):
            sel = valid[:, j]
            mask_j = np.zeros((s, e), dtype=np.int64)
            mask_j[np.nonzero(sel)[0], idx[sel, j].astype(np.int64)] = 1
            loc_j = np.cumsum(mask_j, axis=0) - 1 + earlier[None, :]
            rows_j = np.nonzero(sel)[0]
            slot[rows_j, j] = loc_j[rows_j, idx[sel, j].astype(np.int64)]
            earlier += mask_j.sum(axis=0)
        counts = earlier

    dst = np.full((s, k), -1, dtype=np.int64)
    if capacity > 0:
        rows = e * capacity
        keep = slot[tt, jj] < capacity
        dst[tt[keep], jj[keep]] = xx[keep] * capacity + slot[tt[keep], jj[keep]]
        kept = np.minimum(counts, capacity)
        offsets = np.arange(e + 1, dtype=np.int64) * capacity
    else:
        rows = s * k + e * (pad_multiple - 1)
        seg = -(-counts // pad_multiple) * pad_multiple
        offsets = np.concatenate([[0], np.cumsum(seg)])
        dst[tt, jj] = offsets[xx] + slot[tt, jj]
        kept = counts.copy()

    src = np.full(rows, -1, dtype=np.int64)
    placed = dst >= 0
    src[dst[placed]] = np.nonzero(placed)[0]
    return Layout(
        s=s, e=e, k=k, capacity=capacity if capacity > 0 else 0, rows=rows,
        idx=idx.copy(), counts=counts.astype(np.int32), kept=kept.astype(np.int32),
        offsets=offsets.astype(np.int32), dst=dst.astype(np.int32), src=src.astype(np.int32),
        flags=flags, checksum=routing_checksum(idx),
    )


# ----------------------------------------------------------------------------
# steps 3 and 4: dispatch and weighted combine


def dispatch(layout: Layout, x: np.ndarray) -> np.ndarray:
    """Copy each token's row into the buffer row of every placed route.

    [DS-8195] part 3: tokens are routed through their capacity slots directly;
    unused capacity rows stay zero. [DS-8213] first commit: tokens are taken
    before top-k expansion and replicated to each selected expert. A bit copy:
    no arithmetic touches the values.
    """
    s, k = layout.s, layout.k
    out = np.zeros((layout.rows,) + x.shape[1:], dtype=x.dtype)
    placed = layout.dst >= 0
    tok = np.broadcast_to(np.arange(s)[:, None], (s, k))
    out[layout.dst[placed]] = x[tok[placed]]
    return out


def dispatch_replay(layout: Layout, x: np.ndarray, idx: np.ndarray | None = None):
    """Dispatch from a saved layout, without rebuilding it.

    [AM-3684] section 1, "How": the recompute consumes the forward's saved
    handle instead of recomputing the layout; if the routing handed in differs
    from the routing the layout was built on, that is reported, not hidden.
    Returns (buffer, flags).
    """
    flags = layout.flags
    if idx is not None and not np.array_equal(np.asarray(idx, np.int32), layout.idx):
        flags |= FLAG_REPLAY_MISMATCH
    return dispatch(layout, x), flags


def _route_sum(layout: Layout, rows32: np.ndarray, w: np.ndarray | None) -> np.ndarray:
    """acc[t] = sum over placed routes j (in order) of w[t,j]*rows32[dst[t,j]], in float32."""
    s, k = layout.s, layout.k
    acc = np.zeros((s,) + rows32.shape[1:], dtype=np.float32)
    for j in range(k):
        sel = layout.dst[:, j] >= 0
        r = layout.dst[sel, j]
        term = rows32[r]
        if w is not None:
            term = np.asarray(w, np.float32)[sel, j][:, None] * term  # float32 product
        acc[sel] = acc[sel] + term  # float32 add, separate from the product
    return acc


def combine(layout: Layout, expert_out: np.ndarray, w: np.ndarray, dtype: str) -> np.ndarray:
    """y[t] = sum_j w[t,j] * E[dst[t,j]] over placed routes, float32 accumulation.

    [DS-8195] part 3: combine accumulates in fp32, as the dense einsum did.
    [DS-8213] first commit and the review thread on combine weights: combine
    reduces the weighted sum, so the weights are applied here. Dropped routes
    add nothing; a token with every route dropped gets a zero row.
    """
    acc = _route_sum(layout, to_f32(expert_out, dtype), w)
    return from_f32(acc, dtype)


# ----------------------------------------------------------------------------
# step 5: backward


def combine_backward(layout: Layout, grad_y: np.ndarray, expert_out: np.ndarray,
                     w: np.ndarray, dtype: str) -> tuple[np.ndarray, np.ndarray]:
    """Gradients of combine: a weighted dispatch of grad_y, and the weight gradient.

    [DS-8213] first commit: combine and dispatch are adjoint, so this backward is a
    weighted dispatch on the same handle. grad_E[dst[t,j]] = w[t,j] * grad_y[t] (float32 product, rounded to
    the element type), rows no route points to are zero. [DS-8213] review-fix
    commit: the weights' gradient grad_w[t,j] = <grad_y[t], E[dst[t,j]]> must be
    returned (zero for a dropped route).
    """
    s, k = layout.s, layout.k
    gy32 = to_f32(grad_y, dtype)
    e32 = to_f32(expert_out, dtype)
    gE = zeros((layout.rows,) + grad_y.shape[1:], dtype)
    gw = np.zeros((s, k), np.float32)
    w32 = np.asarray(w, np.float32)
    for j in range(k):
        sel = layout.dst[:, j] >= 0
        r = layout.dst[sel, j]
        gE[r] = from_f32(w32[sel, j][:, None] * gy32[sel], dtype)
        dots = (gy32[sel].astype(np.float64) * e32[r].astype(np.float64)).sum(axis=1)
        gw[sel, j] = dots.astype(np.float32)
    return gE, gw


def dispatch_backward(layout: Layout, grad_out: np.ndarray, dtype: str) -> np.ndarray:
    """Gradient of dispatch: an unweighted combine of the buffer gradient.

    [DS-8213] first commit: by the same adjointness this backward is an unweighted
    combine on the same handle. grad_x[t] = sum over placed routes of grad_out[dst[t,j]], float32
    in route order, rounded once.
    """
    acc = _route_sum(layout, to_f32(grad_out, dtype), None)
    return from_f32(acc, dtype)


# ----------------------------------------------------------------------------
# variants: weights applied at dispatch, renormalisation over kept routes


def dispatch_weighted(layout: Layout, x: np.ndarray, w: np.ndarray, dtype: str) -> np.ndarray:
    """Dispatch with the routing weight applied to each copy (weights before the experts).

    [DS-8213] review thread on combine weights and the commit that applies them:
    the weights are applied either before or after the expert MLP (score_apply).
    Before: out[dst[t,j]] = w[t,j] * x[t], a float32 product rounded to the
    element type; the combine that follows is then unweighted.
    """
    out = zeros((layout.rows,) + x.shape[1:], dtype)
    x32 = to_f32(x, dtype)
    w32 = np.asarray(w, np.float32)
    for j in range(layout.k):
        sel = layout.dst[:, j] >= 0
        out[layout.dst[sel, j]] = from_f32(w32[sel, j][:, None] * x32[sel], dtype)
    return out


def dispatch_weighted_backward(layout: Layout, grad_out: np.ndarray, x: np.ndarray,
                               w: np.ndarray, dtype: str) -> tuple[np.ndarray, np.ndarray]:
    """Gradients of the weighted dispatch: a weighted combine, and the weight gradient.

    grad_x[t] = sum over placed routes j, in order, of w[t,j] * grad_out[dst[t,j]]
    (float32, separate multiply and add, rounded once); grad_w[t,j] =
    <grad_out[dst[t,j]], x[t]> in float64, rounded once (0 for a dropped route).
    """
    s, k = layout.s, layout.k
    g32 = to_f32(grad_out, dtype)
    gx = from_f32(_route_sum(layout, g32, w), dtype)
    x32 = to_f32(x, dtype)
    gw = np.zeros((s, k), np.float32)
    for j in range(k):
        sel = layout.dst[:, j] >= 0
        dots = (x32[sel].astype(np.float64) * g32[layout.dst[sel, j]].astype(np.float64)).sum(axis=1)
        gw[sel, j] = dots.astype(np.float32)
    return gx, gw


def renormalize_kept(layout: Layout, w: np.ndarray) -> np.ndarray:
    """Weights renormalised over each token's kept routes after the capacity drop.

    w'[t,j] = w[t,j] / S_t for kept routes, S_t = sum of the token's kept weights
    (float64 in route order); 0 for dropped routes, and 0 everywhere if none is
    kept. Rounded once to float32. (The alternative reading of where the
    renormalisation sits relative to the drop.) Sums run in route order.
    """
    w64 = np.asarray(w, np.float32).astype(np.float64)
    kept = layout.dst >= 0
    S = _route_order_sum(np.where(kept, w64, 0.0))
    safe = np.where(S != 0, S, 1.0)
    return np.where(kept & (S != 0), w64 / safe, 0.0).astype(np.float32)


def _route_order_sum(a64: np.ndarray) -> np.ndarray:
    """Row sums in float64, adding the k columns in route order j = 0..k-1."""
    acc = np.zeros((a64.shape[0], 1), np.float64)
    for j in range(a64.shape[1]):
        acc[:, 0] = acc[:, 0] + a64[:, j]
    return acc


def renormalize_kept_backward(layout: Layout, w: np.ndarray, grad_out: np.ndarray) -> np.ndarray:
    """Gradient of renormalize_kept with respect to the original weights.

    With u_j = w_j / S over kept routes: grad_w_i = (g_i - sum_q u_q g_q) / S for
    kept i, and 0 for dropped i (float64, rounded once).
    """
    w64 = np.asarray(w, np.float32).astype(np.float64)
    g64 = np.asarray(grad_out, np.float32).astype(np.float64)
    kept = layout.dst >= 0
    S = _route_order_sum(np.where(kept, w64, 0.0))
    safe = np.where(S != 0, S, 1.0)
    u = np.where(kept, w64 / safe, 0.0)
    dot = _route_order_sum(np.where(kept, u * g64, 0.0))
    return np.where(kept & (S != 0), (g64 - dot) / safe, 0.0).astype(np.float32)


# ----------------------------------------------------------------------------
# the grouped expert GEMM that consumes the layout


def expert_gemm(layout: Layout, a: np.ndarray, weights: np.ndarray, dtype: str, gather: bool,
                route_w: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Per-expert projection of the buffer rows, with the dispatch optionally fused in.

    For expert x and each placed row r of its segment:
        out[r] = A(r) @ weights[x]^T,  A(r) = a[src[r]] if gather else a[r]
    weights: [e, n, m] (output features x input features). The products are summed
    exactly (float64 of float32-widened operands, one matmul per expert), rounded to
    float32 as a float32 accumulator would hold them, optionally scaled by the route's
    weight (a float32 product: weights applied after the experts), and rounded once to
    the element type. Rows no route fills are zero.
    [DS-8213] review-fix commit: the grouped GEMM takes its row groups from the per-
    expert offsets (counts = differences of the prefix sum) and ignores rows past them;
    the dispatch is fused into its operand loads here instead of materialising the
    permuted buffer ([DS-8213] first commit: arrivals grouped by expert for the grouped
    GEMM).
    Returns (out, exact): exact holds the float64 sums (for tolerance checks).
    """
    e, n, m = weights.shape
    a32 = to_f32(a, dtype).astype(np.float64)
    exact = np.zeros((layout.rows, n), np.float64)
    row_w = np.ones(layout.rows, np.float32)
    if route_w is not None:
        placed = layout.dst >= 0
        row_w[layout.dst[placed]] = np.asarray(route_w, np.float32)[placed]
    for x in range(layout.e):
        r0 = int(layout.offsets[x])
        r1 = r0 + int(layout.kept[x])
        if r1 == r0:
            continue
        rows = np.arange(r0, r1)
        lhs = a32[layout.src[rows]] if gather else a32[rows]
        w64 = to_f32(weights[x], dtype).astype(np.float64)  # [n, m], one expert at a time
        exact[rows] = lhs @ w64.T
    acc32 = exact.astype(np.float32)
    if route_w is not None:
        acc32 = row_w[:, None] * acc32  # float32 product
    out = from_f32(acc32, dtype)
    out[layout.src < 0] = 0
    return out, exact


def expert_gemm_dgrad(layout: Layout, grad_out: np.ndarray, weights: np.ndarray,
                      dtype: str) -> tuple[np.ndarray, np.ndarray]:
    """Gradient of the grouped expert GEMM with respect to its input rows.

    With out[r] = A(r) @ weights[x]^T for the placed rows r of expert x (expert_gemm),
        grad_A[r] = grad_out[r] @ weights[x]          [rows, m]
    for those rows, and zero for rows no route fills. The gradient of the token rows x
    is then the dispatch backward of grad_A (each token sums its routes' rows), the same
    route-order sum as every other dispatch backward. The sums are exact (float64), rounded
    to float32 as a float32 accumulator holds them, then once to the element type.
    [DS-8213] first commit: the backward runs through the forward's handle (dispatch and
    combine are adjoint);
    review-fix commit: the groups are the offsets' segments.
    Returns (grad_A, exact float64).
    """
    e, n, m = weights.shape
    g64 = to_f32(grad_out, dtype).astype(np.float64)
    exact = np.zeros((layout.rows, m), np.float64)
    for x in range(layout.e):
        r0 = int(layout.offsets[x])
        r1 = r0 + int(layout.kept[x])
        if r1 == r0:
            continue
        w64 = to_f32(weights[x], dtype).astype(np.float64)  # [n, m]
        exact[r0:r1] = g64[r0:r1] @ w64
    out = from_f32(exact.astype(np.float32), dtype)
    out[layout.src < 0] = 0
    return out, exact

def expert_gemm_wgrad(layout: Layout, a: np.ndarray, grad_out: np.ndarray, dtype: str,
                      gather: bool, out_dtype: str = "f32") -> tuple[np.ndarray, np.ndarray]:
    """Gradient of the grouped expert GEMM with respect to its weights.

    With out[r] = A(r) @ weights[x]^T for the placed rows r of expert x (expert_gemm),
        grad_weights[x] = sum over those rows r of outer(grad_out[r], A(r)),
    an [n, m] matrix per expert; A(r) = a[src[r]] if gather else a[r], so the rows are
    gathered straight from the token rows here too. Experts with no placed row get zeros.
    The sums are exact (float64 of float32-widened operands, one matmul per expert) and
    rounded once to float32 (weight gradients are usually kept in float32); with
    out_dtype equal to dtype that float32 value is then rounded to nearest even in the
    element type, for gradients kept in the weights' own type.
    [DS-8213] review-fix commit: the groups are the offsets' segments; rows past them are
    in no group. First commit: the backward of the expert step replays the same grouping.
    Returns (grad_weights [e, n, m] of out_dtype, exact float64 [e, n, m]).
    """
    if out_dtype not in ("f32", dtype):
        raise ValueError(f"out_dtype must be f32 or {dtype}")
    n = grad_out.shape[1]
    m = a.shape[1]
    a32 = to_f32(a, dtype).astype(np.float64)
    g64 = to_f32(grad_out, dtype).astype(np.float64)
    exact = np.zeros((layout.e, n, m), np.float64)
    for x in range(layout.e):
        r0 = int(layout.offsets[x])
        r1 = r0 + int(layout.kept[x])
        if r1 == r0:
            continue
        rows = np.arange(r0, r1)
        lhs = a32[layout.src[rows]] if gather else a32[rows]
        exact[x] = g64[rows].T @ lhs
    return from_f32(exact.astype(np.float32), out_dtype), exact
