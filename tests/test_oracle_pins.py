"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

None of these re-run the oracle's own formula. Each compares it with something
independent of it: a hand-worked fixture, a brute-force loop on tiny inputs,
the dense one-hot einsum the index path replaced (DeepSpeed PR "MoE dispatch:
fix silent Tutel + TP corruption, speed up native and Tutel paths", part 3 and
its Testing section), a library softmax, finite differences, adjoint
identities, or an exact closed form.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_small.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# independent helpers (brute force), written for the tests only


def brute_layout(idx, e, capacity):
    """Route-by-route walk in token order: each route's slot is the number of
    earlier tokens already sent to the same expert."""
    s, k = idx.shape
    seen = [0] * e
    slot = {}
    bad = 0
    for t in range(s):
        taken = []
        for j in range(k):
            x = int(idx[t, j])
            if not 0 <= x < e:
                bad |= 1
                continue
            if x in taken:
                bad |= 2
                continue
            taken.append(x)
            slot[(t, j)] = seen[x]
            seen[x] += 1
    counts = seen
    if capacity > 0:
        rows = e * capacity
        base = [x * capacity for x in range(e + 1)]
        kept = [min(c, capacity) for c in counts]
    else:
        rows = s * k
        base = [0]
        for c in counts:
            base.append(base[-1] + c)
        kept = list(counts)
    dst = -np.ones((s, k), np.int64)
    src = -np.ones(rows, np.int64)
    for (t, j), q in slot.items():
        x = int(idx[t, j])
        if capacity > 0 and q >= capacity:
            continue
        dst[t, j] = base[x] + q
        src[base[x] + q] = t
    return dict(counts=counts, kept=kept, offsets=base, dst=dst, src=src, rows=rows, flags=bad)


def dense_masks(layout, w):
    """The old path's dense dispatch mask ([s, e, c], one-hot) and its combine weights."""
    s, k, e = layout.s, layout.k, layout.e
    if layout.capacity > 0:
        c = layout.capacity
    else:
        c = max(1, int(layout.counts.max()) if e else 1)
    D = np.zeros((s, e, c), np.float64)
    C = np.zeros((s, e, c), np.float64)
    for t in range(s):
        for j in range(k):
            r = int(layout.dst[t, j])
            if r < 0:
                continue
            x = int(layout.idx[t, j])
            q = r - int(layout.offsets[x])
            D[t, x, q] = 1.0
            C[t, x, q] = float(w[t, j])
    return D, C


def dense_to_rows(layout, ecm):
    """Map a dense [e, c, m] result to the layout's buffer rows."""
    m = ecm.shape[2]
    out = np.zeros((layout.rows, m), np.float64)
    for x in range(layout.e):
        n = int(layout.kept[x])
        base = int(layout.offsets[x])
        out[base:base + n] = ecm[x, :n]
    return out


def ulp32(v):
    v = np.abs(np.asarray(v, np.float32))
    return np.spacing(v).astype(np.float64)


# ----------------------------------------------------------------------------
# hand-worked fixture


def test_golden_layout():
    g = golden()["layout"]
    idx = np.array(g["idx"], np.int32)
    for case in g["cases"]:
        L = oracle.dispatch_layout(idx, g["e"], case["capacity"])
        assert L.rows == case["rows"]
        assert L.counts.tolist() == g["counts"]
        assert L.kept.tolist() == case["kept"]
        assert L.offsets.tolist() == case["offsets"]
        assert L.dst.tolist() == case["dst"]
        assert L.src.tolist() == case["src"]
        assert L.checksum == g["checksum"]
        assert L.flags == 0


def test_golden_combine_and_backward():
    g = golden()
    idx = np.array(g["layout"]["idx"], np.int32)
    c = g["combine"]
    x = np.array(c["x"], np.float32)
    w = np.array(c["w"], np.float32)
    gy = np.array(c["grad_y"], np.float32)
    for case in c["cases"]:
        L = oracle.dispatch_layout(idx, g["layout"]["e"], case["capacity"])
        E = oracle.dispatch(L, x)
        assert oracle.combine(L, E, w, "f32").tolist() == case["y"]
        ones = np.ones_like(w)
        assert oracle.combine(L, E, ones, "f32").tolist() == case["y_unit_weights"]
        gE, gw = oracle.combine_backward(L, gy, E, w, "f32")
        assert gw.tolist() == case["grad_w"]
        assert gE.tolist() == case["grad_E"]
        assert oracle.dispatch_backward(L, gE, "f32").tolist() == case["grad_x"]


def test_golden_gate():
    g = golden()["gate"]
    for case in g["cases"]:
        logits = np.array([case["logits"]], np.float32)
        idx, w = oracle.gate_topk(logits, case["k"])
        assert idx[0].tolist() == case["idx"]
        assert w[0].tolist() == case["w"]
    b = g["backward"]
    gl = oracle.gate_topk_backward(np.array([b["idx"]], np.int32), np.array([b["w"]], np.float32),
                                   np.array([b["grad_w"]], np.float32), b["e"])
    assert gl[0].tolist() == b["grad_logits"]


# ----------------------------------------------------------------------------
# gate


def brute_topk(row, k):
    return sorted(range(len(row)), key=lambda i: (-float(row[i]), i))[:k]


@pytest.mark.parametrize("seed", range(6))
def test_gate_indices_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    s, e = 40, 11
    # small integer logits force many ties; include signed zeros
    logits = rng.integers(-3, 4, size=(s, e)).astype(np.float32)
    logits[rng.random((s, e)) < 0.1] = -0.0
    for k in (1, 2, 5, e):
        idx, _ = oracle.gate_topk(logits, k)
        for t in range(s):
            assert idx[t].tolist() == brute_topk(logits[t], k)


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_gate_weights_against_library_softmax(k):
    rng = np.random.default_rng(10 + k)
    s, e = 64, 16
    logits = (rng.standard_normal((s, e)) * 3).astype(np.float32)
    idx, w = oracle.gate_topk(logits, k)
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    ref = scipy.special.softmax(sel, axis=1)  # softmax over the k selected logits
    assert np.all(np.abs(w.astype(np.float64) - ref) <= ulp32(ref))
    if k == 1:
        assert np.all(w == 1.0)
    # descending weights, summing to one within float32 rounding
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -24)


def test_gate_weights_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((32, 9)).astype(np.float32)
    idx, w = oracle.gate_topk(logits, 9)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    ref = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    assert np.all(np.abs(w - ref) <= ulp32(ref))


def test_gate_backward_finite_differences():
    rng = np.random.default_rng(7)
    s, e, k = 12, 10, 4
    logits = rng.standard_normal((s, e)).astype(np.float32)
    idx, w = oracle.gate_topk(logits, k)
    gw = rng.standard_normal((s, k)).astype(np.float32)
    gl = oracle.gate_topk_backward(idx, w, gw, e)
    h = 1e-6
    for t in range(s):
        sel = idx[t].astype(np.int64)
        base = logits[t].astype(np.float64)

        def f(lv):
            return float(np.dot(gw[t].astype(np.float64), scipy.special.softmax(lv[sel])))

        for i in range(e):
            lp, lm = base.copy(), base.copy()
            lp[i] += h
            lm[i] -= h
            fd = (f(lp) - f(lm)) / (2 * h)
            if i not in sel:
                assert gl[t, i] == 0.0
            assert abs(gl[t, i] - fd) <= 1e-6 + 1e-5 * abs(fd)


# ----------------------------------------------------------------------------
# layout


def check_layout_invariants(L, idx):
    s, k = idx.shape
    placed = L.dst >= 0
    assert int(L.counts.sum()) <= s * k
    assert np.array_equal(L.kept, np.minimum(L.counts, L.capacity) if L.capacity else L.counts)
    assert int(placed.sum()) == int(L.kept.sum())
    # src is the inverse of dst
    tok = np.broadcast_to(np.arange(s)[:, None], (s, k))
    assert np.array_equal(L.src[L.dst[placed]], tok[placed])
    assert int((L.src >= 0).sum()) == int(placed.sum())
    # each expert's placed rows are a prefix of its segment, in token order
    for x in range(L.e):
        seg = L.src[L.offsets[x]:L.offsets[x] + L.kept[x]]
        assert np.all(seg >= 0)
        assert np.all(np.diff(seg) > 0)
        assert np.all(L.src[L.offsets[x] + L.kept[x]:L.offsets[x + 1]] == -1)
    if L.capacity == 0:
        assert L.offsets[-1] == L.counts.sum()


@settings(max_examples=150, deadline=None)
@given(s=st.integers(0, 40), e=st.integers(1, 12), kk=st.integers(1, 12),
       cap=st.integers(-1, 12), seed=st.integers(0, 2**31 - 1))
def test_layout_matches_brute_force(s, e, kk, cap, seed):
    k = min(kk, e)
    rng = np.random.default_rng(seed)
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, cap)
    B = brute_layout(idx, e, cap)
    assert L.rows == B["rows"]
    assert L.counts.tolist() == B["counts"]
    assert L.kept.tolist() == B["kept"]
    assert L.offsets.tolist() == B["offsets"]
    assert np.array_equal(L.dst, B["dst"])
    assert np.array_equal(L.src, B["src"])
    assert L.flags == 0
    check_layout_invariants(L, idx)


@settings(max_examples=80, deadline=None)
@given(s=st.integers(1, 30), e=st.integers(1, 8), k=st.integers(1, 6),
       cap=st.integers(0, 5), seed=st.integers(0, 2**31 - 1))
def test_layout_invalid_routes_flagged_and_skipped(s, e, k, cap, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-2, e + 2, size=(s, k)).astype(np.int32)
    L = oracle.dispatch_layout(idx, e, cap)
    B = brute_layout(idx, e, cap)
    assert L.flags == B["flags"]
    assert np.array_equal(L.dst, B["dst"])
    assert np.array_equal(L.src, B["src"])
    assert L.counts.tolist() == B["counts"]


def test_layout_skew_all_tokens_one_expert():
    rng = np.random.default_rng(0)
    s, e, k = 300, 16, 4
    idx = W.skewed_idx(rng, s, e, k, hot=5)
    for cap in (0, 1, 8, 40, 300):
        L = oracle.dispatch_layout(idx, e, cap)
        B = brute_layout(idx, e, cap)
        assert np.array_equal(L.dst, B["dst"])
        assert L.counts[5] == s
        if cap:
            assert L.kept[5] == min(s, cap)


def test_layout_checksum_orders_matter():
    idx = np.array([[0, 1], [2, 3]], np.int32)
    a = oracle.routing_checksum(idx)
    b = oracle.routing_checksum(idx[::-1].copy())
    c = oracle.routing_checksum(idx[:, ::-1].copy())
    assert a == 1 * 1 + 2 * 2 + 3 * 3 + 4 * 4
    assert b == 3 * 1 + 4 * 2 + 1 * 3 + 2 * 4
    assert c == 2 * 1 + 1 * 2 + 4 * 3 + 3 * 4
    # wraps modulo 2**64 and reads ids as signed
    assert oracle.routing_checksum(np.array([[-1]], np.int32)) == 0
    big = np.full((1, 1), 2**31 - 1, np.int32)
    assert oracle.routing_checksum(big) == 2**31


def test_layout_empty_and_degenerate():
    idx = np.zeros((0, 3), np.int32)
    L = oracle.dispatch_layout(idx, 5, 4)
    assert L.rows == 20 and np.all(L.src == -1) and L.counts.sum() == 0
    L = oracle.dispatch_layout(idx, 5, 0)
    assert L.rows == 0 and L.offsets.tolist() == [0] * 6
    # k == e: every token in every expert
    idx = np.tile(np.arange(4, dtype=np.int32)[::-1], (6, 1))
    L = oracle.dispatch_layout(idx, 4, 0)
    assert L.counts.tolist() == [6] * 4
    # capacity 1: only the first token reaches each expert
    L = oracle.dispatch_layout(idx, 4, 1)
    assert L.src.tolist() == [0, 0, 0, 0]


def test_replay_reproduces_layout_and_rows():
    rng = np.random.default_rng(5)
    idx = W.random_idx(rng, 100, 12, 3)
    x = rng.standard_normal((100, 8)).astype(np.float32)
    L1 = oracle.dispatch_layout(idx, 12, 20)
    L2 = oracle.dispatch_layout(idx.copy(), 12, 20)
    for f in ("counts", "kept", "offsets", "dst", "src"):
        assert np.array_equal(getattr(L1, f), getattr(L2, f))
    out, flags = oracle.dispatch_replay(L1, x, idx)
    assert flags == 0 and np.array_equal(out, oracle.dispatch(L2, x))
    other = idx.copy()
    other[3, 1] = (other[3, 1] + 1) % 12
    _, flags = oracle.dispatch_replay(L1, x, other)
    assert flags & oracle.FLAG_REPLAY_MISMATCH


# ----------------------------------------------------------------------------
# dispatch and combine against the dense one-hot einsum


@pytest.mark.parametrize("k,cap", [(1, 6), (2, 6), (3, 6), (2, 0), (3, 0), (3, 2)])
def test_index_path_matches_dense_einsum(k, cap):
    rng = np.random.default_rng(100 + k * 10 + cap)
    s, e, m = 24, 5, 7
    idx = W.random_idx(rng, s, e, k)
    x = rng.standard_normal((s, m)).astype(np.float32)
    w = W.random_weights(rng, s, k)
    L = oracle.dispatch_layout(idx, e, cap)
    D, C = dense_masks(L, w)
    out = oracle.dispatch(L, x)
    ref = dense_to_rows(L, np.einsum("sec,sm->ecm", D, x.astype(np.float64)))
    assert np.array_equal(out.astype(np.float64), ref)

    E = rng.standard_normal((L.rows, m)).astype(np.float32)
    ecm = np.zeros((e, D.shape[2], m))
    for xx in range(e):
        n = int(L.kept[xx])
        ecm[xx, :n] = E[L.offsets[xx]:L.offsets[xx] + n]
    y = oracle.combine(L, E, w, "f32").astype(np.float64)
    yref = np.einsum("sec,ecm->sm", C, ecm)
    bound = np.einsum("sec,ecm->sm", np.abs(C), np.abs(ecm))
    assert np.all(np.abs(y - yref) <= k * 2.0 ** -23 * bound + 1e-45)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("cap", [0, 3, 9])
def test_unit_weight_round_trip_is_exact(dtype, cap):
    """combine(dispatch(x), 1) equals each row times its kept-route count, exactly."""
    rng = np.random.default_rng(11)
    s, e, k, m = 50, 6, 3, 12
    idx = W.random_idx(rng, s, e, k)
    # values with few mantissa bits so the float32 sum of <= k copies is exact
    x32 = oracle.to_f32(W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16"), "bf16")
    x = W.cast_input(x32, dtype)
    L = oracle.dispatch_layout(idx, e, cap)
    y = oracle.combine(L, oracle.dispatch(L, x), np.ones((s, k), np.float32), dtype)
    kept_t = (L.dst >= 0).sum(axis=1)
    # "+ 0.0": a token with no kept route gets a +0 row, not 0 * (negative x) = -0
    exact = kept_t[:, None] * oracle.to_f32(x, dtype).astype(np.float64) + 0.0
    want = oracle.from_f32(exact.astype(np.float32), dtype)
    assert np.array_equal(y, want)


def test_combine_rounds_once_to_bf16():
    """The float32 sum is rounded once: compare with exact rational arithmetic."""
    rng = np.random.default_rng(2)
    s, e, k, m = 30, 4, 3, 16
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 0)
    E = W.cast_input(rng.standard_normal((L.rows, m)).astype(np.float32), "bf16")
    w = W.random_weights(rng, s, k)
    y = oracle.to_f32(oracle.combine(L, E, w, "bf16"), "bf16").astype(np.float64)
    E64 = oracle.to_f32(E, "bf16").astype(np.float64)
    exact = np.zeros((s, m))
    mag = np.zeros((s, m))
    for j in range(k):
        exact += w[:, j, None].astype(np.float64) * E64[L.dst[:, j]]
        mag += np.abs(w[:, j, None].astype(np.float64) * E64[L.dst[:, j]])
    # one bf16 rounding (half an ulp, 2**-9 relative) on top of a float32 sum
    err = np.abs(y - exact)
    assert np.all(err <= 2.0 ** -8 * np.abs(exact) + k * 2.0 ** -23 * mag + 1e-38)


# ----------------------------------------------------------------------------
# backward


@pytest.mark.parametrize("cap", [0, 2, 7])
def test_adjoint_identities(cap):
    rng = np.random.default_rng(21 + cap)
    s, e, k, m = 40, 6, 3, 9
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, cap)
    x = rng.standard_normal((s, m)).astype(np.float32)
    G = rng.standard_normal((L.rows, m)).astype(np.float32)
    # <dispatch(x), G> == <x, dispatch_backward(G)>
    lhs = float(np.sum(oracle.dispatch(L, x).astype(np.float64) * G))
    gx = oracle.dispatch_backward(L, G, "f32")
    rhs = float(np.sum(x.astype(np.float64) * gx))
    mag = float(np.sum(np.abs(oracle.dispatch(L, x).astype(np.float64) * G)))
    assert abs(lhs - rhs) <= k * 2.0 ** -23 * mag
    # <combine(E, w), gy> == <E, grad_E>
    E = rng.standard_normal((L.rows, m)).astype(np.float32)
    w = W.random_weights(rng, s, k)
    gy = rng.standard_normal((s, m)).astype(np.float32)
    lhs = float(np.sum(oracle.combine(L, E, w, "f32").astype(np.float64) * gy))
    gE, gw = oracle.combine_backward(L, gy, E, w, "f32")
    rhs = float(np.sum(E.astype(np.float64) * gE))
    mag = float(np.sum(np.abs(E.astype(np.float64) * gE)))
    assert abs(lhs - rhs) <= 2 * k * 2.0 ** -23 * mag
    # gradient rows nobody points at are zero
    assert np.all(gE[L.src < 0] == 0)


def test_weight_gradient_matches_finite_difference_of_dense_combine():
    rng = np.random.default_rng(31)
    s, e, k, m = 16, 5, 3, 6
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 4)
    E = rng.standard_normal((L.rows, m)).astype(np.float32)
    w = W.random_weights(rng, s, k)
    gy = rng.standard_normal((s, m)).astype(np.float32)
    _, gw = oracle.combine_backward(L, gy, E, w, "f32")
    cmax = L.capacity
    ecm = E.astype(np.float64).reshape(e, cmax, m)

    def loss(wv):
        _, C = dense_masks(L, wv)
        return float(np.sum(np.einsum("sec,ecm->sm", C, ecm) * gy))

    h = 1e-3
    for t, j in itertools.product(range(s), range(k)):
        wp, wm = w.astype(np.float64), w.astype(np.float64)
        wp = wp.copy(); wm = wm.copy()
        wp[t, j] += h
        wm[t, j] -= h
        fd = (loss(wp) - loss(wm)) / (2 * h)  # combine is linear in w: exact up to rounding
        if L.dst[t, j] < 0:
            assert gw[t, j] == 0.0
        assert abs(gw[t, j] - fd) <= 1e-9 + 1e-6 * abs(fd)


def test_identity_expert_closed_forms():
    rng = np.random.default_rng(41)
    s, e, k, m = 64, 8, 4, 10
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 0)
    x = rng.standard_normal((s, m)).astype(np.float32)
    w = W.random_weights(rng, s, k)
    gy = rng.standard_normal((s, m)).astype(np.float32)
    E = oracle.dispatch(L, x)
    gE, gw = oracle.combine_backward(L, gy, E, w, "f32")
    dots = (gy.astype(np.float64) * x.astype(np.float64)).sum(1)
    assert np.allclose(gw, dots[:, None].astype(np.float32), rtol=0, atol=0)
    gx = oracle.dispatch_backward(L, gE, "f32").astype(np.float64)
    want = w.astype(np.float64).sum(1)[:, None] * gy
    assert np.all(np.abs(gx - want) <= 2 * k * 2.0 ** -23 * np.abs(w).sum(1)[:, None] * np.abs(gy))


# ----------------------------------------------------------------------------
# element types


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(1)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.3895314e38,
                  np.finfo(np.float32).max, 1e-40, 0.0, -0.0], np.float32),
    ])
    r = oracle.to_f32(oracle.from_f32(a, "bf16"), "bf16").astype(np.float64)
    a64 = a.astype(np.float64)
    # candidates: truncation toward zero and the next bf16 away from zero
    u = a.view(np.uint32)
    lo = ((u >> 16) << 16).view(np.float32).astype(np.float64)
    hi = (((u >> 16) + 1) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    for v, got, l, h in zip(a64, r, lo, hi):
        # past the largest finite value, IEEE rounding measures against 2**128
        hv = math.copysign(2.0 ** 128, v) if math.isinf(h) else h
        dl, dh = abs(v - l), abs(hv - v)
        if dl < dh:
            assert got == l
        elif dh < dl:
            assert got == h
        else:  # tie: even mantissa
            el = int(np.float32(l).view(np.uint32) >> 16) & 1
            assert got == (l if el == 0 else h)
    assert oracle.from_f32(np.array([1.0 + 2.0 ** -8], np.float32), "bf16")[0] == 0x3F80
    assert oracle.from_f32(np.array([1.0 + 3 * 2.0 ** -8], np.float32), "bf16")[0] == 0x3F82
    assert oracle.from_f32(np.array([np.finfo(np.float32).max], np.float32), "bf16")[0] == 0x7F80


def test_workload_shapes():
    w = W.WORKLOADS["tiny_capacity_top2"]
    assert w.capacity == 80
    w = W.WORKLOADS["gshard_capacity_drop"]
    assert w.capacity == 1024
    assert w.rows == 64 * 1024
    assert W.WORKLOADS["zipf_skew_h4096"].rows == 65536
    assert math.isclose(W.WORKLOADS["checkpoint_replay_h2816"].rows, 262144)
