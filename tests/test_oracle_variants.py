"""Pins for the oracle's variant functions: route-major capacity priority, padded
dropless segments, weights applied at dispatch, renormalisation over kept routes."""
import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings, strategies as st

import oracle
import workloads as W
from tests.test_oracle_pins import dense_masks


def brute_layout_general(idx, e, capacity, route_major, pad):
    """Walk routes in (route, token) order if route_major, else (token, route)."""
    s, k = idx.shape
    order = [(t, j) for j in range(k) for t in range(s)] if route_major else \
            [(t, j) for t in range(s) for j in range(k)]
    seen = [0] * e
    slot = {}
    for t, j in order:
        x = int(idx[t, j])
        if not 0 <= x < e or x in [int(v) for v in idx[t, :j]]:
            continue
        slot[(t, j)] = seen[x]
        seen[x] += 1
    if capacity > 0:
        base = [x * capacity for x in range(e + 1)]
        rows = e * capacity
    else:
        base = [0]
        for c in seen:
            base.append(base[-1] + -(-c // pad) * pad)
        rows = s * k + e * (pad - 1)
    dst = -np.ones((s, k), np.int64)
    src = -np.ones(rows, np.int64)
    for (t, j), q in slot.items():
        if capacity > 0 and q >= capacity:
            continue
        dst[t, j] = base[int(idx[t, j])] + q
        src[dst[t, j]] = t
    return dict(counts=seen, offsets=base, dst=dst, src=src, rows=rows)


@settings(max_examples=120, deadline=None)
@given(s=st.integers(0, 40), e=st.integers(1, 10), kk=st.integers(1, 6), cap=st.integers(-1, 9),
       rm=st.booleans(), pad=st.sampled_from([1, 2, 3, 8]), seed=st.integers(0, 2**31 - 1))
def test_layout_options_match_brute_force(s, e, kk, cap, rm, pad, seed):
    k = min(kk, e)
    if cap > 0:
        pad = 1
    idx = W.random_idx(np.random.default_rng(seed), s, e, k)
    L = oracle.dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
    B = brute_layout_general(idx, e, cap, rm, pad)
    assert L.rows == B["rows"]
    assert L.counts.tolist() == B["counts"]
    assert L.offsets.tolist() == B["offsets"]
    assert np.array_equal(L.dst, B["dst"])
    assert np.array_equal(L.src, B["src"])
    if cap <= 0:
        assert np.all(L.offsets % pad == 0)
        assert np.all(L.offsets[1:] - L.offsets[:-1] >= L.counts)


def test_route_major_gives_first_choices_priority():
    """GShard priority: an expert at capacity keeps first choices before second ones."""
    rng = np.random.default_rng(4)
    s, e, k, cap = 400, 4, 2, 60
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, cap, route_major=True)
    for x in range(e):
        first = (idx[:, 0] == x)
        second = (idx[:, 1] == x)
        kept_first = (L.dst[:, 0] >= 0) & first
        kept_second = (L.dst[:, 1] >= 0) & second
        if kept_second.any():
            assert kept_first.sum() == first.sum()  # every first choice fits before any second
        assert kept_first.sum() + kept_second.sum() == min(cap, first.sum() + second.sum())
    # token order differs from route-major as soon as a capacity binds
    T = oracle.dispatch_layout(idx, e, cap)
    assert not np.array_equal(T.dst, L.dst)


def test_route_major_without_drops_only_reorders_segments():
    rng = np.random.default_rng(5)
    idx = W.random_idx(rng, 200, 6, 3)
    T = oracle.dispatch_layout(idx, 6, 0)
    R = oracle.dispatch_layout(idx, 6, 0, route_major=True)
    assert np.array_equal(T.offsets, R.offsets)
    for x in range(6):
        seg_t = T.src[T.offsets[x]:T.offsets[x + 1]]
        seg_r = R.src[R.offsets[x]:R.offsets[x + 1]]
        assert sorted(seg_t.tolist()) == sorted(seg_r.tolist())


# ----------------------------------------------------------------------------
# weights applied at dispatch


@pytest.mark.parametrize("cap", [0, 5])
def test_weighted_dispatch_matches_dense_einsum(cap):
    rng = np.random.default_rng(50 + cap)
    s, e, k, m = 30, 5, 3, 6
    idx = W.random_idx(rng, s, e, k)
    x = rng.standard_normal((s, m)).astype(np.float32)
    w = W.random_weights(rng, s, k)
    L = oracle.dispatch_layout(idx, e, cap)
    D, C = dense_masks(L, w)
    ref = np.einsum("sec,sm->ecm", C, x.astype(np.float64))
    out = oracle.dispatch_weighted(L, x, w, "f32").astype(np.float64)
    for xx in range(e):
        n = int(L.kept[xx])
        seg = out[L.offsets[xx]:L.offsets[xx] + n]
        assert np.all(np.abs(seg - ref[xx, :n]) <= np.spacing(np.abs(ref[xx, :n]).astype(np.float32)))


def test_weights_before_or_after_experts_agree_in_float32():
    """Unweighted sum of weighted copies == weighted sum of plain copies, bit for bit in f32."""
    rng = np.random.default_rng(6)
    s, e, k, m = 80, 7, 4, 10
    idx = W.random_idx(rng, s, e, k)
    x = rng.standard_normal((s, m)).astype(np.float32)
    w = W.random_weights(rng, s, k)
    for cap in (0, 9):
        L = oracle.dispatch_layout(idx, e, cap)
        before = oracle.dispatch_backward(L, oracle.dispatch_weighted(L, x, w, "f32"), "f32")
        after = oracle.combine(L, oracle.dispatch(L, x), w, "f32")
        assert np.array_equal(before, after)


@pytest.mark.parametrize("cap", [0, 4])
def test_weighted_dispatch_backward_adjoint_and_finite_difference(cap):
    rng = np.random.default_rng(70 + cap)
    s, e, k, m = 24, 5, 3, 7
    idx = W.random_idx(rng, s, e, k)
    x = rng.standard_normal((s, m)).astype(np.float32)
    w = W.random_weights(rng, s, k)
    L = oracle.dispatch_layout(idx, e, cap)
    G = rng.standard_normal((L.rows, m)).astype(np.float32)
    gx, gw = oracle.dispatch_weighted_backward(L, G, x, w, "f32")
    out = oracle.dispatch_weighted(L, x, w, "f32").astype(np.float64)
    lhs = float(np.sum(out * G))
    rhs = float(np.sum(x.astype(np.float64) * gx))
    mag = float(np.sum(np.abs(out * G)))
    assert abs(lhs - rhs) <= 4 * k * 2.0 ** -23 * mag
    def loss(wv):
        _, C = dense_masks(L, wv)
        ecm = np.einsum("sec,sm->ecm", C, x.astype(np.float64))
        rows = np.zeros((L.rows, m))
        for xx in range(e):
            n = int(L.kept[xx])
            rows[L.offsets[xx]:L.offsets[xx] + n] = ecm[xx, :n]
        return float(np.sum(rows * G))

    h = 1e-3
    for t in range(s):
        for j in range(k):
            wp = w.astype(np.float64).copy()
            wm = wp.copy()
            wp[t, j] += h
            wm[t, j] -= h
            fd = (loss(wp) - loss(wm)) / (2 * h)
            if L.dst[t, j] < 0:
                assert gw[t, j] == 0
            assert abs(gw[t, j] - fd) <= 1e-9 + 1e-6 * abs(fd)


# ----------------------------------------------------------------------------
# renormalisation over kept routes


def test_renormalized_gate_weights_are_softmax_over_kept_logits():
    rng = np.random.default_rng(8)
    s, e, k, cap = 500, 6, 3, 120
    logits = rng.standard_normal((s, e)).astype(np.float32)
    logits[:, 0] += 1.5  # make expert 0 overflow
    idx, w = oracle.gate_topk(logits, k)
    L = oracle.dispatch_layout(idx, e, cap)
    assert (L.dst < 0).any()
    wr = oracle.renormalize_kept(L, w)
    for t in range(s):
        kept = L.dst[t] >= 0
        if not kept.any():
            assert np.all(wr[t] == 0)
            continue
        ref = scipy.special.softmax(logits[t, idx[t, kept]].astype(np.float64))
        assert np.all(np.abs(wr[t, kept] - ref) <= 2 * np.spacing(ref.astype(np.float32)))
        assert np.all(wr[t, ~kept] == 0)


def test_renormalize_backward_matches_finite_differences_through_the_gate():
    rng = np.random.default_rng(9)
    s, e, k, cap = 60, 5, 3, 14
    logits = rng.standard_normal((s, e)).astype(np.float32)
    idx, w = oracle.gate_topk(logits, k)
    L = oracle.dispatch_layout(idx, e, cap)
    g = rng.standard_normal((s, k)).astype(np.float32)
    gl = oracle.gate_topk_backward(idx, w, oracle.renormalize_kept_backward(L, w, g), e)
    h = 1e-6
    for t in range(s):
        kept = L.dst[t] >= 0
        sel = idx[t, kept].astype(np.int64)

        def f(lv):
            return float(np.dot(g[t, kept].astype(np.float64), scipy.special.softmax(lv[sel]))) if len(sel) else 0.0

        base = logits[t].astype(np.float64)
        for i in range(e):
            lp, lm = base.copy(), base.copy()
            lp[i] += h
            lm[i] -= h
            fd = (f(lp) - f(lm)) / (2 * h)
            assert abs(gl[t, i] - fd) <= 1e-6 + 1e-5 * abs(fd)


def test_renormalize_all_dropped_is_zero():
    idx = np.array([[0, 1], [0, 1], [1, 0]], np.int32)
    L = oracle.dispatch_layout(idx, 2, 1)
    w = np.array([[0.7, 0.3], [0.6, 0.4], [0.5, 0.5]], np.float32)
    wr = oracle.renormalize_kept(L, w)
    assert np.array_equal(wr[0], w[0])  # token 0 keeps both routes; their sum is exactly 1
    assert np.all(wr[1] == 0) and np.all(wr[2] == 0)
    gw = oracle.renormalize_kept_backward(L, w, np.ones_like(w))
    assert np.all(gw[1:] == 0)
