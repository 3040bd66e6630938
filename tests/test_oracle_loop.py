"""The loop oracle (plain per-element Python loops) against the vectorised oracle.

Two independent CPU implementations of the same definitions: ids, layouts and
buffers must be equal, float32 route-order sums bit-equal, and values formed in
float64 (gate weights, weight gradients, logit gradients) within one float32 ulp,
since the two sum float64 values in different orders. Small batches only.
"""
import numpy as np
import pytest

import oracle
import oracle.loop as LO
import workloads as W


def ulps(a, b):
    def key(v):
        u = np.ascontiguousarray(v, np.float32).view(np.int32).astype(np.int64)
        return np.where(u < 0, -(u & 0x7FFFFFFF), u)
    return np.abs(key(a) - key(b))


CASES = [
    # s, e, k, m, capacity, dtype, tie-prone logits
    (40, 6, 2, 8, 0, "f32", False),
    (40, 6, 2, 8, 5, "bf16", True),
    (33, 9, 4, 16, 0, "f16", True),
    (60, 4, 4, 8, 9, "bf16", False),
    (20, 12, 1, 8, 2, "f32", True),
    (1, 3, 3, 8, 0, "bf16", False),
]


@pytest.mark.parametrize("s,e,k,m,cap,dt,ties", CASES)
def test_loop_oracle_equals_vectorised_oracle(s, e, k, m, cap, dt, ties):
    rng = np.random.default_rng(s * 13 + e + k + cap)
    if ties:
        logits = (rng.integers(-2, 3, (s, e)) / 2).astype(np.float32)
        logits[rng.random((s, e)) < 0.2] = -0.0
    else:
        logits = rng.standard_normal((s, e)).astype(np.float32)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dt)
    gy = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dt)

    idx_l, w_l = LO.gate_topk(logits, k)
    idx_v, w_v = oracle.gate_topk(logits, k)
    assert np.array_equal(idx_l, idx_v)
    assert ulps(w_l, w_v).max() <= 1

    Ll = LO.dispatch_layout(idx_v, e, cap)
    Lv = oracle.dispatch_layout(idx_v, e, cap)
    arr = LO.layout_arrays(Ll)
    for f in ("counts", "kept", "offsets", "dst", "src"):
        assert np.array_equal(arr[f], getattr(Lv, f)), f
    assert (Ll.flags, Ll.checksum, Ll.rows) == (Lv.flags, Lv.checksum, Lv.rows)

    E_l = LO.dispatch(Ll, x)
    E_v = oracle.dispatch(Lv, x)
    assert np.array_equal(E_l.view(np.uint8), E_v.view(np.uint8))
    # expert rows that differ from the dispatched ones, so that a swapped row shows
    E = W.cast_input(rng.standard_normal((Lv.rows, m)).astype(np.float32), dt)
    assert np.array_equal(LO.combine(Ll, E, w_v, dt).view(np.uint8), oracle.combine(Lv, E, w_v, dt).view(np.uint8))
    gE_l, gw_l = LO.combine_backward(Ll, gy, E, w_v, dt)
    gE_v, gw_v = oracle.combine_backward(Lv, gy, E, w_v, dt)
    assert np.array_equal(gE_l.view(np.uint8), gE_v.view(np.uint8))
    assert ulps(gw_l, gw_v).max() <= 1
    assert np.array_equal(LO.dispatch_backward(Ll, gE_v, dt).view(np.uint8),
                          oracle.dispatch_backward(Lv, gE_v, dt).view(np.uint8))
    gl_l = LO.gate_topk_backward(idx_v, w_v, gw_v, e)
    gl_v = oracle.gate_topk_backward(idx_v, w_v, gw_v, e)
    assert np.array_equal(gl_l == 0, gl_v == 0)
    # float64 sums in different orders: one float32 ulp, or rounding noise where the
    # centred term cancels
    w64, g64 = w_v.astype(np.float64), gw_v.astype(np.float64)
    scale = np.zeros((s, e))
    np.put_along_axis(scale, idx_v.astype(np.int64),
                      np.abs(w64) * (np.abs(g64) + np.abs(w64 * g64).sum(1, keepdims=True)), axis=1)
    big = np.maximum(np.abs(gl_l.astype(np.float64)), np.abs(gl_v))
    ulp = np.ldexp(1.0, np.frexp(np.maximum(big, 2.0 ** -126))[1] - 24)
    assert np.all(np.abs(gl_l.astype(np.float64) - gl_v) <= ulp + 2.0 ** -45 * scale)


def test_loop_oracle_flags_invalid_routes():
    idx = np.array([[0, 0], [5, 1], [1, 2]], np.int32)
    Ll = LO.dispatch_layout(idx, 3, 0)
    Lv = oracle.dispatch_layout(idx, 3, 0)
    assert Ll.flags == Lv.flags == 3
    assert np.array_equal(LO.layout_arrays(Ll)["dst"], Lv.dst)


def test_loop_bf16_narrowing_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: ties to the even 1.0;
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: ties to the even 1 + 2^-6
    assert int(LO.narrow(1.0 + 2.0 ** -8, "bf16")) == 0x3F80
    assert int(LO.narrow(1.0 + 3 * 2.0 ** -8, "bf16")) == 0x3F82
    assert LO.widen(0x3F82, "bf16") == 1.0 + 2.0 ** -6
