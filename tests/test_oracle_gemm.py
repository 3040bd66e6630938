"""Pins for the oracle's grouped expert GEMM (the consumer of the layout's offsets)."""
import numpy as np
import pytest

import oracle
import workloads as W


def brute_gemm(L, a, weights, gather):
    """Triple loop over placed rows, output features and input features."""
    e, n, m = weights.shape
    out = np.zeros((L.rows, n))
    for x in range(L.e):
        for r in range(int(L.offsets[x]), int(L.offsets[x]) + int(L.kept[x])):
            row = a[L.src[r]] if gather else a[r]
            for j in range(n):
                out[r, j] = sum(float(row[c]) * float(weights[x, j, c]) for c in range(m))
    return out


@pytest.mark.parametrize("cap,gather", [(0, True), (0, False), (3, True), (5, False)])
def test_expert_gemm_matches_brute_force(cap, gather):
    rng = np.random.default_rng(10 + cap)
    s, e, k, m, n = 12, 4, 2, 5, 3  # non-square, so a transposed operand would fail
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, cap)
    x = rng.standard_normal((s, m)).astype(np.float32)
    a = x if gather else oracle.dispatch(L, x)
    wts = rng.standard_normal((e, n, m)).astype(np.float32)
    out, exact = oracle.expert_gemm(L, a, wts, "f32", gather)
    ref = brute_gemm(L, a, wts, gather)
    assert np.allclose(exact, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out, exact.astype(np.float32))
    assert np.all(out[L.src < 0] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("cap", [0, 6])
def test_fused_gather_equals_gemm_on_the_dispatched_buffer(dtype, cap):
    rng = np.random.default_rng(20)
    s, e, k, m, n = 60, 5, 3, 16, 24
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, cap)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    wts = W.cast_input(rng.standard_normal((e * n, m)).astype(np.float32), dtype).reshape(e, n, m)
    fused, _ = oracle.expert_gemm(L, x, wts, dtype, True)
    plain, _ = oracle.expert_gemm(L, oracle.dispatch(L, x), wts, dtype, False)
    assert np.array_equal(fused, plain)


def test_scaled_identity_weights_route_rows_to_the_right_expert():
    """W[x] = 2**x * I: each segment's rows come out scaled by its own expert's power."""
    rng = np.random.default_rng(30)
    s, e, k, m = 40, 6, 2, 8
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 0)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16")
    wts = np.stack([np.eye(m, dtype=np.float32) * (2.0 ** xx) for xx in range(e)])
    out, _ = oracle.expert_gemm(L, x, W.cast_input(wts.reshape(e * m, m), "bf16").reshape(e, m, m), "bf16", True)
    x32 = oracle.to_f32(x, "bf16")
    for xx in range(e):
        for r in range(int(L.offsets[xx]), int(L.offsets[xx + 1])):
            assert np.array_equal(oracle.to_f32(out[r:r + 1], "bf16")[0], x32[L.src[r]] * 2.0 ** xx)


def test_route_weights_scale_each_row():
    rng = np.random.default_rng(40)
    s, e, k, m, n = 30, 4, 2, 8, 8
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 4)
    x = rng.standard_normal((s, m)).astype(np.float32)
    wts = rng.standard_normal((e, n, m)).astype(np.float32)
    rw = (2.0 ** rng.integers(-3, 3, size=(s, k))).astype(np.float32)
    plain, _ = oracle.expert_gemm(L, x, wts, "f32", True)
    scaled, _ = oracle.expert_gemm(L, x, wts, "f32", True, route_w=rw)
    for t in range(s):
        for j in range(k):
            r = L.dst[t, j]
            if r >= 0:
                assert np.array_equal(scaled[r], plain[r] * rw[t, j])
    assert np.all(scaled[L.src < 0] == 0)
