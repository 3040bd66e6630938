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


# ----------------------------------------------------------------------------
# the weight gradient of the grouped GEMM


def brute_wgrad(L, a, g, gather):
    """grad_w[x][j][c] = sum over placed rows r of expert x of g[r, j] * A(r)[c], by loops."""
    n, m = g.shape[1], a.shape[1]
    out = np.zeros((L.e, n, m))
    for x in range(L.e):
        for r in range(int(L.offsets[x]), int(L.offsets[x]) + int(L.kept[x])):
            row = a[L.src[r]] if gather else a[r]
            for j in range(n):
                for c in range(m):
                    out[x, j, c] += float(g[r, j]) * float(row[c])
    return out


@pytest.mark.parametrize("cap,gather", [(0, True), (0, False), (3, True), (5, False)])
def test_expert_gemm_wgrad_matches_brute_force(cap, gather):
    rng = np.random.default_rng(40 + cap)
    s, e, k, m, n = 12, 5, 2, 5, 3  # non-square; e = 5 with s*k = 24 routes
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, cap)
    x = rng.standard_normal((s, m)).astype(np.float32)
    a = x if gather else oracle.dispatch(L, x)
    g = rng.standard_normal((L.rows, n)).astype(np.float32)
    gw, exact = oracle.expert_gemm_wgrad(L, a, g, "f32", gather)
    assert gw.shape == (e, n, m) and gw.dtype == np.float32
    assert np.allclose(exact, brute_wgrad(L, a, g, gather), rtol=1e-12, atol=1e-12)
    assert np.array_equal(gw, exact.astype(np.float32))


def test_expert_gemm_wgrad_is_the_adjoint_of_the_forward():
    """<G, forward(A, W)> = sum_x <W[x], wgrad(A, G)[x]> (exact sums, float64)."""
    rng = np.random.default_rng(41)
    s, e, k, m, n = 50, 6, 3, 7, 4
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 9)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16")
    wts = W.cast_input(rng.standard_normal((e * n, m)).astype(np.float32), "bf16").reshape(e, n, m)
    g = W.cast_input(rng.standard_normal((L.rows, n)).astype(np.float32), "bf16")
    _, y = oracle.expert_gemm(L, x, wts, "bf16", True)
    _, gw = oracle.expert_gemm_wgrad(L, x, g, "bf16", True)
    lhs = float(np.sum(oracle.to_f32(g, "bf16").astype(np.float64) * y))
    rhs = float(np.sum(oracle.to_f32(wts.reshape(e * n, m), "bf16").astype(np.float64).reshape(e, n, m) * gw))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_expert_gemm_wgrad_is_the_exact_derivative_on_integers():
    """f(W) = <G, forward(A, W)> is linear in W: raising one weight by 1 raises f by exactly
    that weight's gradient (small integers: every sum is exact)."""
    rng = np.random.default_rng(42)
    s, e, k, m, n = 30, 4, 2, 6, 5
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 0)
    x = rng.integers(-3, 4, (s, m)).astype(np.float32)
    wts = rng.integers(-3, 4, (e, n, m)).astype(np.float32)
    g = rng.integers(-3, 4, (L.rows, n)).astype(np.float32)
    _, gw = oracle.expert_gemm_wgrad(L, x, g, "f32", True)

    def f(wv):
        _, y = oracle.expert_gemm(L, x, wv, "f32", True)
        return float(np.sum(g.astype(np.float64) * y))

    base = f(wts)
    for _ in range(12):
        xe, j, c = rng.integers(0, e), rng.integers(0, n), rng.integers(0, m)
        bumped = wts.copy()
        bumped[xe, j, c] += 1.0
        assert f(bumped) - base == gw[xe, j, c]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_expert_gemm_wgrad_fused_equals_unfused_and_idle_experts_are_zero(dtype):
    rng = np.random.default_rng(43)
    s, e, k, m, n = 40, 6, 2, 16, 8
    idx = W.random_idx(rng, s, e - 1, k)  # expert e - 1 gets no route
    L = oracle.dispatch_layout(idx, e, 0)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    g = W.cast_input(rng.standard_normal((L.rows, n)).astype(np.float32), dtype)
    fused, _ = oracle.expert_gemm_wgrad(L, x, g, dtype, True)
    plain, _ = oracle.expert_gemm_wgrad(L, oracle.dispatch(L, x), g, dtype, False)
    assert np.array_equal(fused, plain)
    assert L.kept[e - 1] == 0 and not np.any(fused[e - 1])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_expert_gemm_wgrad_narrowed_output_rounds_to_nearest_even(dtype):
    """Gradients kept in the element type: column sums of ones that land between two
    representable values. bf16 holds 8 significant bits, so 257 (a tie) goes to the even
    256, 259 (a tie) to 260, 258 stays; f16 holds 11 bits, the same at 2049 / 2050 / 2051.
    Sums below 2^24 are exact in float32, so the element-type rounding is the only one."""
    base = 256 if dtype == "bf16" else 2048
    counts = [base + 1, base + 2, base + 3, 1, 0, base - 1, 7, base]
    want = [base, base + 2, base + 4, 1, 0, base - 1, 7, base]
    s, m, n = counts[0] + 2, 8, len(counts)
    idx = np.zeros((s, 1), np.int32)  # every token to the one expert
    L = oracle.dispatch_layout(idx, 1, 0)
    ones = 1.0 if dtype == "f16" else 0x3F80  # 1.0 in the element type
    x = np.full((s, m), ones, np.float16 if dtype == "f16" else np.uint16)
    g32 = np.zeros((L.rows, n), np.float32)
    for j, c in enumerate(counts):
        g32[:c, j] = 1.0
    g = g32.astype(np.float16) if dtype == "f16" else (g32.view(np.uint32) >> 16).astype(np.uint16)
    got, exact = oracle.expert_gemm_wgrad(L, x, g, dtype, True, out_dtype=dtype)
    assert np.array_equal(exact[0, :, 0], counts)
    got32 = oracle.to_f32(got, dtype)
    assert got.dtype == (np.float16 if dtype == "f16" else np.uint16)
    assert np.array_equal(got32[0], np.repeat(np.array(want, np.float32)[:, None], m, axis=1))
    f32, _ = oracle.expert_gemm_wgrad(L, x, g, dtype, True)
    assert f32.dtype == np.float32 and np.array_equal(f32[0, :, 0], counts)
    with pytest.raises(ValueError):
        oracle.expert_gemm_wgrad(L, x, g, dtype, True, out_dtype="f16" if dtype == "bf16" else "bf16")


# ----------------------------------------------------------------------------
# the input-row gradient of the grouped GEMM


@pytest.mark.parametrize("cap", [0, 4])
def test_expert_gemm_dgrad_matches_brute_force(cap):
    rng = np.random.default_rng(50 + cap)
    s, e, k, m, n = 14, 4, 2, 5, 3
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, cap)
    g = rng.standard_normal((L.rows, n)).astype(np.float32)
    wts = rng.standard_normal((e, n, m)).astype(np.float32)
    out, exact = oracle.expert_gemm_dgrad(L, g, wts, "f32")
    ref = np.zeros((L.rows, m))
    for x in range(e):
        for r in range(int(L.offsets[x]), int(L.offsets[x]) + int(L.kept[x])):
            for c in range(m):
                ref[r, c] = sum(float(g[r, j]) * float(wts[x, j, c]) for j in range(n))
    assert np.allclose(exact, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out, exact.astype(np.float32))
    assert np.all(out[L.src < 0] == 0)


def test_expert_gemm_dgrad_is_the_adjoint_of_the_forward():
    """<dgrad(G), A_rows> = <G, forward(A)> over the placed rows (exact sums, float64)."""
    rng = np.random.default_rng(51)
    s, e, k, m, n = 50, 6, 3, 7, 4
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 9)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16")
    wts = W.cast_input(rng.standard_normal((e * n, m)).astype(np.float32), "bf16").reshape(e, n, m)
    g = W.cast_input(rng.standard_normal((L.rows, n)).astype(np.float32), "bf16")
    _, y = oracle.expert_gemm(L, x, wts, "bf16", True)
    _, ga = oracle.expert_gemm_dgrad(L, g, wts, "bf16")
    a_rows = oracle.to_f32(oracle.dispatch(L, x), "bf16").astype(np.float64)
    lhs = float(np.sum(ga * a_rows))
    rhs = float(np.sum(oracle.to_f32(g, "bf16").astype(np.float64) * y))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_expert_gemm_input_gradient_is_the_exact_derivative_on_integers():
    """f(x) = <G, forward(x, W)>: raising one token's feature by 1 raises f by exactly the
    dispatch backward of dgrad(G) at that feature (small integers: every sum is exact)."""
    rng = np.random.default_rng(52)
    s, e, k, m, n = 30, 4, 2, 6, 5
    idx = W.random_idx(rng, s, e, k)
    L = oracle.dispatch_layout(idx, e, 11)  # some routes dropped
    x = rng.integers(-3, 4, (s, m)).astype(np.float32)
    wts = rng.integers(-3, 4, (e, n, m)).astype(np.float32)
    g = rng.integers(-3, 4, (L.rows, n)).astype(np.float32)
    ga, _ = oracle.expert_gemm_dgrad(L, g, wts, "f32")
    gx = oracle.dispatch_backward(L, ga, "f32")

    def f(xv):
        _, y = oracle.expert_gemm(L, xv, wts, "f32", True)
        return float(np.sum(g.astype(np.float64) * y))

    base = f(x)
    for _ in range(12):
        t, c = rng.integers(0, s), rng.integers(0, m)
        bumped = x.copy()
        bumped[t, c] += 1.0
        assert f(bumped) - base == gx[t, c]
