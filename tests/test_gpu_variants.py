"""GPU parity for the variants: route-major capacity priority, padded dropless
segments, weights applied at dispatch (and its backward), renormalisation over
kept routes, and their autograd wiring. Same bars as the main path: maps and
buffers bit-exact; float32 route-order sums bit-exact given the same inputs;
float64 dot products within 1e-6 of sum |terms|; float64 weight maths bit-exact
(both sides use the same operation order and IEEE division)."""
import numpy as np
import pytest
import torch

import combine_moe_gate_amd as M
import combine_moe_gate_amd.autograd as A
import oracle
import workloads as W
from tests.gpu_util import assert_bits_equal, f32_ulps, to_dev, to_host, weight_grad_bound
from tests.test_gpu_parity import check_buffer_chunked, check_layout

pytestmark = pytest.mark.gpu


def announce(*what):
    print("CASE", *what, flush=True)


OPTION_CASES = [
    # s, e, k, capacity, route_major, pad
    (1000, 40, 3, 30, True, 1), (1000, 40, 3, 0, True, 1), (257, 8, 8, 40, True, 1),
    (3000, 129, 5, 0, False, 16), (3000, 129, 5, 0, True, 128), (1, 3, 2, 0, False, 4),
    (0, 5, 2, 0, False, 8), (777, 1024, 16, 0, True, 1), (5000, 8, 2, 300, True, 1),
    # more than 256 tiles of items (tokens, or routes in route-major order)
    (40000, 128, 8, 0, True, 1), (70000, 129, 5, 0, False, 16), (9000, 40, 8, 1500, True, 1),
]


@pytest.mark.parametrize("s,e,k,cap,rm,pad", OPTION_CASES)
def test_layout_options_match_oracle(s, e, k, cap, rm, pad):
    announce("layout options", s, e, k, cap, rm, pad)
    rng = np.random.default_rng(s + e + k + cap + pad)
    idx = W.random_idx(rng, s, e, k)
    Lg = M.moe_dispatch_layout(to_dev(idx) if s else torch.zeros((0, k), dtype=torch.int32, device="cuda"),
                               e, cap, route_major=rm, pad_multiple=pad)
    Lo = oracle.dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
    check_layout(Lg, Lo, f"s={s} e={e} k={k} c={cap} rm={rm} pad={pad}")
    if s:
        x = W.cast_input(rng.standard_normal((s, 24)).astype(np.float32), "bf16")
        buf = M.moe_dispatch(Lg, to_dev(x, "bf16"))
        assert_bits_equal(to_host(buf), oracle.dispatch(Lo, x), "dispatch")


@pytest.mark.parametrize("name,rm,pad", [("gshard_capacity_drop", True, 1),
                                          ("dropless_top8_h2816", False, 128),
                                          ("zipf_skew_h4096", True, 1)])
def test_layout_options_on_workloads(name, rm, pad):
    announce("workload options", name, rm, pad)
    inp = W.make_inputs(name)
    w = inp.workload
    idx, _ = oracle.gate_topk(inp.logits, w.k)
    Lg = M.moe_dispatch_layout(to_dev(idx), w.e, w.capacity, route_major=rm, pad_multiple=pad)
    Lo = oracle.dispatch_layout(idx, w.e, w.capacity, route_major=rm, pad_multiple=pad)
    check_layout(Lg, Lo, name)
    buf = M.moe_dispatch(Lg, to_dev(inp.x, w.dtype))
    check_buffer_chunked(buf, inp.x, Lo.src, "dispatch")
    if pad > 1:  # padded rows stay zero through the backward too
        E = buf
        gE, _ = M.moe_combine_backward(Lg, to_dev(inp.grad_y, w.dtype), E, to_dev(oracle.gate_topk(inp.logits, w.k)[1]))
        pad_rows = torch.from_numpy(np.nonzero(Lo.src < 0)[0]).cuda()
        assert int(gE.index_select(0, pad_rows).view(torch.int16).abs().sum()) == 0


ROW_CASES = [(1000, 264, "bf16", 40, 3, 0, 1), (1000, 264, "bf16", 40, 3, 60, 1),
             (777, 72, "f16", 16, 4, 200, 1), (513, 36, "f32", 9, 2, 0, 8),
             (2000, 1032, "bf16", 128, 8, 0, 32), (129, 520, "f16", 3, 1, 20, 1)]


@pytest.mark.parametrize("s,m,dtype,e,k,cap,pad", ROW_CASES)
def test_weighted_dispatch_and_backward_match_oracle(s, m, dtype, e, k, cap, pad):
    announce("weighted dispatch", s, m, dtype, e, k, cap, pad)
    rng = np.random.default_rng(s + m + e + k + cap + pad)
    idx = W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    w = W.random_weights(rng, s, k)
    Lo = oracle.dispatch_layout(idx, e, cap, pad_multiple=pad)
    G = W.cast_input(rng.standard_normal((Lo.rows, m)).astype(np.float32), dtype)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap, pad_multiple=pad)

    out = M.moe_dispatch_weighted(Lg, to_dev(x, dtype), to_dev(w))
    assert_bits_equal(to_host(out), oracle.dispatch_weighted(Lo, x, w, dtype), "weighted dispatch")
    y = M.moe_combine(Lg, to_dev(G, dtype), None)
    assert_bits_equal(to_host(y), oracle.dispatch_backward(Lo, G, dtype), "unweighted combine")

    gx, gw = M.moe_dispatch_weighted_backward(Lg, to_dev(G, dtype), to_dev(x, dtype), to_dev(w))
    gx_o, gw_o = oracle.dispatch_weighted_backward(Lo, G, x, w, dtype)
    assert_bits_equal(to_host(gx), gx_o, "weighted dispatch backward: grad_x")
    bound = weight_grad_bound(oracle.to_f32(x, dtype), oracle.to_f32(G, dtype), Lo.dst)
    err = np.abs(to_host(gw).astype(np.float64) - gw_o)
    assert np.all(err <= 1e-6 * bound)
    assert f32_ulps(to_host(gw), gw_o).max() <= 1


@pytest.mark.parametrize("s,e,k,cap", [(2000, 16, 4, 300), (4096, 64, 8, 400), (300, 4, 2, 60), (50, 2, 2, 1)])
def test_renormalize_kept_matches_oracle(s, e, k, cap):
    announce("renormalize", s, e, k, cap)
    rng = np.random.default_rng(s + e)
    logits = rng.standard_normal((s, e)).astype(np.float32)
    logits[:, 0] += 2.0  # overflow expert 0 so routes drop
    idx, w = oracle.gate_topk(logits, k)
    Lo = oracle.dispatch_layout(idx, e, cap)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap)
    wr = M.moe_renormalize_kept(Lg, to_dev(w))
    assert_bits_equal(to_host(wr), oracle.renormalize_kept(Lo, w), "renormalized weights")
    g = rng.standard_normal((s, k)).astype(np.float32)
    gw = M.moe_renormalize_kept_backward(Lg, to_dev(w), to_dev(g))
    assert_bits_equal(to_host(gw), oracle.renormalize_kept_backward(Lo, w, g), "renormalize backward")


def test_autograd_weights_before_experts_and_renormalized():
    """gate -> layout(route-major, capacity) -> renormalize -> weighted dispatch -> sum."""
    announce("autograd variants")
    s, m, e, k, cap, dtype = 900, 64, 12, 3, 80, "f32"
    inp = W.random_case(91, s, m, e, k, cap, dtype)
    x = to_dev(inp.x).requires_grad_(True)
    logits = to_dev(inp.logits).requires_grad_(True)
    gy = to_dev(inp.grad_y)
    idx, w = A.route(logits, k)
    L, _ = A.layout(idx, e, cap, route_major=True)
    wr = A.renormalize(w, L)
    buf = A.dispatch_on(x, L, w=wr)
    y = A.combine(buf, None, L)
    (y * gy).sum().backward()

    idx_o, w_o = oracle.gate_topk(inp.logits, k)
    Lo = oracle.dispatch_layout(idx_o, e, cap, route_major=True)
    wr_o = oracle.renormalize_kept(Lo, w_o)
    y_o = oracle.dispatch_backward(Lo, oracle.dispatch_weighted(Lo, inp.x, wr_o, dtype), dtype)
    assert np.allclose(to_host(y), y_o, rtol=1e-6, atol=1e-6)
    # backward chain in the oracle: unweighted sum -> dispatch of grad_y; weighted dispatch
    # backward; renormalisation backward; gate backward
    g_buf = oracle.dispatch(Lo, inp.grad_y)
    gx_o, gwr_o = oracle.dispatch_weighted_backward(Lo, g_buf, inp.x, wr_o, dtype)
    gw_o = oracle.renormalize_kept_backward(Lo, w_o, gwr_o)
    gl_o = oracle.gate_topk_backward(idx_o, w_o, gw_o, e)
    assert np.allclose(to_host(x.grad), gx_o, rtol=1e-5, atol=1e-6)
    gl = to_host(logits.grad)
    assert np.all(gl[gl_o == 0] == 0)
    assert np.abs(gl - gl_o).max() <= 1e-5 * max(1e-30, np.abs(gl_o).max())


@pytest.mark.parametrize("seed", range(32))
def test_variant_random_configurations(seed):
    """Seeded random sizes, routing modes and dtypes (the row path's random configurations,
    other seeds) through the variants: weighted dispatch and its backward, the unweighted
    combine, renormalisation over kept routes and its backward, and the replay with its
    routing check, each to the bars above."""
    from tests.test_gpu_parity import random_config

    rng, s, e, k, dtype, m, cap, rm, pad, skew = random_config(1000 + seed)
    announce("variant random config", seed, s, e, k, dtype, m, cap, rm, pad, skew)
    idx = W.skewed_idx(rng, s, e, k) if skew else W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    w = W.random_weights(rng, s, k)
    Lo = oracle.dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
    G = W.cast_input(rng.standard_normal((Lo.rows, m)).astype(np.float32), dtype)
    g = rng.standard_normal((s, k)).astype(np.float32)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap, route_major=rm, pad_multiple=pad)

    out = M.moe_dispatch_weighted(Lg, to_dev(x, dtype), to_dev(w))
    assert_bits_equal(to_host(out), oracle.dispatch_weighted(Lo, x, w, dtype), "weighted dispatch")
    y = M.moe_combine(Lg, to_dev(G, dtype), None)
    assert_bits_equal(to_host(y), oracle.dispatch_backward(Lo, G, dtype), "unweighted combine")
    gx, gw = M.moe_dispatch_weighted_backward(Lg, to_dev(G, dtype), to_dev(x, dtype), to_dev(w))
    gx_o, gw_o = oracle.dispatch_weighted_backward(Lo, G, x, w, dtype)
    assert_bits_equal(to_host(gx), gx_o, "weighted dispatch backward: grad_x")
    bound = weight_grad_bound(oracle.to_f32(x, dtype), oracle.to_f32(G, dtype), Lo.dst)
    err = np.abs(to_host(gw).astype(np.float64) - gw_o)
    assert np.all(err <= 1e-6 * bound), f"grad_w err {err.max()}"

    wr = M.moe_renormalize_kept(Lg, to_dev(w))
    assert_bits_equal(to_host(wr), oracle.renormalize_kept(Lo, w), "renormalized weights")
    gwr = M.moe_renormalize_kept_backward(Lg, to_dev(w), to_dev(g))
    assert_bits_equal(to_host(gwr), oracle.renormalize_kept_backward(Lo, w, g), "renormalize backward")

    xd = to_dev(x, dtype)
    buf = M.moe_dispatch(Lg, xd)
    rep = M.moe_dispatch_replay(Lg, xd, to_dev(idx))
    assert_bits_equal(to_host(rep), to_host(buf), "replay")
    assert M.moe_layout_read(Lg)[0] == Lo.flags, "flags after a faithful replay"
    if s > 0 and k < e:  # one route of the last token moved to an expert it did not pick
        idx2 = idx.copy()
        idx2[-1, 0] = next(q for q in range(e) if q not in set(idx[-1].tolist()))
        rep2 = M.moe_dispatch_replay(Lg, xd, to_dev(idx2))
        assert M.moe_layout_read(Lg)[0] & M.FLAG_REPLAY_MISMATCH, "changed routing not flagged"
        assert_bits_equal(to_host(rep2), to_host(buf), "flagged replay still follows the layout")
