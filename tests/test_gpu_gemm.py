"""GPU parity for the grouped expert GEMM with the dispatch fused into its operand loads.

Bars:
  - the fused call (rows gathered from x through the layout) and the unfused one (on
    the dispatched buffer) are bitwise identical, with and without route weights;
  - every output is within the float32 accumulation bound of the oracle's exact
    products: |got - want| <= ulp_dtype(max(|got|, |want|)) + 2^-23 max(|got|, |want|)
    + |w| (m + 2) 2^-23 sum_m |a b|  (summation order on the matrix cores is not fixed;
    the oracle sums exactly and rounds once, so the bound is the worst-case error of an
    m-term float32 sum plus one rounding to the element type);
  - with small-integer operands every partial sum is exact in float32, so the output is
    bit-exact against the oracle;
  - rows no route fills are +0.0.
"""
import numpy as np
import pytest
import torch

import combine_moe_gate_amd as M
import oracle
import workloads as W
from tests.gpu_util import TORCH_DTYPE, assert_bits_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


def announce(*what):
    print("CASE", *what, flush=True)


def dtype_ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of dtype values at |v| (bf16: 8 significant bits, f16: 11), subnormal floor."""
    p, emin = (8, -126) if dtype == "bf16" else (11, -14)
    ex = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** emin)))
    return 2.0 ** (ex - (p - 1))


def abs_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    return (a & np.uint16(0x7FFF)) if dtype == "bf16" else np.abs(a)


def row_weights(Lo: oracle.Layout, w: np.ndarray | None) -> np.ndarray:
    rw = np.ones(Lo.rows)
    if w is not None:
        placed = Lo.dst >= 0
        rw[Lo.dst[placed]] = np.abs(w[placed].astype(np.float64))
    return rw


def check_gemm(got: np.ndarray, Lo: oracle.Layout, a: np.ndarray, wts: np.ndarray, dtype: str,
               gather: bool, route_w: np.ndarray | None, what: str):
    want, _ = oracle.expert_gemm(Lo, a, wts, dtype, gather, route_w)
    _, absb = oracle.expert_gemm(Lo, abs_bits(a, dtype), abs_bits(wts, dtype), dtype, gather)
    m = a.shape[1]
    g = oracle.to_f32(got, dtype).astype(np.float64)
    wv = oracle.to_f32(want, dtype).astype(np.float64)
    big = np.maximum(np.abs(g), np.abs(wv))
    tol = dtype_ulp(big, dtype) + 2.0 ** -23 * big + \
        row_weights(Lo, route_w)[:, None] * (m + 2) * 2.0 ** -23 * absb
    err = np.abs(g - wv)
    bad = np.argwhere(~(err <= tol))
    assert len(bad) == 0, (f"{what}: {len(bad)} outputs outside the bound, first {tuple(bad[0])}: "
                           f"got {g[tuple(bad[0])]!r} want {wv[tuple(bad[0])]!r} tol {tol[tuple(bad[0])]!r}")
    unfilled = Lo.src < 0
    assert not np.any(oracle.to_f32(got[unfilled], dtype).view(np.uint32)), f"{what}: unfilled rows not +0.0"


GEMM_CASES = [
    # s, m, n, e, k, capacity, pad, route_major, dtype
    (300, 64, 64, 4, 2, 0, 1, False, "bf16"),
    (1000, 264, 200, 8, 2, 0, 1, False, "bf16"),     # ragged K step and column tile
    (1000, 136, 136, 8, 3, 200, 1, True, "f16"),     # capacity drop, route-major slots
    (3000, 128, 256, 129, 5, 0, 16, False, "bf16"),  # padded segments, many experts
    (2000, 512, 384, 16, 4, 0, 128, False, "f16"),
    (1, 8, 8, 3, 2, 0, 1, False, "bf16"),            # smallest row length
    (5000, 96, 520, 2, 2, 0, 1, False, "bf16"),      # long segments: many row-blocks each
    (777, 64, 64, 1024, 16, 0, 1, True, "bf16"),     # most experts empty
    (3000, 72, 136, 2, 2, 0, 1, False, "f16"),       # long segments, f16
    (4000, 64, 64, 4, 2, 600, 1, False, "bf16"),     # large capacity with drops
]


@pytest.mark.parametrize("s,m,n,e,k,cap,pad,rm,dtype", GEMM_CASES)
def test_expert_gemm_matches_oracle(s, m, n, e, k, cap, pad, rm, dtype):
    announce("expert gemm", s, m, n, e, k, cap, pad, rm, dtype)
    rng = np.random.default_rng(s + m + n + e + k + cap + pad)
    idx = W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    wts = W.expert_weights(s + n, e, n, m, dtype)
    rw = W.random_weights(rng, s, k)
    Lo = oracle.dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap, route_major=rm, pad_multiple=pad)
    xd, wd, rwd = to_dev(x, dtype), to_dev(wts, dtype), to_dev(rw)

    fused = M.moe_expert_gemm(Lg, xd, wd, gather=True)
    check_gemm(to_host(fused), Lo, x, wts, dtype, True, None, "fused")
    buf = M.moe_dispatch(Lg, xd)
    unfused = M.moe_expert_gemm(Lg, buf, wd, gather=False)
    assert_bits_equal(to_host(unfused), to_host(fused), "unfused vs fused")

    fused_w = M.moe_expert_gemm(Lg, xd, wd, gather=True, w=rwd)
    check_gemm(to_host(fused_w), Lo, x, wts, dtype, True, rw, "fused, route weights")
    unfused_w = M.moe_expert_gemm(Lg, buf, wd, gather=False, w=rwd)
    assert_bits_equal(to_host(unfused_w), to_host(fused_w), "unfused vs fused, route weights")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_expert_gemm_integer_operands_bit_exact(dtype):
    """Operands in {-3..3}: each partial sum is an integer below 2^24, exact in float32."""
    announce("expert gemm integers", dtype)
    s, m, n, e, k = 700, 520, 136, 6, 2
    rng = np.random.default_rng(7)
    idx = W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.integers(-3, 4, (s, m)).astype(np.float32), dtype)
    wts = W.cast_input(rng.integers(-3, 4, (e, n, m)).astype(np.float32), dtype)
    rw = (2.0 ** rng.integers(-3, 3, (s, k))).astype(np.float32)
    Lo = oracle.dispatch_layout(idx, e, 0)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, 0)
    for w in (None, rw):
        got = M.moe_expert_gemm(Lg, to_dev(x, dtype), to_dev(wts, dtype), gather=True,
                                w=None if w is None else to_dev(w))
        want, _ = oracle.expert_gemm(Lo, x, wts, dtype, True, w)
        assert_bits_equal(to_host(got), want, f"integer operands, weights {w is not None}")


def test_expert_gemm_invalid_routes_leave_zero_rows():
    announce("expert gemm invalid routes")
    s, m, n, e, k = 400, 64, 72, 5, 3
    rng = np.random.default_rng(11)
    idx = W.random_idx(rng, s, e, k)
    idx[::7, 1] = -1
    idx[::11, 2] = e + 3
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16")
    wts = W.expert_weights(3, e, n, m, "bf16")
    Lo = oracle.dispatch_layout(idx, e, 0)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, 0)
    out = torch.full((Lg.rows, n), 7.0, dtype=torch.bfloat16, device="cuda")  # stale contents
    M.moe_expert_gemm(Lg, to_dev(x, "bf16"), to_dev(wts, "bf16"), gather=True, out=out)
    check_gemm(to_host(out), Lo, x, wts, "bf16", True, None, "invalid routes")


def test_expert_gemm_empty_and_rejects():
    announce("expert gemm empty")
    e, k, m, n = 4, 2, 16, 16
    Lg = M.moe_dispatch_layout(torch.zeros((0, k), dtype=torch.int32, device="cuda"), e, 0)
    x = torch.zeros((0, m), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((e, n, m), dtype=torch.bfloat16, device="cuda")
    out = M.moe_expert_gemm(Lg, x, wd, gather=True)
    assert out.shape == (0, n)
    idx = torch.zeros((4, k), dtype=torch.int32, device="cuda")
    idx[:, 1] = 1
    Lg = M.moe_dispatch_layout(idx, e, 0)
    x = torch.zeros((4, m), dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoeError):  # float32 has no matrix-core path here
        M.moe_expert_gemm(Lg, x, torch.zeros((e, n, m), device="cuda"), gather=True)
    x = torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoeError):  # 12 bf16 elements is not a whole 16-byte chunk count
        M.moe_expert_gemm(Lg, x, torch.zeros((e, n, 12), dtype=torch.bfloat16, device="cuda"), gather=True)


def sampled_sub_layout(Lo: oracle.Layout, rows: np.ndarray):
    """An oracle layout holding only the given placed rows, grouped by their expert, and
    the experts it keeps (in order)."""
    seg = np.searchsorted(Lo.offsets, rows, side="right") - 1
    experts = np.unique(seg)
    kept = np.array([np.sum(seg == x) for x in experts], np.int32)
    order = np.argsort(seg, kind="stable")
    rows = rows[order]
    offsets = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
    sub = oracle.Layout(s=Lo.s, e=len(experts), k=Lo.k, capacity=0, rows=len(rows), idx=Lo.idx,
                        counts=kept, kept=kept, offsets=offsets, dst=np.full_like(Lo.dst, -1),
                        src=Lo.src[rows], flags=0, checksum=0)
    return sub, experts, rows


# full size: the headline (256-row tiles, Zipf segments), the f16 capacity workload
# (256-row tiles over a padded [e, c] buffer) and the 4096-token dropless one (128-row tiles)
FULL_GEMM_WORKLOADS = [W.HEADLINE, "gshard_capacity_drop", "dropless_top8_h2816"]


def placed_rows(Lo: oracle.Layout, rng: np.random.Generator, count: int) -> list:
    """Random placed rows (capacity buffers also hold padding rows, which no token fills)."""
    placed = np.nonzero(Lo.src >= 0)[0]
    return rng.choice(placed, min(count, len(placed)), replace=False).tolist()


@pytest.mark.parametrize("name", FULL_GEMM_WORKLOADS)
def test_expert_gemm_full_workload_sampled(name):
    """A workload's routing and rows at the benchmark's expert width; outputs sampled at
    segment edges, tile edges and random rows are checked against the oracle."""
    inp = W.make_inputs(name)
    w = inp.workload
    n = W.EXPERT_WIDTH
    announce("expert gemm full", name, n)
    idx, _ = oracle.gate_topk(inp.logits, w.k)
    Lo = oracle.dispatch_layout(idx, w.e, w.capacity)
    Lg = M.moe_dispatch_layout(to_dev(idx), w.e, w.capacity)
    wts = W.expert_weights(w.seed + 1, w.e, n, w.m, w.dtype)
    xd, wd = to_dev(inp.x, w.dtype), to_dev(wts, w.dtype)
    fused = M.moe_expert_gemm(Lg, xd, wd, gather=True)
    buf = M.moe_dispatch(Lg, xd)
    unfused = M.moe_expert_gemm(Lg, buf, wd, gather=False)
    assert torch.equal(fused.view(torch.int16), unfused.view(torch.int16)), "unfused vs fused"
    del buf, unfused

    rng = np.random.default_rng(5)
    heavy = np.argsort(-Lo.kept)[:3]
    pick = set()
    for x in list(heavy) + [int(np.argmin(np.where(Lo.kept > 0, Lo.kept, 1 << 30))), w.e - 1]:
        r0, kx = int(Lo.offsets[x]), int(Lo.kept[x])
        for d in (0, 127, 128, kx - 1):
            if 0 <= d < kx:
                pick.add(r0 + d)
    pick.update(placed_rows(Lo, rng, 24))
    rows = np.array(sorted(pick))
    sub, experts, rows = sampled_sub_layout(Lo, rows)
    got = to_host(fused.index_select(0, torch.from_numpy(rows).cuda()))
    check_gemm(got, sub, inp.x, np.ascontiguousarray(wts[experts]), w.dtype, True, None,
               f"{name} sampled rows")


def test_layer_with_gemm_and_its_gradients_replays_from_a_hip_graph():
    """gate -> layout -> fused GEMM with the route weights in its epilogue -> unweighted
    combine, then the GEMM's input-row gradient and its weight gradient (float32 and bf16),
    captured once; every replay (with eager work between) equals the eager run."""
    announce("gemm hip graph")
    s, m, n, e, k = 2048, 96, 136, 8, 4  # 1024 rows per expert on average: 256-row tiles
    rng = np.random.default_rng(21)
    logits = to_dev(rng.standard_normal((s, e)).astype(np.float32))
    x = to_dev(W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16"), "bf16")
    wts = to_dev(W.expert_weights(22, e, n, m, "bf16"), "bf16")
    ws = torch.empty(M.workspace_bytes(s, e, k, 0), dtype=torch.uint8, device="cuda")
    idx = torch.empty((s, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((s, k), dtype=torch.float32, device="cuda")
    h = torch.empty((s * k, n), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((s, n), dtype=torch.bfloat16, device="cuda")
    ga = torch.empty((s * k, m), dtype=torch.bfloat16, device="cuda")
    gW = torch.empty((e, n, m), dtype=torch.float32, device="cuda")
    gWn = torch.empty((e, n, m), dtype=torch.bfloat16, device="cuda")

    def step():
        M.moe_gate_topk(logits, k, idx_out=idx, w_out=wt)
        L = M.moe_dispatch_layout(idx, e, 0, workspace=ws)
        M.moe_expert_gemm(L, x, wts, gather=True, w=wt, out=h)
        M.moe_combine(L, h, None, out=y)
        # h stands in for the gradient arriving at the GEMM's output
        M.moe_expert_gemm_dgrad(L, h, wts, out=ga)
        M.moe_expert_gemm_wgrad(L, x, h, gather=True, out=gW)
        M.moe_expert_gemm_wgrad(L, x, h, gather=True, out=gWn)

    outs = (idx, wt, h, y, ga, gW, gWn)
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    bits = lambda t: (t.view(torch.int16) if t.dtype == torch.bfloat16 else
                      t.view(torch.int32) if t.dtype == torch.float32 else t)
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(bits(a), bits(b)), f"replay {rep}"
        M.moe_gate_topk(logits.flip(0), k)  # eager work between replays
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# weight gradient


def check_wgrad(got: np.ndarray, Lo: oracle.Layout, a: np.ndarray, g: np.ndarray, dtype: str,
                gather: bool, what: str):
    """Within the float32 accumulation bound of the oracle's exact sums:
    |got - exact| <= 2^-23 |exact| + (K_x + 2) 2^-23 sum_r |g a|, K_x the expert's rows."""
    _, exact = oracle.expert_gemm_wgrad(Lo, a, g, dtype, gather)
    _, absb = oracle.expert_gemm_wgrad(Lo, abs_bits(a, dtype), abs_bits(g, dtype), dtype, gather)
    kx = Lo.kept.astype(np.float64)[:, None, None]
    tol = 2.0 ** -23 * np.abs(exact) + (kx + 2) * 2.0 ** -23 * absb
    err = np.abs(got.astype(np.float64) - exact)
    bad = np.argwhere(~(err <= tol))
    assert len(bad) == 0, (f"{what}: {len(bad)} outside the bound, first {tuple(bad[0])}: got "
                           f"{got[tuple(bad[0])]!r} exact {exact[tuple(bad[0])]!r} tol {tol[tuple(bad[0])]!r}")
    idle = Lo.kept == 0
    assert not np.any(got[idle].view(np.uint32)), f"{what}: idle experts not +0.0"


def check_wgrad_narrowed(got: np.ndarray, Lo: oracle.Layout, a: np.ndarray, g: np.ndarray, dtype: str,
                         what: str):
    """Gradients rounded to the element type: the float32 bound above plus one rounding,
    |got - exact| <= 2^-23 |exact| + (K_x + 2) 2^-23 sum_r |g a| + ulp_dtype(max(|got|, |exact|))."""
    _, exact = oracle.expert_gemm_wgrad(Lo, a, g, dtype, True)
    _, absb = oracle.expert_gemm_wgrad(Lo, abs_bits(a, dtype), abs_bits(g, dtype), dtype, True)
    kx = Lo.kept.astype(np.float64)[:, None, None]
    g64 = oracle.to_f32(got, dtype).astype(np.float64)
    big = np.maximum(np.abs(g64), np.abs(exact))
    tol = 2.0 ** -23 * np.abs(exact) + (kx + 2) * 2.0 ** -23 * absb + dtype_ulp(big, dtype)
    err = np.abs(g64 - exact)
    bad = np.argwhere(~(err <= tol))
    assert len(bad) == 0, (f"{what}: {len(bad)} outside the bound, first {tuple(bad[0])}: got "
                           f"{g64[tuple(bad[0])]!r} exact {exact[tuple(bad[0])]!r} tol {tol[tuple(bad[0])]!r}")
    idle = Lo.kept == 0
    assert not np.any(oracle.to_f32(got[idle], dtype).view(np.uint32)), f"{what}: idle experts not +0.0"


WGRAD_CASES = [
    # s, m, n, e, k, capacity, pad, route_major, dtype
    (300, 64, 64, 4, 2, 0, 1, False, "bf16"),
    (1000, 264, 200, 8, 2, 0, 1, False, "bf16"),     # ragged column tiles, 100-row K tail
    (1000, 136, 136, 8, 3, 200, 1, True, "f16"),     # capacity drop, route-major slots
    (3000, 128, 520, 129, 5, 0, 16, False, "bf16"),  # padded segments, idle experts
    (5000, 96, 72, 2, 2, 0, 1, False, "bf16"),       # 5000-row segments: many K steps
    (1, 8, 8, 3, 2, 0, 1, False, "f16"),
    (777, 64, 64, 1024, 16, 0, 1, True, "bf16"),     # most experts idle
]


@pytest.mark.parametrize("s,m,n,e,k,cap,pad,rm,dtype", WGRAD_CASES)
def test_expert_gemm_wgrad_matches_oracle(s, m, n, e, k, cap, pad, rm, dtype):
    announce("expert gemm wgrad", s, m, n, e, k, cap, pad, rm, dtype)
    rng = np.random.default_rng(s + 3 * m + n + e + k + cap + pad)
    idx = W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    Lo = oracle.dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
    g = W.cast_input(rng.standard_normal((Lo.rows, n)).astype(np.float32), dtype)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap, route_major=rm, pad_multiple=pad)
    xd, gd = to_dev(x, dtype), to_dev(g, dtype)
    stale = torch.full((e, n, m), 7.0, dtype=torch.float32, device="cuda")
    fused = M.moe_expert_gemm_wgrad(Lg, xd, gd, gather=True, out=stale)
    check_wgrad(to_host(fused), Lo, x, g, dtype, True, "fused")
    unfused = M.moe_expert_gemm_wgrad(Lg, M.moe_dispatch(Lg, xd), gd, gather=False)
    assert_bits_equal(to_host(unfused), to_host(fused), "unfused vs fused")
    # kept in the element type: the same float32 sums, each rounded once to nearest even
    stale_n = torch.full((e, n, m), 7.0, dtype=TORCH_DTYPE[dtype], device="cuda")
    narrowed = M.moe_expert_gemm_wgrad(Lg, xd, gd, gather=True, out=stale_n)
    assert narrowed.dtype == TORCH_DTYPE[dtype]
    assert torch.equal(narrowed.view(torch.int16), fused.to(TORCH_DTYPE[dtype]).view(torch.int16)), \
        "narrowed output is not the rounding of the float32 output"
    check_wgrad_narrowed(to_host(narrowed), Lo, x, g, dtype, "narrowed")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_expert_gemm_wgrad_integer_operands_bit_exact(dtype):
    """Operands in {-3..3}: every partial sum is an integer below 2^24, exact in float32."""
    announce("expert gemm wgrad integers", dtype)
    s, m, n, e, k = 1500, 136, 264, 5, 2
    rng = np.random.default_rng(17)
    idx = W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.integers(-3, 4, (s, m)).astype(np.float32), dtype)
    Lo = oracle.dispatch_layout(idx, e, 0)
    g = W.cast_input(rng.integers(-3, 4, (Lo.rows, n)).astype(np.float32), dtype)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, 0)
    got = M.moe_expert_gemm_wgrad(Lg, to_dev(x, dtype), to_dev(g, dtype), gather=True)
    want, _ = oracle.expert_gemm_wgrad(Lo, x, g, dtype, True)
    assert_bits_equal(to_host(got), want, "integer operands")
    if dtype == "bf16":
        assert np.abs(want).max() > 256  # sums that bf16 has to round
    got_n = M.moe_expert_gemm_wgrad(Lg, to_dev(x, dtype), to_dev(g, dtype), gather=True,
                                    out_dtype=TORCH_DTYPE[dtype])
    want_n, _ = oracle.expert_gemm_wgrad(Lo, x, g, dtype, True, out_dtype=dtype)
    assert_bits_equal(to_host(got_n), want_n, "integer operands, narrowed output")


def test_expert_gemm_wgrad_empty_layout_zeroes_everything():
    announce("expert gemm wgrad empty")
    e, k, m, n = 3, 2, 16, 24
    Lg = M.moe_dispatch_layout(torch.zeros((0, k), dtype=torch.int32, device="cuda"), e, 0)
    x = torch.zeros((0, m), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((0, n), dtype=torch.bfloat16, device="cuda")
    out = torch.full((e, n, m), 3.0, dtype=torch.float32, device="cuda")
    M.moe_expert_gemm_wgrad(Lg, x, g, gather=True, out=out)
    assert int(out.view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("name", FULL_GEMM_WORKLOADS)
def test_expert_gemm_wgrad_full_workload_sampled(name):
    """A workload's routing and rows at the benchmark's expert width; a block of sampled
    output features x input features of every expert is checked against the oracle (the
    gradient separates over output and input features, so the oracle runs on those
    columns only)."""
    inp = W.make_inputs(name)
    w = inp.workload
    n = W.EXPERT_WIDTH
    announce("expert gemm wgrad full", name, n)
    idx, _ = oracle.gate_topk(inp.logits, w.k)
    Lo = oracle.dispatch_layout(idx, w.e, w.capacity)
    Lg = M.moe_dispatch_layout(to_dev(idx), w.e, w.capacity)
    rng = np.random.default_rng(9)
    g = W.cast_input(rng.standard_normal((Lo.rows, n), dtype=np.float32), w.dtype)
    xd, gd = to_dev(inp.x, w.dtype), to_dev(g, w.dtype)
    got = M.moe_expert_gemm_wgrad(Lg, xd, gd, gather=True)
    unfused = M.moe_expert_gemm_wgrad(Lg, M.moe_dispatch(Lg, xd), gd, gather=False)
    assert torch.equal(got.view(torch.int32), unfused.view(torch.int32)), "unfused vs fused"
    del unfused
    narrowed = M.moe_expert_gemm_wgrad(Lg, xd, gd, gather=True, out_dtype=TORCH_DTYPE[w.dtype])
    assert torch.equal(narrowed.view(torch.int16), got.to(TORCH_DTYPE[w.dtype]).view(torch.int16)), \
        "narrowed output is not the rounding of the float32 output"
    del narrowed
    J = np.unique(np.concatenate([[0, 255, 256, n - 1], rng.choice(n, 12, replace=False)]))
    C = np.unique(np.concatenate([[0, 255, 256, w.m - 1], rng.choice(w.m, 12, replace=False)]))
    sub = got.index_select(1, torch.from_numpy(J).cuda()).index_select(2, torch.from_numpy(C).cuda())
    check_wgrad(to_host(sub), Lo, np.ascontiguousarray(inp.x[:, C]), np.ascontiguousarray(g[:, J]),
                w.dtype, True, f"{name} sampled features")


# ----------------------------------------------------------------------------
# input-row gradient


def check_dgrad(got: np.ndarray, Lo: oracle.Layout, g: np.ndarray, wts: np.ndarray, dtype: str,
                what: str):
    want, _ = oracle.expert_gemm_dgrad(Lo, g, wts, dtype)
    _, absb = oracle.expert_gemm_dgrad(Lo, abs_bits(g, dtype), abs_bits(wts, dtype), dtype)
    n = g.shape[1]
    gv = oracle.to_f32(got, dtype).astype(np.float64)
    wv = oracle.to_f32(want, dtype).astype(np.float64)
    big = np.maximum(np.abs(gv), np.abs(wv))
    tol = dtype_ulp(big, dtype) + 2.0 ** -23 * big + (n + 2) * 2.0 ** -23 * absb
    bad = np.argwhere(~(np.abs(gv - wv) <= tol))
    assert len(bad) == 0, (f"{what}: {len(bad)} outside the bound, first {tuple(bad[0])}: got "
                           f"{gv[tuple(bad[0])]!r} want {wv[tuple(bad[0])]!r}")
    assert not np.any(oracle.to_f32(got[Lo.src < 0], dtype).view(np.uint32)), f"{what}: unfilled rows"


DGRAD_CASES = [
    # s, m, n, e, k, capacity, pad, route_major, dtype
    (300, 64, 64, 4, 2, 0, 1, False, "bf16"),
    (1000, 200, 264, 8, 2, 0, 1, False, "bf16"),     # ragged K step (n) and column tile (m)
    (1000, 136, 136, 8, 3, 200, 1, True, "f16"),     # capacity drop, route-major slots
    (3000, 520, 128, 129, 5, 0, 16, False, "bf16"),  # padded segments, many experts
    (5000, 72, 96, 2, 2, 0, 1, False, "f16"),        # long segments
    (1, 8, 8, 3, 2, 0, 1, False, "bf16"),
]


@pytest.mark.parametrize("s,m,n,e,k,cap,pad,rm,dtype", DGRAD_CASES)
def test_expert_gemm_dgrad_matches_oracle(s, m, n, e, k, cap, pad, rm, dtype):
    announce("expert gemm dgrad", s, m, n, e, k, cap, pad, rm, dtype)
    rng = np.random.default_rng(s + m + 5 * n + e + k + cap + pad)
    idx = W.random_idx(rng, s, e, k)
    Lo = oracle.dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
    g = W.cast_input(rng.standard_normal((Lo.rows, n)).astype(np.float32), dtype)
    wts = W.expert_weights(s + m, e, n, m, dtype)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap, route_major=rm, pad_multiple=pad)
    stale = torch.full((Lo.rows, m), 5.0, dtype=TORCH_DTYPE[dtype], device="cuda")
    ga = M.moe_expert_gemm_dgrad(Lg, to_dev(g, dtype), to_dev(wts, dtype), out=stale)
    check_dgrad(to_host(ga), Lo, g, wts, dtype, "grad_a")
    # the token gradient: the dispatch backward of grad_a, bit-exact given the same rows
    gx = M.moe_dispatch_backward(Lg, ga)
    assert_bits_equal(to_host(gx), oracle.dispatch_backward(Lo, to_host(ga), dtype), "grad_x")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_expert_gemm_dgrad_integer_operands_bit_exact(dtype):
    announce("expert gemm dgrad integers", dtype)
    s, m, n, e, k = 900, 136, 520, 6, 2
    rng = np.random.default_rng(19)
    idx = W.random_idx(rng, s, e, k)
    Lo = oracle.dispatch_layout(idx, e, 0)
    g = W.cast_input(rng.integers(-3, 4, (Lo.rows, n)).astype(np.float32), dtype)
    wts = W.cast_input(rng.integers(-3, 4, (e, n, m)).astype(np.float32), dtype)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, 0)
    got = M.moe_expert_gemm_dgrad(Lg, to_dev(g, dtype), to_dev(wts, dtype))
    want, _ = oracle.expert_gemm_dgrad(Lo, g, wts, dtype)
    assert_bits_equal(to_host(got), want, "integer operands")


@pytest.mark.parametrize("name", FULL_GEMM_WORKLOADS)
def test_expert_gemm_dgrad_full_workload_sampled(name):
    inp = W.make_inputs(name)
    w = inp.workload
    n = W.EXPERT_WIDTH
    announce("expert gemm dgrad full", name, n)
    idx, _ = oracle.gate_topk(inp.logits, w.k)
    Lo = oracle.dispatch_layout(idx, w.e, w.capacity)
    Lg = M.moe_dispatch_layout(to_dev(idx), w.e, w.capacity)
    rng = np.random.default_rng(8)
    g = W.cast_input(rng.standard_normal((Lo.rows, n), dtype=np.float32), w.dtype)
    wts = W.expert_weights(w.seed + 1, w.e, n, w.m, w.dtype)
    ga = M.moe_expert_gemm_dgrad(Lg, to_dev(g, w.dtype), to_dev(wts, w.dtype))
    heavy = np.argsort(-Lo.kept)[:3]
    pick = set()
    for x in list(heavy) + [w.e - 1]:
        r0, kx = int(Lo.offsets[x]), int(Lo.kept[x])
        for d in (0, 255, 256, kx - 1):
            if 0 <= d < kx:
                pick.add(r0 + d)
    pick.update(placed_rows(Lo, rng, 24))
    sub, experts, rows = sampled_sub_layout(Lo, np.array(sorted(pick)))
    got = to_host(ga.index_select(0, torch.from_numpy(rows).cuda()))
    check_dgrad(got, sub, np.ascontiguousarray(g[rows]), np.ascontiguousarray(wts[experts]), w.dtype,
                f"{name} sampled rows")


# ----------------------------------------------------------------------------
# seeded random configurations: forward and both gradients


@pytest.mark.parametrize("seed", range(24))
def test_gemm_random_configurations(seed):
    """Sizes, routing mode and dtype drawn from one seeded generator; the forward (with
    route weights half the time), the input-row gradient and the weight gradient (float32
    and the element type) each within their bounds of the oracle."""
    rng = np.random.default_rng(7000 + seed)
    s = int(rng.integers(1, 1500))
    e = int(rng.integers(1, 40))
    k = int(rng.integers(1, min(e, 8) + 1))
    m = 8 * int(rng.integers(1, 70))
    n = 8 * int(rng.integers(1, 70))
    dtype = ["bf16", "f16"][int(rng.integers(0, 2))]
    cap = 0 if rng.random() < 0.5 else int(rng.integers(1, max(2, 2 * s * k // e)))
    rm = bool(rng.random() < 0.3) and cap > 0
    pad = int([1, 1, 16, 128][int(rng.integers(0, 4))]) if cap == 0 else 1
    announce("gemm random config", seed, s, e, k, m, n, dtype, cap, rm, pad)
    idx = W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    wts = W.expert_weights(seed, e, n, m, dtype)
    rw = W.random_weights(rng, s, k) if rng.random() < 0.5 else None
    Lo = oracle.dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
    g = W.cast_input(rng.standard_normal((Lo.rows, n)).astype(np.float32), dtype)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap, route_major=rm, pad_multiple=pad)
    xd, wd, gd = to_dev(x, dtype), to_dev(wts, dtype), to_dev(g, dtype)

    out = M.moe_expert_gemm(Lg, xd, wd, gather=True, w=None if rw is None else to_dev(rw))
    check_gemm(to_host(out), Lo, x, wts, dtype, True, rw, "forward")
    ga = M.moe_expert_gemm_dgrad(Lg, gd, wd)
    check_dgrad(to_host(ga), Lo, g, wts, dtype, "input-row gradient")
    gw = M.moe_expert_gemm_wgrad(Lg, xd, gd, gather=True)
    check_wgrad(to_host(gw), Lo, x, g, dtype, True, "weight gradient")
    gwn = M.moe_expert_gemm_wgrad(Lg, xd, gd, gather=True, out_dtype=TORCH_DTYPE[dtype])
    assert torch.equal(gwn.view(torch.int16), gw.to(TORCH_DTYPE[dtype]).view(torch.int16)), \
        "narrowed weight gradient is not the rounding of the float32 one"
    check_wgrad_narrowed(to_host(gwn), Lo, x, g, dtype, "weight gradient, element type")
