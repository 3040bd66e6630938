"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bars: expert ids, counts, offsets, slot maps and permuted buffers bit-exact;
combine, dispatch backward and grad_E bit-exact when both sides are given the
same weights (both accumulate in float32 in route order, separate multiply and
add, one rounding); grad_w within 1e-6 of sum_m |grad_y * E| (float64 sums on
both sides, summed in different orders); gate weights and gate gradients within
one float32 ulp (float64 on both sides). End to end, where each side uses its
own gate weights, outputs agree within 1e-6 relative (float32) or one ulp of
the element type (bf16/f16), the tolerance the weights' last-ulp freedom needs.
"""
import numpy as np
import pytest
import torch

import combine_moe_gate_amd as M
import oracle
import workloads as W
from tests.gpu_util import (TORCH_DTYPE, assert_bits_equal, compact_layout, f32_ulps, tagged_rows,
                            to_dev, to_host, token_chunks, weight_grad_bound)

pytestmark = pytest.mark.gpu

ALL = list(W.WORKLOADS)


def announce(*what):
    print("CASE", *what, flush=True)


def check_layout(Lg: M.Layout, Lo: oracle.Layout, what: str):
    assert Lg.rows == Lo.rows, what
    assert_bits_equal(to_host(Lg.counts), Lo.counts, f"{what} counts")
    assert_bits_equal(to_host(Lg.kept), Lo.kept, f"{what} kept")
    assert_bits_equal(to_host(Lg.offsets), Lo.offsets, f"{what} offsets")
    assert_bits_equal(to_host(Lg.dst), Lo.dst, f"{what} dst")
    assert_bits_equal(to_host(Lg.src), Lo.src, f"{what} src")
    assert_bits_equal(to_host(Lg.route_idx), Lo.idx, f"{what} route copy")
    flags, checksum = M.moe_layout_read(Lg)
    assert flags == Lo.flags, f"{what} flags {flags} != {Lo.flags}"
    assert checksum == Lo.checksum, f"{what} checksum"


def check_buffer_chunked(buf_dev: torch.Tensor, x: np.ndarray, src: np.ndarray, what: str,
                         chunk_rows: int = 16384):
    """Every buffer row equals x[src[r]] bit for bit, or zero where src[r] = -1."""
    rows = buf_dev.shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        got = to_host(buf_dev[r0:r1])
        s = src[r0:r1]
        want = np.zeros_like(got)
        have = s >= 0
        want[have] = x[s[have]]
        assert_bits_equal(got, want, f"{what} rows {r0}:{r1}")


# ----------------------------------------------------------------------------
# step 1: gate


@pytest.mark.parametrize("name", ALL)
def test_gate_matches_oracle_on_workload(name):
    announce("gate", name)
    inp = W.make_inputs(name)
    w = inp.workload
    idx, wt = M.moe_gate_topk(to_dev(inp.logits), w.k)
    idx_o, wt_o = oracle.gate_topk(inp.logits, w.k)
    assert_bits_equal(to_host(idx), idx_o, f"{name} idx")
    ulps = f32_ulps(to_host(wt), wt_o)
    assert ulps.max() <= 1, f"{name} weights differ by {ulps.max()} ulp"


@pytest.mark.parametrize("e,k", [(8, 1), (8, 8), (64, 2), (100, 8), (130, 16), (1024, 16), (1024, 1)])
def test_gate_ties_signed_zeros_and_shapes(e, k):
    announce("gate ties", e, k)
    rng = np.random.default_rng(e * 100 + k)
    s = 300 + (e + k) % 4  # the last workgroup of four tokens partly filled, in most cases
    logits = rng.integers(-2, 3, size=(s, e)).astype(np.float32)
    logits[rng.random((s, e)) < 0.2] = -0.0
    logits[:5] = 0.0  # all-equal rows
    idx, wt = M.moe_gate_topk(to_dev(logits), k)
    idx_o, wt_o = oracle.gate_topk(logits, k)
    assert_bits_equal(to_host(idx), idx_o, "idx")
    assert f32_ulps(to_host(wt), wt_o).max() <= 1


@pytest.mark.parametrize("e,k", [(8, 2), (128, 8), (600, 16)])
def test_gate_batches_smaller_than_a_workgroup(e, k):
    """One to seven tokens: a workgroup forms the weights of its four tokens in one wave,
    so a batch that leaves some of those four empty must still give every token's."""
    announce("gate small batches", e, k)
    rng = np.random.default_rng(e + 17 * k)
    for s in range(1, 8):
        logits = rng.standard_normal((s, e)).astype(np.float32)
        idx, wt = M.moe_gate_topk(to_dev(logits), k)
        idx_o, wt_o = oracle.gate_topk(logits, k)
        assert_bits_equal(to_host(idx), idx_o, f"idx s={s}")
        assert f32_ulps(to_host(wt), wt_o).max() <= 1, s


def test_gate_random_shapes():
    """60 seeded shapes: e from 1 to 1024 (one to sixteen logits per lane), k up to 16, s up
    to 3000 (partly filled last workgroups), a third of them on a coarse grid of logits so
    that ties between experts are common."""
    for seed in range(60):
        rng = np.random.default_rng(50_000 + seed)
        e = int(rng.choice([1, 2, 7, 8, 63, 64, 65, 128, 129, 256, 300, 512, 513, 777, 1024]))
        k = int(rng.integers(1, min(e, 16) + 1))
        s = int(rng.integers(1, 3000))
        announce("gate random", seed, s, e, k)
        if rng.random() < 0.35:
            logits = rng.integers(-3, 4, size=(s, e)).astype(np.float32)
            logits[rng.random((s, e)) < 0.1] = -0.0
        else:
            logits = (rng.standard_normal((s, e)) * rng.choice([0.01, 1.0, 30.0])).astype(np.float32)
        idx, wt = M.moe_gate_topk(to_dev(logits), k)
        idx_o, wt_o = oracle.gate_topk(logits, k)
        assert_bits_equal(to_host(idx), idx_o, f"idx seed {seed}")
        assert f32_ulps(to_host(wt), wt_o).max() <= 1, seed


def test_gate_backward_matches_oracle():
    announce("gate backward")
    rng = np.random.default_rng(9)
    for s, e, k in [(1000, 128, 8), (257, 8, 2), (64, 1024, 16), (33, 5, 5)]:
        logits = rng.standard_normal((s, e)).astype(np.float32)
        idx_o, wt_o = oracle.gate_topk(logits, k)
        gw = rng.standard_normal((s, k)).astype(np.float32)
        gl = to_host(M.moe_gate_topk_backward(to_dev(idx_o), to_dev(wt_o), to_dev(gw), e))
        gl_o = oracle.gate_topk_backward(idx_o, wt_o, gw, e)
        assert np.all(gl[gl_o == 0] == 0)
        assert f32_ulps(gl, gl_o).max() <= 1, (s, e, k)


# ----------------------------------------------------------------------------
# step 2: layout


@pytest.mark.parametrize("name", ALL)
def test_layout_matches_oracle_on_workload(name):
    announce("layout", name)
    inp = W.make_inputs(name)
    w = inp.workload
    idx_o, _ = oracle.gate_topk(inp.logits, w.k)
    Lg = M.moe_dispatch_layout(to_dev(idx_o), w.e, w.capacity)
    Lo = oracle.dispatch_layout(idx_o, w.e, w.capacity)
    check_layout(Lg, Lo, name)


LAYOUT_CASES = [
    # s, e, k, capacity, routing
    (1, 1, 1, 0, "uniform"), (1, 4, 4, 1, "uniform"), (255, 3, 2, 0, "uniform"),
    (256, 40, 3, 7, "uniform"), (257, 64, 8, 0, "uniform"), (1000, 129, 5, 40, "uniform"),
    (3000, 1024, 16, 0, "uniform"), (3000, 1024, 16, 50, "uniform"), (2049, 16, 4, 1, "skew"),
    (5000, 8, 2, 0, "skew"), (5000, 8, 8, 1000, "skew"), (700, 2, 1, 0, "uniform"),
    # more than 256 tiles: the tile table is scanned by its own launch
    (70000, 64, 2, 0, "uniform"), (90000, 128, 8, 4000, "skew"),
]


@pytest.mark.parametrize("s,e,k,cap,routing", LAYOUT_CASES)
def test_layout_random_cases(s, e, k, cap, routing):
    announce("layout case", s, e, k, cap, routing)
    rng = np.random.default_rng(s * 7 + e * 3 + k + cap)
    idx = W.skewed_idx(rng, s, e, k) if routing == "skew" else W.random_idx(rng, s, e, k)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap)
    check_layout(Lg, oracle.dispatch_layout(idx, e, cap), f"s={s} e={e} k={k} c={cap}")


@pytest.mark.parametrize("s", [600, 200, 70000])  # several tiles; one (no count launch); > 256 (scanned)
@pytest.mark.parametrize("cap", [0, 3])
def test_layout_invalid_routes_are_flagged_and_skipped(cap, s):
    announce("layout invalid", cap, s)
    rng = np.random.default_rng(77 + cap)
    e, k = 12, 4
    idx = W.random_idx(rng, s, e, k)
    idx[5, 2] = e          # out of range
    idx[17, 0] = -3        # out of range
    idx[s // 2, 3] = idx[s // 2, 1]  # duplicate
    idx[s - 1, 1] = idx[s - 1, 0]
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap)
    Lo = oracle.dispatch_layout(idx, e, cap)
    assert Lo.flags == 3
    check_layout(Lg, Lo, "invalid")
    # the permute leaves the skipped routes' rows as zero padding
    x = rng.standard_normal((s, 16)).astype(np.float32)
    buf = M.moe_dispatch(Lg, to_dev(x))
    assert_bits_equal(to_host(buf), oracle.dispatch(Lo, x), "dispatch with invalid routes")


# ----------------------------------------------------------------------------
# steps 3-5 on small random cases (several tiles, ragged row tails)

ROW_CASES = [
    # s, m, dtype, e, k, capacity
    (1000, 264, "bf16", 40, 3, 0),
    (1000, 264, "bf16", 40, 3, 60),
    (777, 72, "f16", 16, 4, 200),
    (513, 36, "f32", 9, 2, 0),
    (300, 4, "f32", 5, 5, 50),
    (64, 8, "bf16", 1024, 16, 0),
    (2000, 1032, "bf16", 128, 8, 0),
    (129, 520, "f16", 3, 1, 20),
    # rows longer than one group per wave (more than 8 KiB): waves take several groups
    (300, 8200, "bf16", 16, 4, 0),
    (200, 2052, "f32", 8, 2, 30),
]


@pytest.mark.parametrize("s,m,dtype,e,k,cap", ROW_CASES)
def test_rows_forward_backward_bit_exact(s, m, dtype, e, k, cap):
    announce("rows", s, m, dtype, e, k, cap)
    rng = np.random.default_rng(s + m + e + k + cap)
    idx = W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    w = W.random_weights(rng, s, k)
    Lo = oracle.dispatch_layout(idx, e, cap)
    E = W.cast_input(rng.standard_normal((Lo.rows, m)).astype(np.float32), dtype)
    gy = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    G = W.cast_input(rng.standard_normal((Lo.rows, m)).astype(np.float32), dtype)

    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap)
    buf = M.moe_dispatch(Lg, to_dev(x, dtype))
    assert_bits_equal(to_host(buf), oracle.dispatch(Lo, x), "dispatch")

    y = M.moe_combine(Lg, to_dev(E, dtype), to_dev(w))
    assert_bits_equal(to_host(y), oracle.combine(Lo, E, w, dtype), "combine")

    gE, gw = M.moe_combine_backward(Lg, to_dev(gy, dtype), to_dev(E, dtype), to_dev(w))
    gE_o, gw_o = oracle.combine_backward(Lo, gy, E, w, dtype)
    assert_bits_equal(to_host(gE), gE_o, "grad_E")
    bound = weight_grad_bound(oracle.to_f32(gy, dtype), oracle.to_f32(E, dtype), Lo.dst)
    err = np.abs(to_host(gw).astype(np.float64) - gw_o)
    assert np.all(err <= 1e-6 * bound), f"grad_w err {err.max()}"
    assert f32_ulps(to_host(gw), gw_o).max() <= 1

    gx = M.moe_dispatch_backward(Lg, to_dev(G, dtype))
    assert_bits_equal(to_host(gx), oracle.dispatch_backward(Lo, G, dtype), "dispatch backward")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("cap", [0, 5])
def test_unit_weight_round_trip_closed_form(dtype, cap):
    """combine(dispatch(x), 1) equals each row times its kept-route count, exactly."""
    announce("round trip", dtype, cap)
    rng = np.random.default_rng(5)
    s, e, k, m = 1500, 24, 6, 40
    idx = W.random_idx(rng, s, e, k)
    x32 = oracle.to_f32(W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16"), "bf16")
    x = W.cast_input(x32, dtype)
    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap)
    buf = M.moe_dispatch(Lg, to_dev(x, dtype))
    y = to_host(M.moe_combine(Lg, buf, torch.ones((s, k), device="cuda")))
    kept_t = (to_host(Lg.dst) >= 0).sum(1)
    exact = kept_t[:, None] * oracle.to_f32(x, dtype).astype(np.float64) + 0.0
    assert_bits_equal(y, oracle.from_f32(exact.astype(np.float32), dtype), "round trip")


# ----------------------------------------------------------------------------
# whole path on the five workloads, at full size


# tokens per chunk of the full-size sweeps below: every token of every workload is
# compared, a chunk at a time, against the oracle run on just that chunk's rows
CHUNK_TOKENS = 1024


def check_end_to_end_chunk(toks, S, E_c, wt_o, idx_o, dt, e, y_o, gw_o, bound, y_g, gw_g, gl_g, what):
    """One chunk of tokens end to end, each side with its own gate weights: combine within
    1e-6 relative (float32) or one ulp of the element type of the oracle's y_o; grad_w
    (which does not depend on the weights) within 1e-6 of sum_m |grad_y * E| (`bound`) of
    the oracle's gw_o; the gate gradient within its bound."""
    if dt == "f32":
        mag = np.zeros(y_o.shape)
        for j in range(S.k):
            sel = S.dst[:, j] >= 0
            mag[sel] += np.abs(wt_o[toks][sel, j, None].astype(np.float64) * E_c[S.dst[sel, j]])
        assert np.all(np.abs(y_g.astype(np.float64) - y_o) <= 1e-6 * mag + 1e-30), f"{what} combine"
    else:
        yg, yo = oracle.to_f32(y_g, dt).astype(np.float64), oracle.to_f32(y_o, dt).astype(np.float64)
        assert np.all(np.abs(yg - yo) <= dtype_ulp(np.maximum(np.abs(yg), np.abs(yo)), dt)), f"{what} combine"
    assert np.all(np.abs(gw_g.astype(np.float64) - gw_o) <= 1e-6 * bound), f"{what} grad_w"
    gl_o = oracle.gate_topk_backward(idx_o[toks], wt_o[toks], gw_o, e)
    assert np.all(gl_g[gl_o == 0] == 0), f"{what} gate gradient off the selection"
    w64, g64 = wt_o[toks].astype(np.float64), gw_o.astype(np.float64)
    scale = np.zeros((len(toks), e))
    dotmag = np.abs(w64 * g64).sum(1, keepdims=True)
    np.put_along_axis(scale, idx_o[toks].astype(np.int64), np.abs(w64) * (np.abs(g64) + dotmag), axis=1)
    assert np.all(np.abs(gl_g.astype(np.float64) - gl_o) <= 8 * 2.0 ** -24 * scale + 1e-38), \
        f"{what} gate gradient"


@pytest.mark.parametrize("name", ALL)
def test_workload_path_matches_oracle(name):
    """The whole path at full size, every token compared: gate, layout, dispatch and
    replay bit-exact; combine, grad_E and grad_x bit-exact given the oracle's weights,
    grad_w within its bound; end to end with the GPU's own weights within tolerance."""
    announce("workload", name)
    inp = W.make_inputs(name)
    w = inp.workload
    dt = w.dtype
    idx_o, wt_o = oracle.gate_topk(inp.logits, w.k)
    Lo = oracle.dispatch_layout(idx_o, w.e, w.capacity)

    # GPU path end to end
    logits = to_dev(inp.logits)
    x = to_dev(inp.x, dt)
    gy = to_dev(inp.grad_y, dt)
    idx, wt = M.moe_gate_topk(logits, w.k)
    Lg = M.moe_dispatch_layout(idx, w.e, w.capacity)
    buf = M.moe_dispatch(Lg, x)
    y = M.moe_combine(Lg, buf, wt)
    replay = M.moe_dispatch_replay(Lg, x, idx)
    gE, gw = M.moe_combine_backward(Lg, gy, replay, wt)
    gx = M.moe_dispatch_backward(Lg, gE)
    gl = M.moe_gate_topk_backward(idx, wt, gw, w.e)
    torch.cuda.synchronize()

    assert_bits_equal(to_host(idx), idx_o, "idx")
    assert f32_ulps(to_host(wt), wt_o).max() <= 1
    check_layout(Lg, Lo, name)
    check_buffer_chunked(buf, inp.x, Lo.src, "dispatch")
    assert torch.equal(replay.view(torch.uint8), buf.view(torch.uint8)), "replay differs"
    del replay, gE

    # op level, bit exact: the oracle's weights fed to the GPU combine and its backward
    wt_o_dev = to_dev(wt_o)
    y_same_w = to_host(M.moe_combine(Lg, buf, wt_o_dev))
    gE_s, gw_s = M.moe_combine_backward(Lg, gy, buf, wt_o_dev)
    gx_s = to_host(M.moe_dispatch_backward(Lg, gE_s))
    gw_s = to_host(gw_s)
    y_g, gw_g, gl_g = to_host(y), to_host(gw), to_host(gl)
    n_checked = 0
    for toks in token_chunks(w.s, CHUNK_TOKENS):
        what = f"{name} tokens {toks[0]}:{toks[-1] + 1}"
        S, used = compact_layout(Lo, toks)
        E_c = inp.x[S.src]  # the identity expert: each row is its token's row
        y_o = oracle.combine(S, E_c, wt_o[toks], dt)
        assert_bits_equal(y_same_w[toks], y_o, f"{what} combine (same weights)")
        gE_o, gw_o = oracle.combine_backward(S, inp.grad_y[toks], E_c, wt_o[toks], dt)
        assert_bits_equal(to_host(gE_s[torch.from_numpy(used).cuda()]), gE_o, f"{what} grad_E (same weights)")
        bound = weight_grad_bound(oracle.to_f32(inp.grad_y[toks], dt), oracle.to_f32(E_c, dt), S.dst)
        assert np.all(np.abs(gw_s[toks].astype(np.float64) - gw_o) <= 1e-6 * bound), f"{what} grad_w"
        assert_bits_equal(gx_s[toks], oracle.dispatch_backward(S, gE_o, dt), f"{what} dispatch backward")
        check_end_to_end_chunk(toks, S, E_c, wt_o, idx_o, dt, w.e, y_o, gw_o, bound, y_g[toks],
                               gw_g[toks], gl_g[toks], what)
        n_checked += len(toks)
    assert n_checked == w.s


@pytest.mark.parametrize("name", ALL)
def test_tagged_expert_rows_at_full_size(name):
    """Combine and its backward at full size, in the bench's launch configuration, over
    expert rows tagged by a power of two per expert, against the oracle on every token:
    bit-exact combine and grad_E, grad_w within its bound."""
    announce("tagged expert", name)
    inp = W.make_inputs(name)
    w = inp.workload
    dt = w.dtype
    idx_o, wt_o = oracle.gate_topk(inp.logits, w.k)
    Lo = oracle.dispatch_layout(idx_o, w.e, w.capacity)
    # expert of every buffer row, from the segments
    expert_of_row = np.repeat(np.arange(w.e), np.diff(Lo.offsets))
    expert_of_row = np.concatenate([expert_of_row, np.zeros(Lo.rows - len(expert_of_row), np.int64)])
    Lg = M.moe_dispatch_layout(to_dev(idx_o), w.e, w.capacity)
    E_dev = torch.empty((Lo.rows, w.m), dtype=TORCH_DTYPE[dt], device="cuda")
    for r0 in range(0, Lo.rows, 32768):  # the tagged rows, built and uploaded in pieces
        r1 = min(Lo.rows, r0 + 32768)
        E_dev[r0:r1] = to_dev(tagged_rows(inp.x, Lo.src[r0:r1], expert_of_row[r0:r1], dt), dt)
    wt_dev, gy_dev = to_dev(wt_o), to_dev(inp.grad_y, dt)
    y = to_host(M.moe_combine(Lg, E_dev, wt_dev))
    gE, gw = M.moe_combine_backward(Lg, gy_dev, E_dev, wt_dev)
    gw = to_host(gw)
    n_checked = 0
    for toks in token_chunks(w.s, CHUNK_TOKENS):
        what = f"{name} tokens {toks[0]}:{toks[-1] + 1}"
        S, used = compact_layout(Lo, toks)
        E_c = tagged_rows(inp.x, S.src, expert_of_row[used], dt)
        assert_bits_equal(y[toks], oracle.combine(S, E_c, wt_o[toks], dt), f"{what} combine over tagged rows")
        gE_o, gw_o = oracle.combine_backward(S, inp.grad_y[toks], E_c, wt_o[toks], dt)
        assert_bits_equal(to_host(gE[torch.from_numpy(used).cuda()]), gE_o, f"{what} grad_E")
        bound = weight_grad_bound(oracle.to_f32(inp.grad_y[toks], dt), oracle.to_f32(E_c, dt), S.dst)
        err = np.abs(gw[toks].astype(np.float64) - gw_o)
        assert np.all(err <= 1e-6 * bound), f"{what} grad_w err {err.max()}"
        n_checked += len(toks)
    assert n_checked == w.s
    # rows no route fills come back zero in grad_E
    unfilled = np.nonzero(Lo.src < 0)[0]
    if len(unfilled):
        assert not bool(gE[torch.from_numpy(unfilled).cuda()].ne(0).any()), "grad_E unfilled rows"


def dtype_ulp(mag: np.ndarray, dt: str) -> np.ndarray:
    """One unit in the last place of bf16 (8-bit precision) or f16 (11-bit) at |v|."""
    p, tiny = (8, 2.0 ** -133) if dt == "bf16" else (11, 2.0 ** -24)
    _, ex = np.frexp(mag)
    return np.maximum(np.ldexp(1.0, ex - p), tiny)


# ----------------------------------------------------------------------------
# replay, determinism, handles, degenerate sizes


def test_replay_reproduces_rows_and_flags_mismatch():
    announce("replay")
    w = W.WORKLOADS["checkpoint_replay_h2816"]
    inp = W.make_inputs(w)
    idx, wt = M.moe_gate_topk(to_dev(inp.logits), w.k)
    x = to_dev(inp.x, w.dtype)
    L1 = M.moe_dispatch_layout(idx, w.e, w.capacity)
    buf = M.moe_dispatch(L1, x)
    rep = M.moe_dispatch_replay(L1, x, idx)
    assert torch.equal(rep.view(torch.uint8), buf.view(torch.uint8))
    # a second layout from identical routing gives identical row counts and maps
    L2 = M.moe_dispatch_layout(idx.clone(), w.e, w.capacity)
    for f in ("counts", "kept", "offsets", "dst", "src"):
        assert torch.equal(getattr(L1, f), getattr(L2, f)), f
    assert M.moe_layout_read(L1) == (0, M.moe_layout_read(L2)[1])
    # replaying with different routing is reported, not hidden
    other = idx.clone()
    other[123, 4] = (other[123, 4] + 1) % w.e
    M.moe_dispatch_replay(L1, x, other)
    flags, _ = M.moe_layout_read(L1)
    assert flags & M.FLAG_REPLAY_MISMATCH
    assert not (M.moe_layout_read(L2)[0] & M.FLAG_REPLAY_MISMATCH)


def test_results_are_deterministic():
    announce("determinism")
    w = W.WORKLOADS["zipf_skew_h4096"]
    inp = W.make_inputs(w)
    outs = []
    for _ in range(2):
        idx, wt = M.moe_gate_topk(to_dev(inp.logits), w.k)
        L = M.moe_dispatch_layout(idx, w.e, w.capacity)
        buf = M.moe_dispatch(L, to_dev(inp.x, w.dtype))
        y = M.moe_combine(L, buf, wt)
        gE, gw = M.moe_combine_backward(L, to_dev(inp.grad_y, w.dtype), buf, wt)
        gx = M.moe_dispatch_backward(L, gE)
        outs.append([t.clone() for t in (idx, wt, L.dst, L.src, y, gw, gx)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


def test_several_live_layouts():
    """fwd(b1), fwd(b2), bwd(b2), bwd(b1): each layout stays valid."""
    announce("live handles")
    rng = np.random.default_rng(3)
    s, e, k, m = 900, 32, 4, 64
    cases = []
    for cap in (0, 50):
        idx = W.random_idx(rng, s, e, k)
        x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16")
        cases.append((idx, x, cap, M.moe_dispatch_layout(to_dev(idx), e, cap)))
    for idx, x, cap, Lg in reversed(cases):
        Lo = oracle.dispatch_layout(idx, e, cap)
        check_layout(Lg, Lo, f"live c={cap}")
        buf = M.moe_dispatch(Lg, to_dev(x, "bf16"))
        gx = M.moe_dispatch_backward(Lg, buf)
        assert_bits_equal(to_host(gx), oracle.dispatch_backward(Lo, oracle.dispatch(Lo, x), "bf16"), "gx")


def _pipeline(logits, x, gy, k, e, cap):
    """Forward and backward of the whole path on the current stream; every output kept."""
    idx, wt = M.moe_gate_topk(logits, k)
    L = M.moe_dispatch_layout(idx, e, cap)
    buf = M.moe_dispatch(L, x)
    y = M.moe_combine(L, buf, wt)
    gE, gw = M.moe_combine_backward(L, gy, buf, wt)
    gx = M.moe_dispatch_backward(L, gE)
    gl = M.moe_gate_topk_backward(idx, wt, gw, e)
    return {"idx": idx, "w": wt, "dst": L.dst, "src": L.src, "counts": L.counts,
            "offsets": L.offsets, "buf": buf, "y": y, "gE": gE, "gw": gw, "gx": gx, "gl": gl}


def test_two_streams_at_once_match_one_after_the_other():
    """Two independent pipelines enqueued on two streams of default priority run
    concurrently, each with its own workspace: no state is shared between calls, so
    each stream's outputs equal, byte for byte, the same pipeline run alone."""
    announce("two streams")
    rng = np.random.default_rng(21)
    s, e, k, m = 4096, 64, 4, 1024
    ins = []
    for cap in (0, 300):
        logits = to_dev(W.routing_logits(rng, s, e, "uniform"))
        x = to_dev(W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16"), "bf16")
        gy = to_dev(W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16"), "bf16")
        ins.append((logits, x, gy, k, e, cap))
    alone = [_pipeline(*a) for a in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    together = [None, None]
    for i, st in enumerate(streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            together[i] = _pipeline(*ins[i])
    torch.cuda.synchronize()
    for i in range(2):
        for name, t in alone[i].items():
            u = together[i][name]
            assert torch.equal(t.contiguous().view(torch.uint8), u.contiguous().view(torch.uint8)), (i, name)


@pytest.mark.parametrize("cap", [0, 4])
def test_empty_batch(cap):
    announce("empty", cap)
    e, k, m = 6, 2, 8
    idx = torch.zeros((0, k), dtype=torch.int32, device="cuda")
    L = M.moe_dispatch_layout(idx, e, cap)
    assert L.rows == (e * cap if cap else 0)
    x = torch.zeros((0, m), dtype=torch.bfloat16, device="cuda")
    buf = M.moe_dispatch(L, x)
    if cap:
        buf_bits = buf.view(torch.int16)
        assert int(buf_bits.abs().sum()) == 0
        assert torch.all(L.src == -1)
    y = M.moe_combine(L, buf, torch.zeros((0, k), device="cuda"))
    assert y.shape == (0, m)
    gE, gw = M.moe_combine_backward(L, x, buf, torch.zeros((0, k), device="cuda"))
    assert gE.shape == (L.rows, m) and gw.shape == (0, k)
    assert torch.all(L.counts == 0)
    lg, lw = M.moe_gate_topk(torch.zeros((0, e), device="cuda"), k)
    assert lg.shape == (0, k)
    torch.cuda.synchronize()


def test_all_routes_dropped_give_zero_rows():
    announce("all dropped")
    s, e, k, m = 40, 2, 2, 16
    idx = np.tile(np.array([[0, 1]], np.int32), (s, 1))
    Lg = M.moe_dispatch_layout(to_dev(idx), e, 1)  # only token 0 fits
    x = -np.abs(np.random.default_rng(0).standard_normal((s, m))).astype(np.float32)
    buf = M.moe_dispatch(Lg, to_dev(x))
    y = to_host(M.moe_combine(Lg, buf, torch.full((s, k), 0.5, device="cuda")))
    assert np.all(bits(y[1:]) == 0)  # +0.0, not -0.0
    assert np.array_equal(y[0], x[0])


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def test_whole_step_replays_correctly_from_a_hip_graph():
    """The path has no memsets, allocations or host syncs: it can be captured. Each
    replay (with eager work in between) must equal the eager result."""
    announce("hip graph")
    s, m, e, k, cap = 2000, 264, 40, 4, 0
    inp = W.random_case(61, s, m, e, k, cap, "bf16")
    logits = to_dev(inp.logits)
    x = to_dev(inp.x, "bf16")
    gy = to_dev(inp.grad_y, "bf16")
    ws = torch.empty(M.workspace_bytes(s, e, k, cap), dtype=torch.uint8, device="cuda")
    idx = torch.empty((s, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((s, k), dtype=torch.float32, device="cuda")
    rows = s * k
    buf = torch.empty((rows, m), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((s, m), dtype=torch.bfloat16, device="cuda")
    gE = torch.empty_like(buf)
    gw = torch.empty_like(wt)
    gx = torch.empty_like(y)
    gl = torch.empty((s, e), dtype=torch.float32, device="cuda")

    def step():
        M.moe_gate_topk(logits, k, idx_out=idx, w_out=wt)
        L = M.moe_dispatch_layout(idx, e, cap, workspace=ws)
        M.moe_dispatch(L, x, out=buf)
        M.moe_combine(L, buf, wt, out=y)
        M.moe_combine_backward(L, gy, buf, wt, grad_expert_out=gE, grad_w=gw)
        M.moe_dispatch_backward(L, gE, out=gx)
        M.moe_gate_topk_backward(idx, wt, gw, e, out=gl)

    outs = (idx, wt, buf, y, gE, gw, gx, gl)
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
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"replay {rep}"
        # eager work between replays
        M.moe_gate_topk(logits.flip(0), k)
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# seeded random configurations through the whole row path


def random_config(seed: int):
    """Sizes, routing mode and dtype drawn from one seeded generator (rows of whole 16-byte
    chunks, k distinct experts per token)."""
    rng = np.random.default_rng(9000 + seed)
    s = int(rng.integers(1, 2500))
    e = int(rng.integers(1, 300))
    k = int(rng.integers(1, min(e, 16) + 1))
    dtype = ["f32", "bf16", "f16"][int(rng.integers(0, 3))]
    m = int(rng.integers(1, 80)) * (4 if dtype == "f32" else 8)
    cap = 0 if rng.random() < 0.5 else int(rng.integers(1, max(2, 2 * s * k // e)))
    route_major = bool(rng.random() < 0.3) and cap > 0
    pad = int([1, 1, 8, 128][int(rng.integers(0, 4))]) if cap == 0 else 1
    skew = bool(rng.random() < 0.3)
    return rng, s, e, k, dtype, m, cap, route_major, pad, skew


@pytest.mark.parametrize("seed", range(64))
def test_random_configurations_bit_exact(seed):
    rng, s, e, k, dtype, m, cap, rm, pad, skew = random_config(seed)
    announce("random config", seed, s, e, k, dtype, m, cap, rm, pad, skew)
    idx = W.skewed_idx(rng, s, e, k) if skew else W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)
    w = W.random_weights(rng, s, k)
    Lo = oracle.dispatch_layout(idx, e, cap, route_major=rm, pad_multiple=pad)
    E = W.cast_input(rng.standard_normal((Lo.rows, m)).astype(np.float32), dtype)
    gy = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dtype)

    Lg = M.moe_dispatch_layout(to_dev(idx), e, cap, route_major=rm, pad_multiple=pad)
    check_layout(Lg, Lo, f"seed {seed}")
    buf = M.moe_dispatch(Lg, to_dev(x, dtype))
    assert_bits_equal(to_host(buf), oracle.dispatch(Lo, x), "dispatch")
    y = M.moe_combine(Lg, to_dev(E, dtype), to_dev(w))
    assert_bits_equal(to_host(y), oracle.combine(Lo, E, w, dtype), "combine")
    gE, gw = M.moe_combine_backward(Lg, to_dev(gy, dtype), to_dev(E, dtype), to_dev(w))
    gE_o, gw_o = oracle.combine_backward(Lo, gy, E, w, dtype)
    assert_bits_equal(to_host(gE), gE_o, "grad_E")
    bound = weight_grad_bound(oracle.to_f32(gy, dtype), oracle.to_f32(E, dtype), Lo.dst)
    err = np.abs(to_host(gw).astype(np.float64) - gw_o)
    assert np.all(err <= 1e-6 * bound), f"grad_w err {err.max()}"
    gx = M.moe_dispatch_backward(Lg, gE)
    assert_bits_equal(to_host(gx), oracle.dispatch_backward(Lo, gE_o, dtype), "dispatch backward")


# ----------------------------------------------------------------------------
# many tiny seeded cases end to end, gate included


@pytest.mark.parametrize("seed", range(200))
def test_tiny_random_end_to_end(seed):
    """Tiny sizes (s <= 64, e <= 16) with logits on a coarse grid, so that ties between
    experts are common, through gate, layout, dispatch, combine, replay and every backward
    pass. Ids, maps, buffers, combine, grad_E and grad_x bit-exact (the rows steps fed the
    oracle's weights); weights and the gate gradient within one float32 ulp; grad_w within
    its bound."""
    rng = np.random.default_rng(20000 + seed)
    s = int(rng.integers(1, 65))
    e = int(rng.integers(1, 17))
    k = int(rng.integers(1, e + 1))
    dt = ["f32", "bf16", "f16"][int(rng.integers(0, 3))]
    m = int(rng.integers(1, 9)) * (4 if dt == "f32" else 8)
    cap = 0 if rng.random() < 0.4 else int(rng.integers(1, max(2, s * k // e + 2)))
    announce("tiny", seed, s, e, k, dt, m, cap)
    logits = (rng.integers(-3, 4, size=(s, e)) / 2).astype(np.float32)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dt)
    gy = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dt)

    idx, wt = M.moe_gate_topk(to_dev(logits), k)
    idx_o, wt_o = oracle.gate_topk(logits, k)
    assert_bits_equal(to_host(idx), idx_o, "idx")
    assert f32_ulps(to_host(wt), wt_o).max() <= 1, "weights"

    Lg = M.moe_dispatch_layout(idx, e, cap)
    Lo = oracle.dispatch_layout(idx_o, e, cap)
    check_layout(Lg, Lo, f"tiny seed {seed}")
    xd = to_dev(x, dt)
    buf = M.moe_dispatch(Lg, xd)
    E_o = oracle.dispatch(Lo, x)
    assert_bits_equal(to_host(buf), E_o, "dispatch")
    assert_bits_equal(to_host(M.moe_dispatch_replay(Lg, xd, idx)), E_o, "replay")
    w_dev = to_dev(wt_o)
    assert_bits_equal(to_host(M.moe_combine(Lg, buf, w_dev)), oracle.combine(Lo, E_o, wt_o, dt), "combine")
    gE, gw = M.moe_combine_backward(Lg, to_dev(gy, dt), buf, w_dev)
    gE_o, gw_o = oracle.combine_backward(Lo, gy, E_o, wt_o, dt)
    assert_bits_equal(to_host(gE), gE_o, "grad_E")
    bound = weight_grad_bound(oracle.to_f32(gy, dt), oracle.to_f32(E_o, dt), Lo.dst)
    assert np.all(np.abs(to_host(gw).astype(np.float64) - gw_o) <= 1e-6 * bound), "grad_w"
    assert_bits_equal(to_host(M.moe_dispatch_backward(Lg, gE)), oracle.dispatch_backward(Lo, gE_o, dt), "grad_x")
    g32 = gw_o.astype(np.float32)
    gl = to_host(M.moe_gate_topk_backward(idx, w_dev, to_dev(g32), e))
    gl_o = oracle.gate_topk_backward(idx_o, wt_o, g32, e)
    assert np.all(gl[gl_o == 0] == 0)
    # w_j (g_j - sum_q w_q g_q) in float64 on both sides, summed in different orders:
    # apart from each side's rounding to float32 (one ulp together) they differ by at most
    # about k * 2^-53 of |w_j| (|g_j| + sum_q |w_q g_q|), which matters where g_j cancels
    # the sum (e.g. every kept route of a token with the same gradient)
    w64, g64 = wt_o.astype(np.float64), g32.astype(np.float64)
    scale = np.zeros((s, e))
    np.put_along_axis(scale, idx_o.astype(np.int64),
                      np.abs(w64) * (np.abs(g64) + np.abs(w64 * g64).sum(1, keepdims=True)), axis=1)
    big = np.maximum(np.abs(gl.astype(np.float64)), np.abs(gl_o))
    ulp = np.ldexp(1.0, np.frexp(np.maximum(big, 2.0 ** -126))[1] - 24)
    assert np.all(np.abs(gl.astype(np.float64) - gl_o) <= ulp + 2.0 ** -45 * scale), "gate gradient"
    assert M.moe_layout_read(Lg)[0] == 0
