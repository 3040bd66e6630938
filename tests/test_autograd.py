"""Autograd wiring and the activation-checkpoint layout recorder."""
import numpy as np
import pytest
import torch

import combine_moe_gate_amd as M
import combine_moe_gate_amd.autograd as A
import oracle
import workloads as W


# ----------------------------------------------------------------------------
# recorder bookkeeping on the CPU (the layout builder is stubbed)


def test_recorder_records_then_replays_in_order(monkeypatch):
    built = []

    def fake_layout(idx, e, capacity):
        built.append((tuple(idx.shape), e, capacity))
        return object()

    monkeypatch.setattr(A, "moe_dispatch_layout", fake_layout)
    rec = A.LayoutRecorder()
    idx_a, idx_b = torch.zeros(4, 2, dtype=torch.int32), torch.zeros(6, 2, dtype=torch.int32)
    with rec:  # forward: two dispatches, in this order
        la, va = rec.layout_for(idx_a, 8, 0)
        lb, vb = rec.layout_for(idx_b, 8, 3)
    assert rec.layouts_built == 2 and va is None and vb is None
    with rec:  # recompute: handed back in the same order, nothing rebuilt
        ra, _ = rec.layout_for(idx_a, 8, 0)
        rb, _ = rec.layout_for(idx_b, 8, 3)
        assert ra is la and rb is lb
        # a recompute that outruns its log falls back to a full layout
        rc, _ = rec.layout_for(idx_a, 8, 0)
        assert rc is not la
    assert rec.replays == 2 and rec.fallbacks == 1 and rec.layouts_built == 3
    with rec:  # a mismatched request fails loudly instead of replaying the wrong layout
        with pytest.raises(RuntimeError):
            rec.layout_for(idx_b, 8, 3)


def test_recorder_pins_routing_on_recompute(monkeypatch):
    """The recompute gets the forward's ids and weights back (top-k is not run again), a
    layout replayed for that routing is not re-verified, and routing from elsewhere is."""
    gate_calls = []

    class FakeGate:
        @staticmethod
        def apply(logits, k):
            gate_calls.append(logits.shape)
            idx = torch.argsort(logits, dim=1, descending=True)[:, :k].to(torch.int32)
            return idx, torch.softmax(torch.gather(logits, 1, idx.long()), 1)

    monkeypatch.setattr(A, "_Gate", FakeGate)
    monkeypatch.setattr(A, "moe_dispatch_layout", lambda idx, e, capacity, **o: object())
    rec = A.LayoutRecorder()
    assert rec.verify  # on by default
    logits = torch.randn(6, 8)
    with rec:
        idx_f, w_f = rec.route_for(logits, 2)
        lay_f, v_f = rec.layout_for(idx_f, 8, 0)
    assert v_f is None and len(gate_calls) == 1
    with rec:  # recompute with different logits: the recorded routing comes back
        idx_r, w_r = rec.route_for(logits.flip(1) + 3.0, 2)
        lay_r, v_r = rec.layout_for(idx_r, 8, 0)
        assert idx_r is idx_f and torch.equal(w_r, w_f) and lay_r is lay_f
        assert v_r is None  # pinned: nothing to verify
    with rec:  # another recompute whose routing does not come from the recorder's gate
        other = idx_f.clone()
        other[0, 0] = 7
        lay_o, v_o = rec.layout_for(other, 8, 0)
        assert lay_o is lay_f and v_o is other  # replayed, and verified against the record
    assert len(gate_calls) == 1 and rec.routes_replayed == 1 and rec.replays == 2
    with rec:
        with pytest.raises(RuntimeError):  # a recompute routing another shape fails loudly
            rec.route_for(torch.randn(5, 8), 2)


# ----------------------------------------------------------------------------
# on the GPU


def to_dev(a, dtype=None):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def block(rec, x, logits, k, e, cap):
    """gate -> dispatch -> identity expert -> combine, routing pinned through the recorder."""
    idx, w = A.route(logits, k, rec)
    buf, L = A.dispatch(x, idx, e, cap, rec)
    return A.combine(buf, w, L)


def block_unpinned(rec, x, logits, k, e, cap):
    """The same with the gate outside the recorder: only the layout is recorded."""
    idx, w = A.route(logits, k)
    buf, L = A.dispatch(x, idx, e, cap, rec)
    return A.combine(buf, w, L)


CASES = [(700, 64, "bf16", 12, 3, 0), (700, 64, "f32", 12, 3, 100), (300, 136, "f16", 8, 2, 40)]


@pytest.mark.gpu
@pytest.mark.parametrize("s,m,dtype,e,k,cap", CASES)
def test_autograd_gradients_match_oracle(s, m, dtype, e, k, cap):
    print("CASE autograd", s, m, dtype, e, k, cap, flush=True)
    inp = W.random_case(31, s, m, e, k, cap, dtype)
    x = to_dev(inp.x, dtype).requires_grad_(True)
    logits = to_dev(inp.logits).requires_grad_(True)
    gy = to_dev(inp.grad_y, dtype)
    y = block(None, x, logits, k, e, cap)
    (y.float() * gy.float()).sum().backward()

    idx_o, w_o = oracle.gate_topk(inp.logits, k)
    L = oracle.dispatch_layout(idx_o, e, cap)
    E = oracle.dispatch(L, inp.x)
    gE_o, gw_o = oracle.combine_backward(L, inp.grad_y, E, w_o, dtype)
    gx_o = oracle.dispatch_backward(L, gE_o, dtype)
    gl_o = oracle.gate_topk_backward(idx_o, w_o, gw_o, e)
    gx = to_host(x.grad)
    # grad_x passes through grad_E = w * grad_y, so it inherits the weights' last-ulp
    # freedom: compare in float32 within one ulp of the element type per route
    gx32 = oracle.to_f32(gx, dtype).astype(np.float64)
    gxo32 = oracle.to_f32(gx_o, dtype).astype(np.float64)
    p = {"f32": 24, "bf16": 8, "f16": 11}[dtype]
    scale = np.abs(oracle.to_f32(inp.grad_y, dtype)).astype(np.float64) * k
    assert np.all(np.abs(gx32 - gxo32) <= scale * 2.0 ** (1 - p) + 1e-30)
    gl = to_host(logits.grad)
    assert np.all(gl[gl_o == 0] == 0)
    denom = np.abs(gl_o).max()
    assert np.abs(gl.astype(np.float64) - gl_o).max() <= 1e-5 * denom


@pytest.mark.gpu
@pytest.mark.parametrize("perturb", [False, True])
@pytest.mark.parametrize("cap", [0, 60])
def test_checkpoint_replays_layout_and_is_bit_identical(cap, perturb):
    """A checkpointed step equals the plain one bit for bit, with one layout built and one
    replayed; with routing pinned through the recorder this holds even when the
    recompute's logits differ from the forward's (the recorded routing is used)."""
    print("CASE checkpoint", cap, perturb, flush=True)
    s, m, e, k = 1200, 128, 16, 4
    inp = W.random_case(41, s, m, e, k, cap, "bf16")
    calls = {"n": 0}

    def fn(rec, x, logits):
        calls["n"] += 1
        if perturb and calls["n"] > 1:  # the recompute's logits differ (gradient passes through)
            logits = logits + torch.randn(logits.shape, generator=torch.Generator(device="cuda").manual_seed(5),
                                          device="cuda")
        return block(rec, x, logits, k, e, cap)

    def run(ckpt):
        x = to_dev(inp.x, "bf16").requires_grad_(True)
        logits = to_dev(inp.logits).requires_grad_(True)
        gy = to_dev(inp.grad_y, "bf16")
        if ckpt:
            y, rec = A.checkpoint(fn, x, logits)
        else:
            y, rec = block(None, x, logits, k, e, cap), None
        loss = (y.float() * gy.float()).sum()
        loss.backward()
        torch.cuda.synchronize()
        return loss.item(), x.grad.clone(), logits.grad.clone(), rec

    loss0, gx0, gl0, _ = run(False)
    loss1, gx1, gl1, rec = run(True)
    assert loss0 == loss1
    assert torch.equal(gx0.view(torch.int16), gx1.view(torch.int16))
    assert torch.equal(gl0, gl1)
    assert rec.layouts_built == 1 and rec.replays == 1 and rec.fallbacks == 0
    assert rec.routes_replayed == 1 and rec.route_fallbacks == 0
    rec.check()


@pytest.mark.gpu
def test_checkpoint_with_changed_unpinned_routing_fails_loudly():
    """Routing that bypasses the recorder and changes on the recompute makes the backward
    itself raise: the caller does not have to ask."""
    print("CASE checkpoint mismatch", flush=True)
    s, m, e, k = 600, 64, 8, 2
    inp = W.random_case(43, s, m, e, k, 0, "bf16")
    calls = {"n": 0}

    def fn(rec, x, logits):
        calls["n"] += 1
        if calls["n"] > 1:  # the recompute routes differently
            logits = logits.flip(1)
        return block_unpinned(rec, x, logits, k, e, 0)

    x = to_dev(inp.x, "bf16").requires_grad_(True)
    logits = to_dev(inp.logits).requires_grad_(True)
    y, rec = A.checkpoint(fn, x, logits)
    with pytest.raises(RuntimeError, match="differs from the forward"):
        y.float().sum().backward()
    assert rec.replays == 1


@pytest.mark.gpu
def test_checkpoint_with_unchanged_unpinned_routing_passes_verification():
    print("CASE checkpoint unpinned", flush=True)
    s, m, e, k = 600, 64, 8, 2
    inp = W.random_case(44, s, m, e, k, 0, "bf16")
    x = to_dev(inp.x, "bf16").requires_grad_(True)
    logits = to_dev(inp.logits).requires_grad_(True)
    y, rec = A.checkpoint(lambda r, a, b: block_unpinned(r, a, b, k, e, 0), x, logits)
    y.float().sum().backward()
    assert rec.replays == 1 and rec.routes_replayed == 0
    rec.check()


@pytest.mark.gpu
def test_two_forwards_then_two_backwards():
    """fwd(b1), fwd(b2), then one backward through both: each keeps its own layout."""
    print("CASE two forwards", flush=True)
    s, m, e, k = 500, 64, 8, 2
    outs = []
    for seed in (51, 52):
        inp = W.random_case(seed, s, m, e, k, 0, "f32")
        x = to_dev(inp.x).requires_grad_(True)
        logits = to_dev(inp.logits).requires_grad_(True)
        outs.append((inp, x, logits, block(None, x, logits, k, e, 0)))
    (outs[0][3].sum() + outs[1][3].sum()).backward()
    for inp, x, logits, _ in outs:
        idx_o, w_o = oracle.gate_topk(inp.logits, k)
        L = oracle.dispatch_layout(idx_o, e, 0)
        E = oracle.dispatch(L, inp.x)
        gE_o, gw_o = oracle.combine_backward(L, np.ones_like(inp.x), E, w_o, "f32")
        gx_o = oracle.dispatch_backward(L, gE_o, "f32")
        assert np.allclose(to_host(x.grad), gx_o, rtol=1e-6, atol=1e-6)


@pytest.mark.gpu
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("cap", [0, 70])
def test_expert_linear_layer_gradients_match_the_oracle_chain(cap, dt):
    """gate -> layout -> expert_linear (one projection per expert, the dispatch fused into
    the GEMM) -> combine through autograd, against the oracle's chain of the same steps:
    combine_backward, expert_gemm_dgrad + dispatch_backward, expert_gemm_wgrad (in the
    weights' type) and the gate backward. The inputs make every step exact: each token's
    two chosen experts tie on the largest logit, so both weights are exactly 1/2; x, the
    expert weights and grad_y are in {-1, 0, 1}; every sum stays below 2^8 in the element
    type and below 2^24 in float32. All three gradients must then equal the oracle's bit
    for bit, so a gradient off by any factor (say 1.01) fails."""
    print("CASE expert_linear autograd", cap, dt, flush=True)
    s, m, n, e, k = 512, 64, 96, 8, 2
    rng = np.random.default_rng(77 + cap)
    logits_np = rng.uniform(-1.0, 1.0, (s, e)).astype(np.float32)
    for t in range(s):
        logits_np[t, rng.choice(e, 2, replace=False)] = 2.0
    x_np = W.cast_input(rng.integers(-1, 2, (s, m)).astype(np.float32), dt)
    w_np = W.cast_input(rng.integers(-1, 2, (e, n, m)).astype(np.float32), dt)
    gy_np = W.cast_input(rng.integers(-1, 2, (s, n)).astype(np.float32), dt)

    x = to_dev(x_np, dt).requires_grad_(True)
    weights = to_dev(w_np, dt).requires_grad_(True)
    logits = to_dev(logits_np).requires_grad_(True)
    idx, w = A.route(logits, k)
    L, _ = A.layout(idx, e, cap)
    y = A.combine(A.expert_linear(x, weights, L), w, L)
    y.backward(to_dev(gy_np, dt))

    idx_o, w_o = oracle.gate_topk(logits_np, k)
    assert np.all(w_o == 0.5)
    Lo = oracle.dispatch_layout(idx_o, e, cap)
    assert Lo.kept.sum() < s * k or cap == 0  # the capacity case drops routes
    H_o, _ = oracle.expert_gemm(Lo, x_np, w_np, dt, gather=True)
    y_o = oracle.combine(Lo, H_o, w_o, dt)
    gH_o, gw_o = oracle.combine_backward(Lo, gy_np, H_o, w_o, dt)
    gA_o, _ = oracle.expert_gemm_dgrad(Lo, gH_o, w_np, dt)
    gx_o = oracle.dispatch_backward(Lo, gA_o, dt)
    gW_o, _ = oracle.expert_gemm_wgrad(Lo, x_np, gH_o, dt, gather=True, out_dtype=dt)
    gl_o = oracle.gate_topk_backward(idx_o, w_o, gw_o, e)

    assert np.array_equal(to_host(idx), idx_o)
    assert np.array_equal(to_host(y).view(np.uint16), y_o.view(np.uint16)), "forward"
    assert np.array_equal(to_host(x.grad).view(np.uint16), gx_o.view(np.uint16)), "grad_x"
    assert np.array_equal(to_host(weights.grad).view(np.uint16), gW_o.view(np.uint16)), "grad_weights"
    assert np.array_equal(to_host(logits.grad), gl_o), "grad_logits"
    # the checks see something: every gradient has nonzero entries
    assert np.any(oracle.to_f32(gx_o, dt)) and np.any(oracle.to_f32(gW_o, dt)) and np.any(gl_o)
