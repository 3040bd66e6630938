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
    """gate -> dispatch -> identity expert -> combine."""
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
@pytest.mark.parametrize("cap", [0, 60])
def test_checkpoint_replays_layout_and_is_bit_identical(cap):
    print("CASE checkpoint", cap, flush=True)
    s, m, e, k = 1200, 128, 16, 4
    inp = W.random_case(41, s, m, e, k, cap, "bf16")

    def run(ckpt):
        x = to_dev(inp.x, "bf16").requires_grad_(True)
        logits = to_dev(inp.logits).requires_grad_(True)
        gy = to_dev(inp.grad_y, "bf16")
        if ckpt:
            y, rec = A.checkpoint(lambda r, a, b: block(r, a, b, k, e, cap), x, logits, verify=True)
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
    rec.check()


@pytest.mark.gpu
def test_checkpoint_with_changed_routing_fails_loudly():
    print("CASE checkpoint mismatch", flush=True)
    s, m, e, k = 600, 64, 8, 2
    inp = W.random_case(43, s, m, e, k, 0, "bf16")
    calls = {"n": 0}

    def fn(rec, x, logits):
        calls["n"] += 1
        if calls["n"] > 1:  # the recompute routes differently
            logits = logits.flip(1)
        return block(rec, x, logits, k, e, 0)

    x = to_dev(inp.x, "bf16").requires_grad_(True)
    logits = to_dev(inp.logits).requires_grad_(True)
    y, rec = A.checkpoint(fn, x, logits, verify=True)
    y.float().sum().backward()
    assert rec.replays == 1
    with pytest.raises(RuntimeError):
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
@pytest.mark.parametrize("cap", [0, 70])
def test_expert_linear_layer_gradients_match_a_float32_reference(cap):
    """gate -> layout -> expert_linear (one projection per expert, dispatch fused into the
    GEMM) -> combine, against the same layer written with dense float32 PyTorch ops on the
    CPU. Checks the wiring of all three gradients (tokens, expert weights, router); the
    kernels' own parity is tested against the oracle elsewhere."""
    print("CASE expert_linear autograd", cap, flush=True)
    s, m, n, e, k = 512, 64, 96, 8, 2
    rng = np.random.default_rng(77)
    logits_np = rng.standard_normal((s, e)).astype(np.float32)
    x_np = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16")
    w_np = W.expert_weights(78, e, n, m, "bf16")
    gy_np = W.cast_input(rng.standard_normal((s, n)).astype(np.float32), "bf16")

    x = to_dev(x_np, "bf16").requires_grad_(True)
    weights = to_dev(w_np, "bf16").requires_grad_(True)
    logits = to_dev(logits_np).requires_grad_(True)
    idx, w = A.route(logits, k)
    L, _ = A.layout(idx, e, cap)
    y = A.combine(A.expert_linear(x, weights, L), w, L)
    (y.float() * to_dev(gy_np, "bf16").float()).sum().backward()

    # dense float32 reference on the CPU, with the GPU's expert choice and placed routes
    idx_l = torch.from_numpy(to_host(idx).astype(np.int64))
    placed = torch.from_numpy(to_host(L.dst) >= 0).float()
    xr = torch.from_numpy(oracle.to_f32(x_np, "bf16")).requires_grad_(True)
    wr = torch.from_numpy(oracle.to_f32(w_np.reshape(e * n, m), "bf16").reshape(e, n, m)).requires_grad_(True)
    lr = torch.from_numpy(logits_np).requires_grad_(True)
    gate = torch.softmax(torch.gather(lr, 1, idx_l), dim=1) * placed  # softmax over the k chosen
    h = torch.einsum("sm,sknm->skn", xr, wr[idx_l])
    yr = (gate[:, :, None] * h).sum(1)
    (yr * torch.from_numpy(oracle.to_f32(gy_np, "bf16"))).sum().backward()

    for name, got, ref in [("grad_x", to_host(x.grad), xr.grad), ("grad_weights", to_host(weights.grad), wr.grad),
                           ("grad_logits", to_host(logits.grad), lr.grad)]:
        g = oracle.to_f32(got, "bf16") if got.dtype == np.uint16 else got
        r = ref.numpy().astype(np.float64)
        err = np.abs(g.astype(np.float64) - r)
        assert np.all(err <= 2e-2 * np.abs(r) + 2e-2 * np.abs(r).max()), (name, err.max(), np.abs(r).max())
