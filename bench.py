"""Benchmark of the MoE gate / dispatch / combine hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole path over one batch of resident synthetic input:
gate top-k, dispatch layout, dispatch, weighted combine, dispatch replay from the
saved layout (activation-checkpoint recompute), combine backward, dispatch backward
and gate backward. W untimed steps, then K timed steps bracketed by
torch.cuda.synchronize(). Every launch of a step goes to the current HIP stream;
HIP events recorded on that stream around each call give per-kernel durations over
the same timed region.

Prints ONE JSON line. `value` is the headline metric: dispatch + combine tokens/s,
from the median of at least 100 dispatch + combine pairs, each run after a 1 GiB read
of scratch (outside its events) so that neither L2 nor the Infinity Cache holds its
data; "dispatch_combine" gives that pair's GB/s, fraction of HBM peak, p10/p90/min,
and the warm pair inside the back-to-back steps beside it. The whole step's rate is
"step_tokens_per_s" (and ms_per_step). "roofline" covers the kernel with the largest
share of the step; "cpu_baseline" times the CPU oracle's dispatch + combine on the same
full host arrays, one core, median of 3.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (s=8192,m=4096,e=128,k=8)"
HBM_PEAK_GBPS = 8000.0
# The same step with one of the variants: route-major capacity priority, dropless
# segments padded to 128 rows, weights applied at dispatch (before the experts), or
# weights renormalised over the kept routes after the capacity drop; or the forward of a
# layer whose experts are one linear projection each: gate, layout, the grouped expert
# GEMM with the dispatch fused into its operand loads, weighted combine.
VARIANTS = ("route_major", "pad128", "weights_before", "renorm_kept", "expert_gemm")
MFMA_BF16_PEAK_TFLOPS = 2500.0
# cold-cache headline pair: a read of this much scratch before each of at least
# COLD_PAIRS timed dispatch + combine pairs (more than L2 and the 256 MB Infinity Cache
# together), after COLD_WARMUP untimed ones
COLD_FLUSH_MIB = 1024
COLD_PAIRS = 100
COLD_WARMUP = 10
ISOLATED_RUNS = 30  # each op of the step alone after a flush


# sources of the grouped expert GEMM: only the expert_gemm variant runs their kernels
GEMM_SOURCES = ("gemm.hip", "gemm_bwd.hip", "gemm_common.h")
# host code only (argument checks, the workspace plan, the C declarations): no kernel
HOST_SOURCES = ("api.hip", "moe_gate.h")


_COMMENT = re.compile(rb"//[^\n]*|/\*.*?\*/", re.S)


def source_code_bytes(text: bytes) -> bytes:
    """A source's code without its comments and with runs of whitespace folded to one
    space: what a digest of kernel code should see (the kernel sources hold no string
    literals with comment markers)."""
    return b" ".join(_COMMENT.sub(b" ", text).split())


def kernel_source_digest(variant: str | None = None) -> str:
    """sha256 over the code of the HIP sources (and the build flags) whose kernels a run
    of `variant` launches: every kernel source for the expert_gemm variant, all but the
    GEMM's otherwise. Host-only files are left out, and so are comments and layout:
    neither changes a kernel's traffic."""
    import hashlib
    from combine_moe_gate_amd import _build
    h = hashlib.sha256()
    for path in sorted(_build.SOURCES + _build.HEADERS):
        name = os.path.basename(path)
        if name in HOST_SOURCES or (variant != "expert_gemm" and name in GEMM_SOURCES):
            continue
        with open(path, "rb") as f:
            h.update(source_code_bytes(f.read()))
    h.update(" ".join(_build.FLAGS).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, variant: str | None = None) -> dict:
    """Counter-measured HBM bytes per launch from profiles/, if taken on these sources."""
    name = f"traffic_{workload}" + (f"_{variant}" if variant else "") + ".txt"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    traffic, digest = {}, None
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 3 and parts[0] == "traffic":
                traffic[parts[1]] = int(parts[2])
            elif len(parts) == 2 and parts[0] == "source_digest":
                digest = parts[1]
    return traffic if digest == kernel_source_digest(variant) else {}


def algorithmic_bytes(w: W.Workload, kept_routes: int, rows: int | None = None,
                      variant: str | None = None, active_experts: int | None = None) -> dict:
    """Bytes each call must move (zero padding counts: it is part of the output).

    b = element size; K = placed routes. Routing metadata is int32/float32. The expert
    GEMMs read the weights of the experts that receive rows only (`active_experts`, all
    e if not given); the weight gradient writes all e experts' (zeros for idle ones).
    """
    s, m, e, k, b = w.s, w.m, w.e, w.k, W.ELEM_BYTES[w.dtype]
    rows = w.rows if rows is None else rows
    K = kept_routes
    row = m * b
    out = {
        "gate": s * e * 4 + s * k * 8,
        # count + place read the ids twice; dst, route copy, src written; tile tables
        "layout": 2 * s * k * 4 + 2 * s * k * 4 + rows * 4,
        "dispatch": s * row + rows * row + s * k * 4,
        "combine": K * row + s * k * 8 + s * row,
        # the replay also compares the routing with the saved copy
        "replay": s * row + rows * row + s * k * 4 + 2 * s * k * 4,
        "combine_bwd": s * row + K * row + rows * row + s * k * 12,
        "dispatch_bwd": K * row + s * k * 4 + s * row,
        "gate_bwd": s * k * 12 + s * e * 4,
        "renorm": s * k * 12,
        "renorm_bwd": s * k * 16,
    }
    if variant == "expert_gemm":
        n, nb = W.EXPERT_WIDTH, W.EXPERT_WIDTH * b
        ea = e if active_experts is None else active_experts
        # x read once, the active experts' weights once, the [rows, n] output and its row map
        out["expert_gemm"] = s * row + ea * n * row + rows * nb + rows * 4
        out["combine"] = K * nb + s * k * 8 + s * nb
        out["dispatch"] = s * row + rows * row + s * k * 4
        out["expert_gemm_unfused"] = rows * row + ea * n * row + rows * nb + rows * 4
        # x read once, the [rows, n] gradient once, float32 [e, n, m] written (or the same
        # rounded to the element type)
        out["expert_gemm_wgrad"] = s * row + rows * nb + e * n * m * 4 + rows * 4
        out["expert_gemm_wgrad_narrow"] = s * row + rows * nb + e * n * row + rows * 4
        # the [rows, n] gradient and the active experts' weights read once, [rows, m] written
        out["expert_gemm_dgrad"] = rows * nb + ea * n * row + rows * row
    if variant == "weights_before":
        # dispatch and replay read the weights; the combine is unweighted; the combine
        # backward is a plain dispatch of grad_y; the dispatch backward also reads x
        out["dispatch"] = s * row + rows * row + s * k * 8
        out["replay"] = out["dispatch"]
        out["combine"] = K * row + s * k * 4 + s * row
        out["combine_bwd"] = s * row + rows * row + s * k * 4
        out["dispatch_bwd"] = K * row + s * row + s * row + s * k * 12
    return out


_WEIGHTS = {}


def cold_pair_summary(s: int, disp_us, comb_us, nbytes: int) -> dict:
    """The headline pair with cold caches, from per-pair event microseconds: the median
    (the rate quoted), its spread and the minimum."""
    d = np.asarray(disp_us, dtype=np.float64)
    c = np.asarray(comb_us, dtype=np.float64)
    pair = d + c
    us = float(np.median(pair))
    gbps = nbytes / us / 1e3
    return {"what": f"median of {pair.size} dispatch + combine pairs, each after a {COLD_FLUSH_MIB} MiB read "
                    "of scratch outside its events (neither L2 nor the Infinity Cache holds the pair's data)",
            "pairs": int(pair.size), "tokens_per_s": round(s / (us / 1e6), 1), "GBps": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "us_median": round(us, 2),
            "us_p10": round(float(np.percentile(pair, 10)), 2), "us_p90": round(float(np.percentile(pair, 90)), 2),
            "us_min": round(float(np.min(pair)), 2), "us_mean": round(float(np.mean(pair)), 2),
            "dispatch_us_median": round(float(np.median(d)), 2), "combine_us_median": round(float(np.median(c)), 2),
            "bytes": int(nbytes)}


def expert_weights(w: W.Workload):
    """The seeded expert projection weights [e, EXPERT_WIDTH, m] (generated once)."""
    if w.name not in _WEIGHTS:
        _WEIGHTS[w.name] = W.expert_weights(w.seed + 1, w.e, W.EXPERT_WIDTH, w.m, w.dtype)
    return _WEIGHTS[w.name]


def to_dev(a, dtype, dev):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def run_gpu(w: W.Workload, steps: int, warmup: int, variant: str | None = None, flush_mib: int = 0,
            cold_pairs: int = COLD_PAIRS, isolated_runs: int = ISOLATED_RUNS):
    import torch

    import combine_moe_gate_amd as M

    if not os.path.exists(M.LIB_PATH):
        from combine_moe_gate_amd import _build
        _build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = W.make_inputs(w)
    logits = to_dev(inp.logits, "f32", dev)
    x = to_dev(inp.x, w.dtype, dev)
    gy = to_dev(inp.grad_y, w.dtype, dev)
    tdt = x.dtype
    s, k, e, m, cap = w.s, w.k, w.e, w.m, w.capacity
    opts = dict(route_major=variant == "route_major", pad_multiple=128 if variant == "pad128" else 1)
    idx = torch.empty((s, k), dtype=torch.int32, device=dev)
    wt = torch.empty((s, k), dtype=torch.float32, device=dev)
    ws = torch.empty(M.workspace_bytes(s, e, k, cap, **opts), dtype=torch.uint8, device=dev)
    M.moe_gate_topk(logits, k, idx_out=idx, w_out=wt)
    rows = M.moe_dispatch_layout(idx, e, cap, workspace=ws, **opts).rows  # host-known
    buf = torch.empty((rows, m), dtype=tdt, device=dev)
    rep = torch.empty((rows, m), dtype=tdt, device=dev)
    y = torch.empty((s, m), dtype=tdt, device=dev)
    gE = torch.empty((rows, m), dtype=tdt, device=dev)
    gw = torch.empty((s, k), dtype=torch.float32, device=dev)
    gx = torch.empty((s, m), dtype=tdt, device=dev)
    gl = torch.empty((s, e), dtype=torch.float32, device=dev)
    wr = torch.empty_like(wt)
    gwr = torch.empty_like(gw)
    st = {}

    def gate():
        M.moe_gate_topk(logits, k, idx_out=idx, w_out=wt)

    def layout():
        st["L"] = M.moe_dispatch_layout(idx, e, cap, workspace=ws, **opts)

    def gate_bwd():
        M.moe_gate_topk_backward(idx, wt, gw, e, out=gl)

    extra = {}
    if variant == "expert_gemm":
        n = W.EXPERT_WIDTH
        wts = to_dev(expert_weights(w), w.dtype, dev)
        H = torch.empty((rows, n), dtype=tdt, device=dev)
        yH = torch.empty((s, n), dtype=tdt, device=dev)
        H2 = torch.empty((rows, n), dtype=tdt, device=dev)
        ops = [
            ("gate", gate), ("layout", layout),
            ("expert_gemm", lambda: M.moe_expert_gemm(st["L"], x, wts, gather=True, out=H)),
            ("combine", lambda: M.moe_combine(st["L"], H, wt, out=yH)),
        ]
        # the same projection unfused, timed after the step: dispatch, then the GEMM on
        # the dispatched buffer
        gW = torch.empty((e, n, m), dtype=torch.float32, device=dev)
        gWn = torch.empty((e, n, m), dtype=tdt, device=dev)
        extra["unfused"] = [
            ("dispatch", lambda: M.moe_dispatch(st["L"], x, out=buf)),
            ("expert_gemm_unfused", lambda: M.moe_expert_gemm(st["L"], buf, wts, gather=False, out=H2)),
            # the weight gradient, rows gathered from x again; the forward's output stands
            # in for the gradient arriving at it
            ("expert_gemm_wgrad", lambda: M.moe_expert_gemm_wgrad(st["L"], x, H, gather=True, out=gW)),
            # the same, kept in the element type (the autograd layer's weight gradient)
            ("expert_gemm_wgrad_narrow", lambda: M.moe_expert_gemm_wgrad(st["L"], x, H, gather=True, out=gWn)),
            ("expert_gemm_dgrad", lambda: M.moe_expert_gemm_dgrad(st["L"], H, wts, out=buf)),
        ]
        # the whole layer as a training step through the autograd wrappers: gate, layout,
        # the fused projection and the weighted combine forward; then the gradients of
        # the tokens, the expert weights (kept in their type) and the router logits
        from combine_moe_gate_amd import autograd as A
        wts.requires_grad_(True)
        gyn = torch.randn((s, n), generator=torch.Generator(device=dev).manual_seed(7), device=dev,
                          dtype=torch.float32).to(tdt)

        def layer_step():
            xl = x.detach().requires_grad_(True)
            ll = logits.detach().requires_grad_(True)
            idx_l, w_l = A.route(ll, k)
            L_l, _ = A.layout(idx_l, e, cap)
            y_l = A.combine(A.expert_linear(xl, wts, L_l), w_l, L_l)
            torch.autograd.grad(y_l, (xl, wts, ll), gyn)

        extra["layer"] = [("layer_train_step", layer_step)]
    elif variant == "weights_before":
        ops = [
            ("gate", gate), ("layout", layout),
            ("dispatch", lambda: M.moe_dispatch_weighted(st["L"], x, wt, out=buf)),
            ("combine", lambda: M.moe_combine(st["L"], buf, None, out=y)),
            ("replay", lambda: M.moe_dispatch_weighted(st["L"], x, wt, out=rep)),
            # the gradient of an unweighted combine is a plain dispatch of grad_y
            ("combine_bwd", lambda: M.moe_dispatch(st["L"], gy, out=gE)),
            ("dispatch_bwd", lambda: M.moe_dispatch_weighted_backward(st["L"], gE, x, wt, grad_x=gx,
                                                                      grad_w=gw)),
            ("gate_bwd", gate_bwd),
        ]
    elif variant == "renorm_kept":
        ops = [
            ("gate", gate), ("layout", layout),
            ("renorm", lambda: M.moe_renormalize_kept(st["L"], wt, out=wr)),
            ("dispatch", lambda: M.moe_dispatch(st["L"], x, out=buf)),
            ("combine", lambda: M.moe_combine(st["L"], buf, wr, out=y)),
            ("replay", lambda: M.moe_dispatch_replay(st["L"], x, idx, out=rep)),
            ("combine_bwd", lambda: M.moe_combine_backward(st["L"], gy, rep, wr, grad_expert_out=gE,
                                                           grad_w=gwr)),
            ("renorm_bwd", lambda: M.moe_renormalize_kept_backward(st["L"], wt, gwr, out=gw)),
            ("dispatch_bwd", lambda: M.moe_dispatch_backward(st["L"], gE, out=gx)),
            ("gate_bwd", gate_bwd),
        ]
    else:
        ops = [
            ("gate", gate), ("layout", layout),
            ("dispatch", lambda: M.moe_dispatch(st["L"], x, out=buf)),
            ("combine", lambda: M.moe_combine(st["L"], buf, wt, out=y)),
            # checkpoint recompute: the dispatch replayed from the saved layout
            ("replay", lambda: M.moe_dispatch_replay(st["L"], x, idx, out=rep)),
            ("combine_bwd", lambda: M.moe_combine_backward(st["L"], gy, rep, wt, grad_expert_out=gE,
                                                           grad_w=gw)),
            ("dispatch_bwd", lambda: M.moe_dispatch_backward(st["L"], gE, out=gx)),
            ("gate_bwd", gate_bwd),
        ]
    names = [n for n, _ in ops]

    def step(ev=None):
        for i, (_, fn) in enumerate(ops):
            if ev is not None:
                ev[i].record()
            fn()
        if ev is not None:
            ev[len(ops)].record()

    # cold-cache mode: before each step, outside its events, read flush_mib MiB of scratch
    # so that neither L2 nor the Infinity Cache holds the step's data (a read leaves clean
    # lines behind, whose eviction costs the step no write-back)
    scratch = torch.zeros((flush_mib << 20) // 4, dtype=torch.float32, device=dev) if flush_mib > 0 else None
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if scratch is not None:
            scratch.sum()
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if scratch is not None:  # the steps alone, from their events: the flushes are not counted
        elapsed = sum(ev[0].elapsed_time(ev[len(ops)]) for ev in events) / 1e3
        del scratch

    per_op = {op: [] for op in names}
    for ev in events:
        for j, op in enumerate(names):
            per_op[op].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)  # microseconds
    if flush_mib == 0:
        # the same eager step without the per-op events (only one event pair around all the
        # steps): on launch-bound batches the events' own host time stretches the step
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            step()
        b.record()
        torch.cuda.synchronize()
        per_op["_plain_step"] = [a.elapsed_time(b) * 1e3 / steps]
        # the same step captured once in a HIP graph and replayed, outside the timed region:
        # the host then launches one graph instead of each kernel (the path has no memsets,
        # allocations or host syncs, so it captures as it is)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        gev[0].record()
        for i in range(steps):
            graph.replay()
            gev[i + 1].record()
        torch.cuda.synchronize()
        per_op["_graph_step"] = [gev[i].elapsed_time(gev[i + 1]) * 1e3 for i in range(steps)]
        del graph
    if flush_mib == 0 and variant != "expert_gemm":
        # the headline pair with cold caches, outside the timed step: before each
        # dispatch + combine, outside its events, read 1 GiB of scratch so that neither L2
        # nor the Infinity Cache holds x or the buffer (a read leaves only clean lines)
        flush = torch.zeros((COLD_FLUSH_MIB << 20) // 4, dtype=torch.float32, device=dev)
        dsp = next(fn for op, fn in ops if op == "dispatch")
        cmb = next(fn for op, fn in ops if op == "combine")
        per_op["_cold_dispatch"], per_op["_cold_combine"] = [], []
        for i in range(COLD_WARMUP + cold_pairs):
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            flush.sum()
            a.record()
            dsp()
            b.record()
            cmb()
            c.record()
            torch.cuda.synchronize()
            if i >= COLD_WARMUP:
                per_op["_cold_dispatch"].append(a.elapsed_time(b) * 1e3)
                per_op["_cold_combine"].append(b.elapsed_time(c) * 1e3)
        del flush
    if flush_mib == 0 and variant != "expert_gemm" and isolated_runs > 0:
        # each op of the step alone, after a 1 GiB read of scratch outside its events (the
        # per-kernel form of the cold pair: no op pays for lines an earlier op left dirty)
        flush = torch.zeros((COLD_FLUSH_MIB << 20) // 4, dtype=torch.float32, device=dev)
        for op, fn in ops:
            key = "_isolated_" + op
            per_op[key] = []
            for i in range(COLD_WARMUP + isolated_runs):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                flush.sum()
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                if i >= COLD_WARMUP:
                    per_op[key].append(a.elapsed_time(b) * 1e3)
        del flush
    for op, fn in extra.get("unfused", []) + extra.get("layer", []):  # outside the timed step
        per_op[op] = []
        fn()  # the first call sets up the autograd graph and allocator
        for _ in range(min(steps, 10)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            per_op[op].append(a.elapsed_time(b) * 1e3)
    L = st["L"]
    kept = int(L.kept.sum().item())
    active = int((L.kept > 0).sum().item())
    # achievable-bandwidth reference: a plain device-to-device copy moving as many bytes
    # (read + write) as dispatch + combine, timed the same way
    ab = algorithmic_bytes(w, kept, rows)
    copy_bytes = (ab["dispatch"] + ab["combine"]) // 2
    csrc = torch.empty(copy_bytes, dtype=torch.uint8, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    per_op["_copy_reference"] = []
    for i in range(min(steps, 10) + 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        cdst.copy_(csrc)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            per_op["_copy_reference"].append(a.elapsed_time(b) * 1e3)
    del csrc, cdst
    if variant == "expert_gemm":
        # library reference: torch.matmul (hipBLASLt) on one dense bf16/f16 product with the
        # same FLOPs ([placed rows, m] x [m, n]), timed the same way
        da = torch.randn((kept, m), device=dev, dtype=torch.float32).to(tdt)
        db = torch.randn((W.EXPERT_WIDTH, m), device=dev, dtype=torch.float32).to(tdt)
        dc = torch.empty((kept, W.EXPERT_WIDTH), device=dev, dtype=tdt)
        per_op["_dense_gemm_reference"] = []
        for i in range(min(steps, 10) + 2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            torch.mm(da, db.t(), out=dc)
            b.record()
            torch.cuda.synchronize()
            if i >= 2:
                per_op["_dense_gemm_reference"].append(a.elapsed_time(b) * 1e3)
        del da, db, dc
        # the usual PyTorch ways to run the same grouped product on the dispatched buffer
        # (the dispatch itself not counted): torch.mm per expert, and torch._grouped_mm
        M.moe_dispatch(L, x, out=buf)
        kept_h, offs_h = L.kept.cpu().numpy(), L.offsets.cpu().numpy()
        H3 = torch.empty((rows, W.EXPERT_WIDTH), dtype=tdt, device=dev)
        wd = wts.detach()

        def per_expert_loop():
            for xe in range(e):
                if kept_h[xe] > 0:
                    r0, r1 = int(offs_h[xe]), int(offs_h[xe] + kept_h[xe])
                    torch.mm(buf[r0:r1], wd[xe].t(), out=H3[r0:r1])

        refs = [("_torch_mm_per_expert", per_expert_loop)]
        if hasattr(torch, "_grouped_mm") and cap <= 0 and opts["pad_multiple"] == 1:
            ends = torch.from_numpy(offs_h[1:].astype(np.int32)).to(dev)
            wT = wd.transpose(1, 2)
            refs.append(("_torch_grouped_mm", lambda: torch._grouped_mm(buf, wT, offs=ends)))
            # and the two gradients (the forward's output standing in for the incoming
            # gradient, as above): rows @ W[x], and per expert grad^T @ rows into [e, n, m]
            refs.append(("_torch_grouped_mm_input_grad", lambda: torch._grouped_mm(H, wd, offs=ends)))
            refs.append(("_torch_grouped_mm_weight_grad", lambda: torch._grouped_mm(H.t(), buf, offs=ends)))
        for op, fn in refs:
            try:
                fn()
            except RuntimeError:  # not supported by this torch build
                continue
            per_op[op] = []
            for i in range(min(steps, 10)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                per_op[op].append(a.elapsed_time(b) * 1e3)
        del H3
    flags, _ = M.moe_layout_read(L)
    if flags != 0:
        raise RuntimeError(f"layout flags {flags} on a valid workload")
    return elapsed, per_op, kept, rows, active


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def run_cpu_baseline(w: W.Workload, variant: str | None = None, step_seconds: float = 6.0,
                     sample_tokens: int = 1024, loop_tokens: int = 16):
    """The oracle, as it stands, on the host's CPU, single-threaded.

    value: the metric's scope. The vectorised oracle's dispatch + combine, given the
    layout, on the same full host arrays as the GPU, median of 3 (tokens = s); beside it
    the gate and the layout on the same arrays, each the median of 3. Parts:
    the whole step on the first `sample_tokens` tokens for about `step_seconds`; and the
    loop oracle (plain per-element Python loops) over the whole step of the tiny
    capacity-bounded workload, and its dispatch + combine on the first `loop_tokens`
    tokens of this workload and of the 4096-token dropless one. The expert_gemm variant times its forward (float64
    matmul per expert) on a 128-token sample instead.
    """
    from threadpoolctl import threadpool_limits

    import oracle
    import oracle.loop as LO

    limit = threadpool_limits(limits=1)  # the BLAS behind numpy's matmul on one core
    opts = dict(route_major=variant == "route_major", pad_multiple=128 if variant == "pad128" else 1)
    inp = W.make_inputs(w)
    out = {"unit": "tokens/s", "cores": 1, "kind": "oracle",
           "host": f"{_cpu_model()}, {os.cpu_count()} logical CPUs (one used)"}

    if variant != "expert_gemm":
        # the gate and the layout on the same full arrays, each the median of 3
        tg, tl = [], []
        for _ in range(3):
            t0 = time.perf_counter()
            idx, wt = oracle.gate_topk(inp.logits, w.k)
            t1 = time.perf_counter()
            L = oracle.dispatch_layout(idx, w.e, w.capacity, **opts)
            t2 = time.perf_counter()
            tg.append(t1 - t0)
            tl.append(t2 - t1)
        out["gate"] = {"tokens_per_s": round(w.s / float(np.median(tg)), 1),
                       "ms": round(float(np.median(tg)) * 1e3, 3)}
        out["layout"] = {"tokens_per_s": round(w.s / float(np.median(tl)), 1),
                         "ms": round(float(np.median(tl)) * 1e3, 3)}
        wc = oracle.renormalize_kept(L, wt) if variant == "renorm_kept" else wt
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            if variant == "weights_before":
                E = oracle.dispatch_weighted(L, inp.x, wc, w.dtype)
                oracle.dispatch_backward(L, E, w.dtype)  # the unweighted combine
            else:
                E = oracle.dispatch(L, inp.x)
                oracle.combine(L, E, wc, w.dtype)
            times.append(time.perf_counter() - t0)
            del E
        med = float(np.median(times))
        kept = int((L.dst >= 0).sum())
        ab = algorithmic_bytes(w, kept, L.rows, variant)
        out.update({
            "value": round(w.s / med, 1),
            "GBps": round((ab["dispatch"] + ab["combine"]) / med / 1e9, 3),
            "sample": (f"dispatch + combine of the vectorised oracle given the layout, on the full {w.name} "
                       f"arrays ({w.s} tokens), median of 3 runs ({', '.join(f'{t * 1e3:.4g}' for t in times)} ms), "
                       "single-threaded numpy"),
        })

    # the whole step on the first tokens of the same workload (time-boxed)
    n = min(sample_tokens if variant != "expert_gemm" else min(sample_tokens, 128), w.s)
    logits, x, gy = inp.logits[:n], inp.x[:n], inp.grad_y[:n]
    cap = w.capacity
    if cap > 0:  # keep the capacity factor of the workload on the sample
        cap = max(1, -(-cap * n // w.s))
    wts = expert_weights(w) if variant == "expert_gemm" else None
    reps = 0
    t0 = time.perf_counter()
    while True:
        idx, wt = oracle.gate_topk(logits, w.k)
        L = oracle.dispatch_layout(idx, w.e, cap, **opts)
        if variant == "expert_gemm":
            H, _ = oracle.expert_gemm(L, x, wts, w.dtype, gather=True)
            oracle.combine(L, H, wt, w.dtype)
        elif variant == "weights_before":
            E = oracle.dispatch_weighted(L, x, wt, w.dtype)
            oracle.dispatch_backward(L, E, w.dtype)
            oracle.dispatch_weighted(L, x, wt, w.dtype)
            gE = oracle.dispatch(L, gy)
            _, gw = oracle.dispatch_weighted_backward(L, gE, x, wt, w.dtype)
        else:
            wc = oracle.renormalize_kept(L, wt) if variant == "renorm_kept" else wt
            E = oracle.dispatch(L, x)
            oracle.combine(L, E, wc, w.dtype)
            E2, _ = oracle.dispatch_replay(L, x, idx)
            gE, gw = oracle.combine_backward(L, gy, E2, wc, w.dtype)
            if variant == "renorm_kept":
                gw = oracle.renormalize_kept_backward(L, wt, gw)
            oracle.dispatch_backward(L, gE, w.dtype)
        if variant != "expert_gemm":  # that variant times the forward only
            oracle.gate_topk_backward(idx, wt, gw, w.e)
        reps += 1
        el = time.perf_counter() - t0
        if el >= step_seconds:
            break
    step = {"tokens_per_s": round(n * reps / el, 1),
            "sample": (f"first {n} of {w.s} tokens of {w.name} (same m, e, k, dtype"
                       f"{', capacity scaled to ' + str(cap) if w.capacity > 0 else ''}), "
                       f"{'forward: gate, layout, expert GEMM, combine' if variant == 'expert_gemm' else 'whole step'}, "
                       f"{reps} passes in {el:.1f} s")}
    if variant == "expert_gemm":
        out.update({"value": step["tokens_per_s"], "sample": step["sample"] + ", single-threaded numpy"})
    else:
        out["whole_step_sample"] = step

    # the loop oracle over the whole step of the tiny workload
    tw = W.WORKLOADS["tiny_capacity_top2"]
    ti = W.make_inputs(tw)
    t0 = time.perf_counter()
    idx, wt = LO.gate_topk(ti.logits, tw.k)
    L = LO.dispatch_layout(idx, tw.e, tw.capacity)
    ta = time.perf_counter()
    E = LO.dispatch(L, ti.x)
    LO.combine(L, E, wt, tw.dtype)
    tb = time.perf_counter()
    E2 = LO.dispatch(L, ti.x)  # the replay
    gE, gw = LO.combine_backward(L, ti.grad_y, E2, wt, tw.dtype)
    LO.dispatch_backward(L, gE, tw.dtype)
    LO.gate_topk_backward(idx, wt, gw, tw.e)
    t1 = time.perf_counter()
    out["loop_oracle_tiny"] = {
        "what": f"the loop oracle (per-element Python loops) on {W.describe(tw)}",
        "whole_step_tokens_per_s": round(tw.s / (t1 - t0), 1),
        "dispatch_combine_tokens_per_s": round(tw.s / (tb - ta), 1),
        "seconds": round(t1 - t0, 3)}
    # and its dispatch + combine on the first tokens of this workload and of the 4096-token
    # dropless one (full row width; the whole arrays would take the loops hours)
    samples = {}
    for name in dict.fromkeys([w.name, "dropless_top8_h2816"]):
        samples[name] = _loop_oracle_sample(W.WORKLOADS[name], loop_tokens)
    out["loop_oracle_samples"] = samples
    limit.unregister()
    return out


def _loop_oracle_sample(w: W.Workload, n: int) -> dict:
    """The loop oracle's dispatch + combine, given its layout, on the first n tokens of w."""
    import oracle.loop as LO

    inp = W.make_inputs(w)
    n = min(n, w.s)
    cap = w.capacity
    if cap > 0:
        cap = max(1, -(-cap * n // w.s))
    idx, wt = LO.gate_topk(inp.logits[:n], w.k)
    L = LO.dispatch_layout(idx, w.e, cap)
    t0 = time.perf_counter()
    E = LO.dispatch(L, inp.x[:n])
    LO.combine(L, E, wt, w.dtype)
    el = time.perf_counter() - t0
    return {"tokens_per_s": round(n / el, 2), "seconds": round(el, 3),
            "sample": f"first {n} of {w.s} tokens (m={w.m}, e={w.e}, k={w.k}, {w.dtype}"
                      f"{', capacity scaled to ' + str(cap) if w.capacity > 0 else ''})"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=W.HEADLINE, choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="time box of the CPU oracle's whole-step sample")
    ap.add_argument("--variant", choices=VARIANTS, default=None,
                    help="time the step with one of the variants instead of the default path")
    ap.add_argument("--flush-mib", type=int, default=0, metavar="MIB",
                    help="cold caches: read MIB MiB of scratch before each timed step, outside its "
                         "events (the step time is then summed from the events, without the flushes)")
    ap.add_argument("--cold-pairs", type=int, default=None, metavar="N",
                    help=f"timed cold-cache dispatch + combine pairs (default max({COLD_PAIRS}, --steps))")
    ap.add_argument("--isolated-runs", type=int, default=ISOLATED_RUNS, metavar="N",
                    help="runs of each op alone after a flush (0: none; short profiled runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run one plain device-to-device copy of MIB MiB "
                         "(a known-size reference for hardware memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU exchange)", file=sys.stderr)
        sys.exit(2)

    w = W.WORKLOADS[args.workload]
    cold_pairs = args.cold_pairs if args.cold_pairs is not None else max(COLD_PAIRS, args.steps)
    if cold_pairs < 1:
        ap.error("--cold-pairs must be at least 1")
    elapsed, per_op, kept, rows, active = run_gpu(w, args.steps, args.warmup, args.variant, args.flush_mib,
                                                  cold_pairs, args.isolated_runs)
    if args.calibrate_copy > 0:
        import torch
        src = torch.ones(args.calibrate_copy << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_per_step = elapsed / args.steps * 1e3
    abytes = algorithmic_bytes(w, kept, rows, args.variant, active)
    copy_us = per_op.pop("_copy_reference")
    layer_us = per_op.pop("layer_train_step", None)
    graph_us = per_op.pop("_graph_step", None)
    plain_us = per_op.pop("_plain_step", None)
    cold_d, cold_c = per_op.pop("_cold_dispatch", None), per_op.pop("_cold_combine", None)
    cold_d = None if not cold_d else cold_d
    dense_us = per_op.pop("_dense_gemm_reference", None)
    grouped_refs = {name[1:]: per_op.pop(name) for name in ("_torch_mm_per_expert", "_torch_grouped_mm",
                                                            "_torch_grouped_mm_input_grad",
                                                            "_torch_grouped_mm_weight_grad")
                    if name in per_op}
    isolated = {name[len("_isolated_"):]: per_op.pop(name) for name in list(per_op) if name.startswith("_isolated_")}
    ops = list(per_op)
    kernels = {}
    for op in ops:
        us = float(np.mean(per_op[op]))
        kernels[op] = {"us": round(us, 2), "us_median": round(float(np.median(per_op[op])), 2),
                       "us_p10": round(float(np.percentile(per_op[op], 10)), 2),
                       "us_p90": round(float(np.percentile(per_op[op], 90)), 2),
                       "us_min": round(float(np.min(per_op[op])), 2),
                       "bytes": abytes[op], "GBps": round(abytes[op] / us / 1e3, 1)}
    step_ops = [op for op in ops if op not in ("expert_gemm_unfused", "expert_gemm_wgrad", "expert_gemm_wgrad_narrow",
                                               "expert_gemm_dgrad") and
                not (args.variant == "expert_gemm" and op == "dispatch")]
    dc_us = kernels["dispatch"]["us"] + kernels["combine"]["us"]
    dc_bytes = abytes["dispatch"] + abytes["combine"]
    dc_gbps = dc_bytes / dc_us / 1e3
    dc_steps = np.array(per_op["dispatch"]) + np.array(per_op["combine"]) if args.variant != "expert_gemm" \
        else np.array([dc_us])
    ab0 = algorithmic_bytes(w, kept, rows)  # the copy reference's size (default path bytes)
    copy_moved = 2 * ((ab0["dispatch"] + ab0["combine"]) // 2)
    copy_gbps = copy_moved / float(np.mean(copy_us)) / 1e3
    dominant = max(step_ops, key=lambda op: kernels[op]["us"])
    dom_gbps = abytes[dominant] / kernels[dominant]["us"] / 1e3
    roofline = {"kernel": dominant, "bound": "hbm", "achieved": round(dom_gbps, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(w.name, args.variant).get(dominant),
                "algorithmic_bytes": abytes[dominant]}
    kernels_isolated = {}
    for op, us_list in isolated.items():
        med = float(np.median(us_list))
        kernels_isolated[op] = {"us_median": round(med, 2), "us_p10": round(float(np.percentile(us_list, 10)), 2),
                                "us_p90": round(float(np.percentile(us_list, 90)), 2),
                                "GBps": round(abytes[op] / med / 1e3, 1),
                                "frac_of_hbm_peak": round(abytes[op] / med / 1e3 / HBM_PEAK_GBPS, 4)}
    if dominant in kernels_isolated:
        roofline["isolated"] = {
            "what": f"the same kernel alone, each of {args.isolated_runs} runs after a {COLD_FLUSH_MIB} MiB read of "
                    "scratch (median); in the step it also pays for evicting lines earlier kernels left dirty",
            "achieved": kernels_isolated[dominant]["GBps"], "frac": kernels_isolated[dominant]["frac_of_hbm_peak"],
            "us_median": kernels_isolated[dominant]["us_median"]}
    if args.variant == "expert_gemm":
        flops = 2 * kept * W.EXPERT_WIDTH * w.m
        for op in ("expert_gemm", "expert_gemm_unfused", "expert_gemm_wgrad", "expert_gemm_wgrad_narrow",
                   "expert_gemm_dgrad"):
            kernels[op]["TFLOPs"] = round(flops / kernels[op]["us"] / 1e6, 1)
        if dominant == "expert_gemm":
            tf = flops / kernels[dominant]["us"] / 1e6
            roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(tf, 1),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic(w.name, args.variant).get(dominant),
                        "algorithmic_flops": flops, "algorithmic_bytes": abytes[dominant]}

    cold = None if cold_d is None else cold_pair_summary(w.s, cold_d, cold_c, abytes["dispatch"] + abytes["combine"])
    step_tps = w.s / (ms_per_step / 1e3)
    warm_pair = None if args.variant == "expert_gemm" else {
        "what": "dispatch + combine inside the back-to-back timed steps (caches warm from the previous step)",
        "tokens_per_s": round(w.s / (dc_us / 1e6), 1), "GBps": round(dc_gbps, 1),
        "frac_of_hbm_peak": round(dc_gbps / HBM_PEAK_GBPS, 4), "us_mean": round(dc_us, 2),
        "us_median": round(float(np.median(dc_steps)), 2),
        "us_p10": round(float(np.percentile(dc_steps, 10)), 2),
        "us_p90": round(float(np.percentile(dc_steps, 90)), 2),
        "us_min": round(float(np.min(dc_steps)), 2),
        "bytes": dc_bytes, "frac_of_copy": round(dc_gbps / copy_gbps, 4)}
    if cold is not None:
        cold["frac_of_copy"] = round(cold["GBps"] / copy_gbps, 4)
        cold["warm"] = warm_pair
    line = {
        "metric": METRIC,
        # the headline metric: dispatch + combine tokens/s, median of the cold-cache pairs
        # (the expert_gemm variant has no such pair: there it is the step's rate)
        "value": cold["tokens_per_s"] if cold is not None else round(step_tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "s": w.s, "m": w.m, "e": w.e, "k": w.k,
                   "capacity": w.capacity if w.capacity > 0 else "dropless",
                   "routing": {"uniform": "N(0,1) logits", "zipf": "N(0,1) + 2 ln Zipf(1.2) bias",
                               "hotspot": "N(0,1), +3 on expert 0 for 10% of tokens"}[w.routing],
                   "step": "+".join(step_ops), "variant": args.variant or "default",
                   "parallelism": "single GPU",
                   **({"flush_mib_before_each_step": args.flush_mib} if args.flush_mib > 0 else {}),
                   **({"expert_width": W.EXPERT_WIDTH} if args.variant == "expert_gemm" else {})},
        "value_is": ("dispatch + combine tokens/s: median of the cold-cache pairs in dispatch_combine"
                     if cold is not None else "tokens/s of the whole step (gate, layout, fused expert GEMM, combine)"),
        "step_tokens_per_s": round(step_tps, 1),
        "dispatch_combine": cold if cold is not None else warm_pair,
        "copy_reference": {"what": "device-to-device copy of the dispatch+combine byte count (read + write)",
                           "bytes": copy_moved, "us": round(float(np.mean(copy_us)), 2),
                           "GBps": round(copy_gbps, 1), "frac_of_hbm_peak": round(copy_gbps / HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "dense_gemm_reference": None if dense_us is None else {
            "what": "torch.mm (hipBLASLt) on one dense [placed rows, m] x [m, n] product of the same "
                    "FLOPs and dtype, no grouping or gather",
            "us": round(float(np.mean(dense_us)), 2),
            "TFLOPs": round(2 * kept * W.EXPERT_WIDTH * w.m / float(np.mean(dense_us)) / 1e6, 1)},
        "grouped_gemm_references": None if not grouped_refs else {
            "what": "the same grouped products in PyTorch on the dispatched buffer (dispatch not counted); "
                    "the gradients' references in the element type",
            **{name: {"us": round(float(np.mean(v)), 2),
                      "TFLOPs": round(2 * kept * W.EXPERT_WIDTH * w.m / float(np.mean(v)) / 1e6, 1)}
               for name, v in grouped_refs.items()}},
        "plain_step": None if plain_us is None else {
            "what": "the same eager step, each kernel launched from Python as in the timed steps, but with one "
                    "event pair around all the steps instead of events around each op",
            "us": round(plain_us[0], 2), "tokens_per_s": round(w.s / (plain_us[0] / 1e6), 1)},
        "graph_step": None if graph_us is None else {
            "what": "the same step captured once in a HIP graph and replayed (HIP events per replay)",
            "us": round(float(np.mean(graph_us)), 2), "us_median": round(float(np.median(graph_us)), 2),
            "tokens_per_s": round(w.s / (float(np.mean(graph_us)) / 1e6), 1),
            "speedup_vs_eager": round(ms_per_step * 1e3 / float(np.mean(graph_us)), 3)},
        "layer_train_step": None if layer_us is None else {
            "what": "autograd forward + backward of the layer: gate, layout, fused expert GEMM, weighted "
                    "combine; gradients of tokens, expert weights (element type) and router logits",
            "us": round(float(np.mean(layer_us)), 2), "us_median": round(float(np.median(layer_us)), 2),
            "tokens_per_s": round(w.s / (float(np.mean(layer_us)) / 1e6), 1),
            "gemm_TFLOPs": round(3 * 2 * kept * W.EXPERT_WIDTH * w.m / float(np.mean(layer_us)) / 1e6, 1)},
        "kernels": kernels,
        "kernels_isolated": kernels_isolated or None,
        "kept_routes": kept,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = run_cpu_baseline(w, args.variant, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
