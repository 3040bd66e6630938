"""CPU oracle for the MoE gate / dispatch / combine path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct CPU
reference that the GPU library is checked against. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it. The product path
(the HIP library and its Python binding) never imports, calls or links anything
here, and this package imports nothing from the product path: the two share no
code. The only thing both consume is the seeded input generator in `workloads`.

Sources (web pages; cited by title and section):

  [DS-8195]  DeepSpeed pull request "MoE dispatch: fix silent Tutel + TP corruption,
             speed up native and Tutel paths" -- parts 1 (route extraction as a
             gather of per-route index/location/gate), 2 (the [e, c, m] buffer),
             3 (index dispatch/combine replacing the dense one-hot einsum, with
             fp32 accumulation in combine), its Testing section, and the review
             comment on fast_cumsum_sub_one (locations = cumsum(mask) - 1).
  [DS-8213]  DeepSpeed pull request "Add an opt-in DeepEP transport for the AutoEP
             expert all-to-all" -- the first commit message (tokens replicated
             before top-k expansion, arrivals grouped by expert, weighted sum
             reduced in combine, backward = combine <-> dispatch on the forward
             handle), the review-fix commit (weights must carry a gradient to the
             router), and the review threads on combine weights and trimming rows
             by the prefix sum.
  [AM-3684]  NeMo Automodel pull request "perf(moe): reuse the DeepEP dispatch
             layout on activation-checkpoint recompute" -- section "1. Reuse the
             DeepEP dispatch layout on recompute" and its "How" part (a saved
             handle replays the layout; replay must reproduce row counts).

Readings where the pages are silent are listed in the module docstrings of
`oracle.moe`. Parity status of every function is stated there as well.
"""
from .moe import (  # noqa: F401
    Layout,
    combine,
    combine_backward,
    dispatch,
    dispatch_backward,
    dispatch_layout,
    dispatch_replay,
    dispatch_weighted,
    dispatch_weighted_backward,
    expert_gemm,
    expert_gemm_dgrad,
    expert_gemm_wgrad,
    renormalize_kept,
    renormalize_kept_backward,
    gate_topk,
    gate_topk_backward,
    gate_weights_f64,
    routing_checksum,
    to_f32,
    from_f32,
    FLAG_EXPERT_OUT_OF_RANGE,
    FLAG_DUPLICATE_EXPERT,
    FLAG_REPLAY_MISMATCH,
)
