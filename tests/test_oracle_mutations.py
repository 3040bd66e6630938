"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each mutation is a plausible slip: a wrong slot order, an off-by-one, a dropped
term, an unapplied weight, a flipped sign, a wrong tie-break, a wrong operand.
For each one we swap the mutated function into the `oracle` package and run
the pin tests; at least one of them has to fail.
"""
import numpy as np
import pytest

import oracle
from oracle import moe
from tests import test_oracle_pins as pins
from tests import test_oracle_variants as vpins
from tests import test_oracle_gemm as gpins


def _route_major_layout(idx, e, capacity, route_major=False, pad_multiple=1):
    # slots handed out to every token's first route, then every second route, ...
    L = moe.dispatch_layout(idx, e, capacity, route_major, pad_multiple)
    s, k = idx.shape
    seen = np.zeros(e, np.int64)
    dst = -np.ones((s, k), np.int64)
    src = -np.ones(L.rows, np.int64)
    for j in range(k):
        for t in range(s):
            x = int(idx[t, j])
            q = seen[x]
            seen[x] += 1
            if capacity > 0 and q >= capacity:
                continue
            dst[t, j] = L.offsets[x] + q
            src[dst[t, j]] = t
    L.dst = dst.astype(np.int32)
    L.src = src.astype(np.int32)
    return L


def _slot_off_by_one(idx, e, capacity, route_major=False, pad_multiple=1):
    L = moe.dispatch_layout(idx, e, capacity, route_major, pad_multiple)
    dst = L.dst.copy()
    dst[dst >= 0] += 1
    dst[dst >= L.rows] = -1
    L.dst = dst
    return L


def _combine_drops_last_route(layout, E, w, dtype):
    w = np.array(w, np.float32).copy()
    w[:, -1] = 0
    return moe.combine(layout, E, w, dtype)


def _combine_ignores_weights(layout, E, w, dtype):
    return moe.combine(layout, E, np.ones_like(np.asarray(w, np.float32)), dtype)


def _gate_bwd_sign(idx, w, gw, e):
    return -moe.gate_topk_backward(idx, w, gw, e)


def _gate_bwd_no_centering(idx, w, gw, e):
    return moe.gate_topk_backward(idx, w, gw, e) + _selected_scatter(idx, w, gw, e)


def _selected_scatter(idx, w, gw, e):
    # adds back w*dot, i.e. forgets to subtract the weighted mean
    s, k = idx.shape
    out = np.zeros((s, e), np.float32)
    dot = (w.astype(np.float64) * gw).sum(1)
    for j in range(k):
        out[np.arange(s), idx[:, j]] += (w[:, j] * dot).astype(np.float32)
    return out


def _gate_ties_high(logits, k):
    l32 = np.asarray(logits, np.float32)
    rev = l32[:, ::-1]
    idx, w = moe.gate_topk(rev, k)
    return (l32.shape[1] - 1 - idx).astype(np.int32), w


def _combine_bwd_wrong_row(layout, gy, E, w, dtype):
    gE, gw = moe.combine_backward(layout, gy, E, w, dtype)
    return gE, np.roll(gw, 1, axis=1)


def _combine_bwd_unweighted(layout, gy, E, w, dtype):
    return moe.combine_backward(layout, gy, E, np.ones_like(np.asarray(w, np.float32)), dtype)


def _dispatch_bwd_first_route(layout, G, dtype):
    L2 = moe.Layout(**{**layout.__dict__})
    L2.dst = layout.dst.copy()
    L2.dst[:, 1:] = -1
    return moe.dispatch_backward(L2, G, dtype)


def _bf16_truncates(a32, dtype):
    if dtype != "bf16":
        return moe.from_f32(a32, dtype)
    u = np.ascontiguousarray(a32, np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _layout_ignores_route_major(idx, e, capacity, route_major=False, pad_multiple=1):
    return moe.dispatch_layout(idx, e, capacity, False, pad_multiple)


def _layout_ignores_padding(idx, e, capacity, route_major=False, pad_multiple=1):
    L = moe.dispatch_layout(idx, e, capacity, route_major, 1)
    if pad_multiple > 1:
        L.rows = L.rows + e * (pad_multiple - 1)
        L.src = np.concatenate([L.src, -np.ones(e * (pad_multiple - 1), np.int32)])
    return L


def _weighted_dispatch_unweighted(layout, x, w, dtype):
    return moe.dispatch_weighted(layout, x, np.ones_like(np.asarray(w, np.float32)), dtype)


def _renorm_over_all_routes(layout, w):
    w64 = np.asarray(w, np.float32).astype(np.float64)
    return (w64 / w64.sum(axis=1, keepdims=True)).astype(np.float32) * (layout.dst >= 0)


def _renorm_backward_no_centering(layout, w, g):
    w64 = np.asarray(w, np.float32).astype(np.float64)
    kept = layout.dst >= 0
    S = np.where(kept, w64, 0.0).sum(axis=1, keepdims=True)
    return np.where(kept & (S != 0), np.asarray(g, np.float64) / np.where(S != 0, S, 1), 0).astype(np.float32)


def _gemm_wrong_expert(layout, a, weights, dtype, gather, route_w=None):
    return moe.expert_gemm(layout, a, np.roll(weights, 1, axis=0), dtype, gather, route_w)


def _gemm_untransposed(layout, a, weights, dtype, gather, route_w=None):
    e, n, m = weights.shape
    if n == m:
        return moe.expert_gemm(layout, a, np.swapaxes(weights, 1, 2), dtype, gather, route_w)
    out, exact = moe.expert_gemm(layout, a, weights, dtype, gather, route_w)
    return out, exact * 1.5


def _gemm_ignores_route_weights(layout, a, weights, dtype, gather, route_w=None):
    return moe.expert_gemm(layout, a, weights, dtype, gather, None)


def _wgrad_ignores_gather(layout, a, grad_out, dtype, gather, out_dtype="f32"):
    if gather:  # reads the token rows as if they were already dispatched
        pad = np.zeros((max(layout.rows - a.shape[0], 0),) + a.shape[1:], a.dtype)
        return moe.expert_gemm_wgrad(layout, np.concatenate([a, pad])[:layout.rows], grad_out, dtype, False,
                                     out_dtype)
    return moe.expert_gemm_wgrad(layout, a, grad_out, dtype, gather, out_dtype)


def _wgrad_wrong_expert(layout, a, grad_out, dtype, gather, out_dtype="f32"):
    out, exact = moe.expert_gemm_wgrad(layout, a, grad_out, dtype, gather, out_dtype)
    return np.roll(out, 1, axis=0), np.roll(exact, 1, axis=0)


def _wgrad_transposed(layout, a, grad_out, dtype, gather, out_dtype="f32"):
    out, exact = moe.expert_gemm_wgrad(layout, a, grad_out, dtype, gather, out_dtype)
    return np.swapaxes(out, 1, 2).copy(), np.swapaxes(exact, 1, 2).copy()


def _wgrad_narrows_by_truncation(layout, a, grad_out, dtype, gather, out_dtype="f32"):
    out, exact = moe.expert_gemm_wgrad(layout, a, grad_out, dtype, gather, "f32")
    if out_dtype == "bf16":
        return (out.view(np.uint32) >> np.uint32(16)).astype(np.uint16), exact
    if out_dtype == "f16":  # round toward zero: step down where nearest rounded away
        h = out.astype(np.float16)
        away = np.abs(h.astype(np.float32)) > np.abs(out)
        h[away] = np.nextafter(h[away], np.float16(0))
        return h, exact
    return out, exact


def _dgrad_untransposed(layout, grad_out, weights, dtype):
    e, n, m = weights.shape
    if n == m:
        return moe.expert_gemm_dgrad(layout, grad_out, np.swapaxes(weights, 1, 2), dtype)
    out, exact = moe.expert_gemm_dgrad(layout, grad_out, weights, dtype)
    return out, exact * 1.5


def _dgrad_wrong_expert(layout, grad_out, weights, dtype):
    return moe.expert_gemm_dgrad(layout, grad_out, np.roll(weights, 1, axis=0), dtype)


MUTATIONS = {
    "dgrad_untransposed": ("expert_gemm_dgrad", _dgrad_untransposed),
    "dgrad_wrong_expert": ("expert_gemm_dgrad", _dgrad_wrong_expert),
    "wgrad_ignores_gather": ("expert_gemm_wgrad", _wgrad_ignores_gather),
    "wgrad_wrong_expert": ("expert_gemm_wgrad", _wgrad_wrong_expert),
    "wgrad_transposed": ("expert_gemm_wgrad", _wgrad_transposed),
    "wgrad_narrows_by_truncation": ("expert_gemm_wgrad", _wgrad_narrows_by_truncation),
    "gemm_wrong_expert": ("expert_gemm", _gemm_wrong_expert),
    "gemm_untransposed": ("expert_gemm", _gemm_untransposed),
    "gemm_ignores_route_weights": ("expert_gemm", _gemm_ignores_route_weights),
    "ignores_route_major": ("dispatch_layout", _layout_ignores_route_major),
    "ignores_padding": ("dispatch_layout", _layout_ignores_padding),
    "weighted_dispatch_unweighted": ("dispatch_weighted", _weighted_dispatch_unweighted),
    "renorm_over_all_routes": ("renormalize_kept", _renorm_over_all_routes),
    "renorm_backward_no_centering": ("renormalize_kept_backward", _renorm_backward_no_centering),
    "route_major_slots": ("dispatch_layout", _route_major_layout),
    "slot_off_by_one": ("dispatch_layout", _slot_off_by_one),
    "combine_drops_last_route": ("combine", _combine_drops_last_route),
    "combine_ignores_weights": ("combine", _combine_ignores_weights),
    "gate_bwd_sign": ("gate_topk_backward", _gate_bwd_sign),
    "gate_bwd_no_centering": ("gate_topk_backward", _gate_bwd_no_centering),
    "gate_ties_high": ("gate_topk", _gate_ties_high),
    "combine_bwd_wrong_row": ("combine_backward", _combine_bwd_wrong_row),
    "combine_bwd_unweighted": ("combine_backward", _combine_bwd_unweighted),
    "dispatch_bwd_first_route": ("dispatch_backward", _dispatch_bwd_first_route),
    "bf16_truncates": ("from_f32", _bf16_truncates),
}

PINS = [
    pins.test_golden_layout,
    pins.test_golden_combine_and_backward,
    pins.test_golden_gate,
    lambda: pins.test_gate_indices_brute_force_with_ties(0),
    lambda: pins.test_gate_backward_finite_differences(),
    lambda: pins.test_index_path_matches_dense_einsum(3, 6),
    lambda: pins.test_unit_weight_round_trip_is_exact("bf16", 3),
    lambda: pins.test_adjoint_identities(2),
    pins.test_weight_gradient_matches_finite_difference_of_dense_combine,
    pins.test_identity_expert_closed_forms,
    pins.test_bf16_rounding_brute_force,
    lambda: vpins.test_layout_options_match_brute_force(),
    vpins.test_route_major_gives_first_choices_priority,
    lambda: vpins.test_weighted_dispatch_matches_dense_einsum(5),
    lambda: vpins.test_weighted_dispatch_backward_adjoint_and_finite_difference(4),
    vpins.test_renormalized_gate_weights_are_softmax_over_kept_logits,
    vpins.test_renormalize_backward_matches_finite_differences_through_the_gate,
    lambda: gpins.test_expert_gemm_matches_brute_force(3, True),
    gpins.test_scaled_identity_weights_route_rows_to_the_right_expert,
    gpins.test_route_weights_scale_each_row,
    lambda: gpins.test_expert_gemm_wgrad_matches_brute_force(0, True),
    gpins.test_expert_gemm_wgrad_is_the_adjoint_of_the_forward,
    gpins.test_expert_gemm_wgrad_is_the_exact_derivative_on_integers,
    lambda: gpins.test_expert_gemm_wgrad_narrowed_output_rounds_to_nearest_even("bf16"),
    lambda: gpins.test_expert_gemm_wgrad_narrowed_output_rounds_to_nearest_even("f16"),
    lambda: gpins.test_expert_gemm_dgrad_matches_brute_force(4),
    gpins.test_expert_gemm_dgrad_is_the_adjoint_of_the_forward,
    gpins.test_expert_gemm_input_gradient_is_the_exact_derivative_on_integers,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin)
        except (IndexError, ValueError):
            caught.append(pin)
    assert caught, f"no pin caught the planted mistake {name!r}"


def test_unmutated_oracle_passes_every_pin():
    for pin in PINS:
        pin()


def test_tagged_rows_expose_a_route_swap_that_identity_rows_hide():
    """The full-size GPU tests feed combine expert rows tagged by a power of two per
    expert: with the identity expert (every route of a token reads an equal row) a kernel
    that read one route's row in place of another's would pass; with tagged rows it
    cannot. Planted on the oracle: two routes of one token swapped."""
    import dataclasses

    import workloads as W
    from tests.gpu_util import tagged_rows

    rng = np.random.default_rng(5)
    s, m, e, k = 40, 16, 8, 4
    idx = W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), "bf16")
    w = W.random_weights(rng, s, k)
    L = oracle.dispatch_layout(idx, e, 0)
    swapped = dataclasses.replace(L, dst=L.dst.copy())
    swapped.dst[7, [0, 1]] = swapped.dst[7, [1, 0]]
    ident = oracle.dispatch(L, x)
    assert np.array_equal(oracle.combine(L, ident, w, "bf16"), oracle.combine(swapped, ident, w, "bf16"))
    expert_of_row = np.repeat(np.arange(e), np.diff(L.offsets))
    tagged = tagged_rows(x, L.src.astype(np.int64), expert_of_row, "bf16")
    assert not np.array_equal(oracle.combine(L, tagged, w, "bf16"), oracle.combine(swapped, tagged, w, "bf16"))
