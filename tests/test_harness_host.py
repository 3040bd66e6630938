"""Host checks of the GPU tests' own machinery (no GPU): the chunked full-size sweep.

The full-size parity tests compare every token a chunk at a time, running the oracle
on a compact copy of just the rows a chunk's routes point at. That is only a valid
stand-in if the chunked oracle reproduces the oracle run on the whole batch, bit for
bit, which these tests check on batches with capacity drops, padding and skew.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import compact_layout, tagged_rows, token_chunks


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("cap,pad,skew", [(0, 1, False), (40, 1, False), (0, 8, True), (7, 1, True)])
def test_chunked_oracle_equals_full_oracle(dt, cap, pad, skew):
    rng = np.random.default_rng(cap * 31 + pad + skew)
    s, e, k, m = 3000, 64, 4, 16
    idx = W.skewed_idx(rng, s, e, k) if skew else W.random_idx(rng, s, e, k)
    x = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dt)
    gy = W.cast_input(rng.standard_normal((s, m)).astype(np.float32), dt)
    w = W.random_weights(rng, s, k)
    L = oracle.dispatch_layout(idx, e, cap, pad_multiple=pad)
    expert_of_row = np.repeat(np.arange(e), np.diff(L.offsets))
    expert_of_row = np.concatenate([expert_of_row, np.zeros(L.rows - len(expert_of_row), np.int64)])
    E = tagged_rows(x, L.src, expert_of_row, dt)
    y = oracle.combine(L, E, w, dt)
    gE, gw = oracle.combine_backward(L, gy, E, w, dt)
    gx = oracle.dispatch_backward(L, gE, dt)

    seen = np.zeros(s, bool)
    rows_seen = np.zeros(L.rows, bool)
    for toks in token_chunks(s, 700):
        S, used = compact_layout(L, toks)
        assert np.all(S.src >= 0)
        E_c = tagged_rows(x, S.src, expert_of_row[used], dt)
        assert np.array_equal(E_c.view(np.uint8), E[used].view(np.uint8))
        assert np.array_equal(oracle.combine(S, E_c, w[toks], dt).view(np.uint8), y[toks].view(np.uint8))
        gE_c, gw_c = oracle.combine_backward(S, gy[toks], E_c, w[toks], dt)
        assert np.array_equal(gE_c.view(np.uint8), gE[used].view(np.uint8))
        assert np.array_equal(gw_c, gw[toks])
        assert np.array_equal(oracle.dispatch_backward(S, gE_c, dt).view(np.uint8), gx[toks].view(np.uint8))
        seen[toks] = True
        rows_seen[used] = True
    assert seen.all()
    # every placed row belongs to exactly one chunk; the rest are the unfilled rows
    assert np.array_equal(rows_seen, L.src >= 0)


def test_token_chunks_cover_once():
    got = np.concatenate(list(token_chunks(2049, 1024)))
    assert np.array_equal(got, np.arange(2049))
    assert list(token_chunks(0, 1024)) == []
