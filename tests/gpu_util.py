"""Helpers for the GPU parity tests: host <-> device conversion and tolerances."""
import numpy as np
import torch

import oracle

DEV = "cuda"
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """Upload a host array; bf16 arrays are uint16 bit patterns."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Download a device tensor; bf16 comes back as uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    """Raw bit patterns, so +0/-0 and NaN payloads compare exactly."""
    a = np.ascontiguousarray(a)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    gb, wb = bits(got), bits(want)
    if not np.array_equal(gb, wb):
        bad = np.argwhere(gb != wb)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements differ, first at {i}: got {got[i]!r}, want {want[i]!r}")


def f32_ulps(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Distance in float32 units in the last place (monotone integer image)."""
    def key(a):
        u = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
        return np.where(u < 0, -(u & 0x7FFFFFFF), u)
    return np.abs(key(got) - key(want))


def compact_layout(L: oracle.Layout, tokens: np.ndarray) -> tuple[oracle.Layout, np.ndarray]:
    """The oracle layout restricted to some tokens, the buffer rows their routes point at
    renumbered 0..n-1 (combine and its backward are per token, so a chunk of tokens can be
    checked against a compact copy of just its rows).

    Returns (layout, used): `used` holds the original row of each compact row, ascending;
    layout.src is the token of each compact row."""
    dst = L.dst[tokens]
    placed = dst >= 0
    used = np.unique(dst[placed]).astype(np.int64)
    cdst = np.full(dst.shape, -1, dtype=np.int32)
    cdst[placed] = np.searchsorted(used, dst[placed]).astype(np.int32)
    sub = oracle.Layout(s=len(tokens), e=L.e, k=L.k, capacity=L.capacity, rows=len(used),
                        idx=L.idx[tokens], counts=L.counts, kept=L.kept, offsets=L.offsets,
                        dst=cdst, src=L.src[used], flags=L.flags, checksum=L.checksum)
    return sub, used


def token_chunks(s: int, chunk: int):
    """Consecutive token ranges covering all s tokens."""
    for t0 in range(0, s, chunk):
        yield np.arange(t0, min(s, t0 + chunk), dtype=np.int64)


def weight_grad_bound(gy32: np.ndarray, E32: np.ndarray, dst: np.ndarray) -> np.ndarray:
    """sum_m |grad_y[t,m] * E[dst[t,j],m]| per route (float64), the scale of grad_w's error."""
    s, k = dst.shape
    out = np.zeros((s, k))
    for j in range(k):
        sel = dst[:, j] >= 0
        out[sel, j] = np.abs(gy32[sel].astype(np.float64) * E32[dst[sel, j]].astype(np.float64)).sum(1)
    return out


def tagged_rows(x: np.ndarray, src: np.ndarray, expert_of_row: np.ndarray, dt: str) -> np.ndarray:
    """Expert rows E[r] = 2^q * x[src[r]], q = expert(r) mod Q (zero rows where src < 0).

    With the identity expert every route of a token reads an equal row, so reading one
    route's row in place of another's goes unseen; scaling by a power of two per expert
    makes the rows differ while staying exact (Q = 8 for f16, whose range is narrow;
    32 otherwise)."""
    Q = 8 if dt == "f16" else 32
    used = src >= 0
    scale = np.where(used, np.ldexp(1.0, (expert_of_row % Q).astype(np.int64)), 0.0).astype(np.float32)
    if dt == "bf16":
        f = (x[np.maximum(src, 0)].astype(np.uint32) << np.uint32(16)).view(np.float32) * scale[:, None]
        tagged = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    else:
        tagged = x[np.maximum(src, 0)] * scale[:, None].astype(x.dtype)
    return np.where(used[:, None], tagged, np.zeros((), x.dtype)).astype(x.dtype)  # +0.0 rows
