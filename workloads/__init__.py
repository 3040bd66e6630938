"""Seeded synthetic inputs for the MoE gate / dispatch / combine path.

This module only draws random numbers and stores them in the element types the
path consumes. It computes nothing of the method itself (no softmax, no top-k,
no slot assignment, no gather), so it can feed both the GPU library and the CPU
oracle without either depending on the other.

Five workloads are defined, named by what they are:

  tiny_capacity_top2       s=256,   m=64,   f32,  e=8,   k=2, capacity 80
  dropless_top8_h2816      s=4096,  m=2816, bf16, e=128, k=8, dropless
  zipf_skew_h4096          s=8192,  m=4096, bf16, e=128, k=8, dropless, Zipf(1.2) expert bias
  gshard_capacity_drop     s=16384, m=1024, f16,  e=64,  k=4, capacity 1024, hotspot on expert 0
  checkpoint_replay_h2816  s=32768, m=2816, bf16, e=128, k=8, dropless

The pages measure on routing replayed from real SFT runs (DiffusionGemma-26B-A4B,
Qwen3-235B-A22B, an AutoEP SFT job); none of that data exists here, so uniform
N(0,1) logits, a Zipf-skewed bias and an expert-0 hotspot stand in for it.

Element types: "f32" arrays are numpy float32; "f16" arrays are numpy float16;
"bf16" arrays are numpy uint16 holding bfloat16 bit patterns (numpy has no
bfloat16 type). Low-precision values are drawn as float32 and converted with
round-to-nearest-even, so every consumer sees the same bytes.
"""
from __future__ import annotations

import dataclasses

import numpy as np

DTYPES = ("f32", "bf16", "f16")
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


def capacity_from_factor(factor_num: int, factor_den: int, s: int, k: int, e: int) -> int:
    """ceil(factor * s * k / e) in exact integer arithmetic (factor = num/den)."""
    num = factor_num * s * k
    den = factor_den * e
    return -(-num // den)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    s: int
    m: int
    dtype: str
    e: int
    k: int
    capacity: int  # <= 0 means dropless
    routing: str  # "uniform" | "zipf" | "hotspot"
    seed: int
    description: str

    @property
    def dropless(self) -> bool:
        return self.capacity <= 0

    @property
    def rows(self) -> int:
        return self.s * self.k if self.dropless else self.e * self.capacity


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_capacity_top2", 256, 64, "f32", 8, 2,
                 capacity_from_factor(5, 4, 256, 2, 8), "uniform", 1001,
                 "tiny capacity-bounded top-2 routing, capacity ceil(1.25*s*k/e)=80"),
        Workload("dropless_top8_h2816", 4096, 2816, "bf16", 128, 8, 0, "uniform", 1002,
                 "dropless top-8 routing shaped like a 26B-A4B MoE layer"),
        Workload("zipf_skew_h4096", 8192, 4096, "bf16", 128, 8, 0, "zipf", 1003,
                 "Zipf(1.2)-skewed dropless top-8 routing at hidden 4096"),
        Workload("gshard_capacity_drop", 16384, 1024, "f16", 64, 4,
                 capacity_from_factor(1, 1, 16384, 4, 64), "hotspot", 1004,
                 "capacity factor 1.0 (c=1024) with 10% of tokens boosted +3 on expert 0"),
        Workload("checkpoint_replay_h2816", 32768, 2816, "bf16", 128, 8, 0, "uniform", 1005,
                 "dropless top-8 training step with checkpoint replay"),
    )
}

# The workload the headline throughput is quoted on.
HEADLINE = "zipf_skew_h4096"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (inputs only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r = r.copy()
        r[nan] = np.uint16(0x7FC0)
    return r


def cast_input(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 draws in the element type of a workload."""
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(a32.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(f"unknown dtype {dtype!r}")


def zipf_bias(e: int, exponent: float, rng: np.random.Generator) -> np.ndarray:
    """Per-expert logit bias 2*ln(p) with p Zipf(exponent) over a seeded expert order.

    Rank r = 1..e gets p_r proportional to r**-exponent; expert perm[r-1] takes rank r.
    """
    perm = rng.permutation(e)
    ranks = np.arange(1, e + 1, dtype=np.float64)
    p = ranks ** (-exponent)
    p /= p.sum()
    bias = np.empty(e, dtype=np.float64)
    bias[perm] = 2.0 * np.log(p)
    return bias


def routing_logits(rng: np.random.Generator, s: int, e: int, routing: str) -> np.ndarray:
    logits = rng.standard_normal((s, e), dtype=np.float32)
    if routing == "uniform":
        return logits
    if routing == "zipf":
        bias = zipf_bias(e, 1.2, rng)
        return (logits.astype(np.float64) + bias[None, :]).astype(np.float32)
    if routing == "hotspot":
        n_hot = int(round(0.1 * s))
        hot = rng.choice(s, size=n_hot, replace=False)
        logits[hot, 0] += np.float32(3.0)
        return logits
    raise ValueError(f"unknown routing {routing!r}")


@dataclasses.dataclass
class Inputs:
    workload: Workload
    logits: np.ndarray  # [s, e] float32
    x: np.ndarray  # [s, m] in workload dtype
    grad_y: np.ndarray  # [s, m] in workload dtype


def make_inputs(w: Workload | str, seed: int | None = None) -> Inputs:
    """Draw (logits, x, grad_y) for a workload, in that order, from PCG64(seed)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    logits = routing_logits(rng, w.s, w.e, w.routing)
    x = cast_input(rng.standard_normal((w.s, w.m), dtype=np.float32), w.dtype)
    gy = cast_input(rng.standard_normal((w.s, w.m), dtype=np.float32), w.dtype)
    return Inputs(w, logits, x, gy)


def random_case(seed: int, s: int, m: int, e: int, k: int, capacity: int, dtype: str,
                routing: str = "uniform") -> Inputs:
    """A small ad-hoc case with the same draw order as the named workloads."""
    w = Workload(f"case_s{s}_m{m}_e{e}_k{k}_c{capacity}_{dtype}", s, m, dtype, e, k, capacity,
                 routing, seed, "ad-hoc case")
    return make_inputs(w)


def random_weights(rng: np.random.Generator, s: int, k: int) -> np.ndarray:
    """Positive float32 per-route weights in (0, 1], for op-level tests of combine."""
    return rng.uniform(0.0, 1.0, size=(s, k)).astype(np.float32) + np.float32(2.0 ** -20)


def random_idx(rng: np.random.Generator, s: int, e: int, k: int) -> np.ndarray:
    """Distinct expert ids per token, uniformly chosen, int32 [s, k]."""
    if s == 0:
        return np.zeros((0, k), np.int32)
    keys = rng.random((s, e))
    return np.argsort(keys, axis=1)[:, :k].astype(np.int32)


def skewed_idx(rng: np.random.Generator, s: int, e: int, k: int, hot: int = 0) -> np.ndarray:
    """Every token routes to expert `hot` plus k-1 distinct others (maximal skew)."""
    idx = random_idx(rng, s, e, k)
    for t in range(s):
        row = idx[t]
        if hot not in row:
            row[-1] = hot
    return idx


# Output features of the expert projection that consumes the dispatched rows (the pages
# fix no expert width; this is the gate/up projection width used for the grouped GEMM).
EXPERT_WIDTH = 3072


def expert_weights(seed: int, e: int, n: int, m: int, dtype: str) -> np.ndarray:
    """Expert projection weights [e, n, m] (output x input features), N(0, 1/m) draws
    stored in dtype, generated expert by expert from one seeded stream."""
    rng = np.random.default_rng(seed)
    out = None
    scale = np.float32(1.0 / np.sqrt(m))
    for x in range(e):
        wx = cast_input(rng.standard_normal((n, m), dtype=np.float32) * scale, dtype)
        if out is None:
            out = np.empty((e, n, m), dtype=wx.dtype)
        out[x] = wx
    return out


def describe(w: Workload) -> str:
    mode = "dropless" if w.dropless else f"capacity {w.capacity}"
    return f"{w.name}: s={w.s} m={w.m} {w.dtype} e={w.e} k={w.k} {mode} ({w.routing})"


def bytes_per_elem(dtype: str) -> int:
    return ELEM_BYTES[dtype]


__all__ = [
    "WORKLOADS", "HEADLINE", "Workload", "Inputs", "make_inputs", "random_case",
    "random_weights", "random_idx", "skewed_idx", "cast_input", "f32_to_bf16_bits",
    "capacity_from_factor", "describe", "bytes_per_elem", "DTYPES", "ELEM_BYTES",
]
