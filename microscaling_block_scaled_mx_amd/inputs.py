"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no arithmetic of the method: it draws normal numbers,
rounds them to bf16 bit patterns and splits token counts over experts.
Recipe: ``numpy.random.default_rng(seed)``; each tensor is
``standard_normal(shape, float32) * sigma``, then rounded to bf16
(nearest-even), drawn in the order listed by each workload builder.

The workloads stand in for the shapes the pages train at (Flux 12B linears
and MLP, and a Qwen3-30B-A3B-sized routed-expert MLP); there are no
datasets or trained weights here, only value scales: activations and
upstream gradients N(0, 1), weights N(0, 0.02), fc1 bias N(0, 0.01).
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest-even (inputs only)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_normal(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return f32_to_bf16_bits(x)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ workloads
def gemm_pair(seed: int, M: int, N: int, K: int, sigma_a=1.0, sigma_b=1.0):
    """A [M,K], B [N,K] bf16 (the 256^3 MXFP4 parity workload uses seed 101)."""
    rng = np.random.default_rng(seed)
    return bf16_normal(rng, (M, K), sigma_a), bf16_normal(rng, (N, K), sigma_b)


def linear(seed: int, M: int, N: int, K: int):
    """MX linear workload: X [M,K] ~N(0,1), W [N,K] ~N(0,0.02), dY [M,N] ~N(0,1).
    The Flux-12B attention-projection shape is M=4096, N=K=3072 (seed 201)."""
    rng = np.random.default_rng(seed)
    X = bf16_normal(rng, (M, K), 1.0)
    W = bf16_normal(rng, (N, K), 0.02)
    dY = bf16_normal(rng, (M, N), 1.0)
    return X, W, dY


def mlp(seed: int, M: int, D: int, F: int, with_bias: bool = True):
    """Fused MLP workload: X [M,D], W1 [F,D], b1 [F], W2 [D,F], dY [M,D].
    The Flux-12B MLP shape is M=8192, D=3072, F=12288 (seed 301)."""
    rng = np.random.default_rng(seed)
    X = bf16_normal(rng, (M, D), 1.0)
    W1 = bf16_normal(rng, (F, D), 0.02)
    b1 = bf16_normal(rng, (F,), 0.01) if with_bias else None
    W2 = bf16_normal(rng, (D, F), 0.02)
    dY = bf16_normal(rng, (M, D), 1.0)
    return X, W1, b1, W2, dY


FLUX_LINEARS = (("qkv", 3072, 9216), ("out", 3072, 3072), ("mlp_up", 3072, 12288),
                ("mlp_down", 12288, 3072), ("adaln", 3072, 18432))


def expert_counts(seed: int, R: int, G: int, zero_expert: int, align: int = 128):
    """Per-expert row counts: multinomial over G experts (one forced empty),
    each rounded to a multiple of ``align``, the remainder added to the
    largest count (lowest index on ties).  Returns (counts, offsets) where
    offsets are cumulative ends (int32)."""
    rng = np.random.default_rng(seed)
    p = np.full(G, 1.0 / (G - 1))
    p[zero_expert] = 0.0
    raw = rng.multinomial(R, p)
    c = (align * np.floor(raw / align + 0.5)).astype(np.int64)
    c[zero_expert] = 0
    c[int(np.argmax(c))] += R - int(c.sum())
    assert c[zero_expert] == 0 and (c % align == 0).all() and c.sum() == R and (c >= 0).all()
    return c, np.cumsum(c).astype(np.int32), rng


def grouped_mlp(seed: int, R: int, D: int, F: int, G: int, zero_expert: int = 3):
    """Routed-expert SwiGLU MLP workload: counts, then X [R,D], W1 [G,2F,D]
    ([gate|up] rows), W2 [G,D,F], dY [R,D] (seed 501 at R=32768, D=2048,
    F=768, G=8)."""
    counts, offsets, rng = expert_counts(seed, R, G, zero_expert)
    X = bf16_normal(rng, (R, D), 1.0)
    W1 = bf16_normal(rng, (G, 2 * F, D), 0.02)
    W2 = bf16_normal(rng, (G, D, F), 0.02)
    dY = bf16_normal(rng, (R, D), 1.0)
    return counts, offsets, X, W1, W2, dY
