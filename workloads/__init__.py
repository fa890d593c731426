"""Seeded synthetic inputs for the five workloads of the FP8 quantize + a8w8 GEMM path.

This module only draws random numbers and rounds them to the storage dtype. It
holds none of the method's arithmetic (no amax, scale, cast or GEMM), so the
CPU oracle and the GPU path can both take their inputs from here without
sharing any of the computation they are compared on.

Every generator uses one ``numpy.random.default_rng(seed)`` (PCG64) stream and
draws the tensors in the order the workload lists them. Values are drawn in
float32; bf16 tensors are rounded to nearest-even by torch on the CPU and
returned as ``uint16`` bit patterns, so every consumer sees identical bytes.

Workloads (sizes as stated for each):
  * tiny per-tensor      X fp32 [16,128], W fp32 [64,128], both N(0,1), seed 0
  * PTPC square          X bf16 [4096,4096] N(0,1) with 0.1% of entries x50,
                         W bf16 [4096,4096] N(0, 0.02^2), seed 1
  * decode skinny        X bf16 [M,7168] Student-t(4), W bf16 [2048,7168]
                         N(0, 0.02^2), seed 2
  * grouped MoE          W bf16 [8,2048,1024] N(0, 0.02^2), X bf16 [8192,1024]
                         N(0,1), per-expert row counts from a seeded multinomial
                         with two zero-probability experts, seed 3
  * training linear      12 layers: X [2048,1024], W [4096,1024], G [2048,4096],
                         bf16, with a per-step log-normal factor, seed 4
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to_bf16_bits", "bf16_bits_to_f32", "tiny_per_tensor", "ptpc_square",
    "decode_skinny", "grouped_moe", "training_linear", "MOE_EXPERT_PROBS",
    "random_bf16", "random_f32",
]

# Expert probabilities for the grouped workload. Two experts have probability
# zero so the "some experts get 0 rows" case always occurs.
MOE_EXPERT_PROBS = (0.25, 0.0, 0.20, 0.15, 0.15, 0.0, 0.15, 0.10)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even, via torch on the CPU); return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for building inputs only)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def random_f32(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    return x


def random_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return to_bf16_bits(random_f32(rng, shape, std))


def tiny_per_tensor(seed: int = 0):
    """X fp32 [16,128] then W fp32 [64,128], both N(0,1)."""
    rng = np.random.default_rng(seed)
    x = random_f32(rng, (16, 128))
    w = random_f32(rng, (64, 128))
    return x, w


def ptpc_square(seed: int = 1, m: int = 4096, n: int = 4096, k: int = 4096,
                outlier_frac: float = 0.001, outlier_mult: float = 50.0):
    """X bf16 [m,k] N(0,1) with round(frac*m*k) distinct entries multiplied by 50
    before the bf16 rounding; W bf16 [n,k] N(0, 0.02^2). Returns uint16 bits."""
    rng = np.random.default_rng(seed)
    x = random_f32(rng, (m, k))
    n_out = int(round(outlier_frac * m * k))
    if n_out:
        idx = rng.choice(m * k, size=n_out, replace=False)
        flat = x.reshape(-1)
        flat[idx] = (flat[idx] * np.float32(outlier_mult)).astype(np.float32)
    w = random_f32(rng, (n, k), std=0.02)
    return to_bf16_bits(x), to_bf16_bits(w)


def decode_skinny(m: int, seed: int = 2, n: int = 2048, k: int = 7168):
    """X bf16 [m,k] Student-t(nu=4); W bf16 [n,k] N(0, 0.02^2). Returns uint16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(4.0, size=(m, k)).astype(np.float32)
    w = random_f32(rng, (n, k), std=0.02)
    return to_bf16_bits(x), to_bf16_bits(w)


def grouped_moe(seed: int = 3, experts: int = 8, n: int = 2048, k: int = 1024,
                tokens: int = 8192, probs=MOE_EXPERT_PROBS):
    """W bf16 [E,n,k] N(0, 0.02^2); X bf16 [tokens,k] N(0,1); per-expert row counts
    from rng.multinomial(tokens, probs); offsets int32 [E+1] = [0, cumsum(counts)]."""
    rng = np.random.default_rng(seed)
    w = random_f32(rng, (experts, n, k), std=0.02)
    x = random_f32(rng, (tokens, k))
    p = np.asarray(probs, dtype=np.float64)
    p = p / p.sum()
    counts = rng.multinomial(tokens, p)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return to_bf16_bits(x), to_bf16_bits(w), offsets


def training_linear(seed: int = 4, layers: int = 12, steps: int = 20, m: int = 2048,
                    k: int = 1024, n: int = 4096):
    """Base tensors per layer (X [m,k] N(0,1), W [n,k] N(0,0.02^2), G [m,n]
    N(0,1e-3^2), float32) and a per-(step, layer, tensor) factor exp(0.2*N(0,1)).

    Returns (base, factors): base[l] = (x, w, g) float32; factors float32
    [steps, layers, 3]. A step's bf16 inputs are to_bf16_bits(base * factor).
    """
    rng = np.random.default_rng(seed)
    base = []
    for _ in range(layers):
        x = random_f32(rng, (m, k))
        w = random_f32(rng, (n, k), std=0.02)
        g = random_f32(rng, (m, n), std=1e-3)
        base.append((x, w, g))
    factors = np.exp(0.2 * rng.standard_normal((steps, layers, 3))).astype(np.float32)
    return base, factors


def training_step_inputs(base, factors, step: int, layer: int):
    """bf16 bits of (X, W, G) for one step and layer: base tensor times its factor."""
    x, w, g = base[layer]
    fx, fw, fg = factors[step, layer]
    return (to_bf16_bits(x * fx), to_bf16_bits(w * fw), to_bf16_bits(g * fg))
