"""Stochastic-rounding E5M2 quantization (for backward gradients).

Oracle (test infrastructure only; see the package docstring).

What is computed (hip-quant README, "Stochastic E5M2 Backward Gradients"): a
value rounds to one of the two adjacent E5M2 values around it, up with
probability proportional to its distance from the lower one, the random number
coming from a stateless per-element hash of (seed, element index).

Readings where the README leaves a step open:
  S1  The hash is the counter-based generator Philox-4x32-10 (Salmon, Moraes,
      Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011),
      written here from its published definition and checked against its
      known-answer vectors. Element i (row-major flat index of the tensor)
      uses word i % 4 of Philox(counter = (i // 4 low 32 bits, i // 4 high 32
      bits, 0, 0), key = (seed low 32 bits, seed high 32 bits)), and
      u = (word >> 8) * 2^-24, a uniform number in [0, 1) on a 2^-24 grid.
  S2  With y = fl32(x * r) (the scaled value, as in the deterministic cast),
      lo <= |y| < hi the adjacent E5M2 magnitudes and p = (|y| - lo) / (hi - lo),
      the magnitude is hi when u < p and lo otherwise (p = 0 for a
      representable |y|, so those never move). |y| >= 57344 (the E5M2 maximum,
      Inf included) saturates to +-57344 as the deterministic cast does; NaN
      gives 0x7F; the sign of y is kept (-0 gives 0x80).
  S3  The scales (amax, s = amax / 57344, r = 1 / s, the ring for delayed
      scaling) are exactly those of the deterministic quantization; only the
      cast changes.
"""
from __future__ import annotations

import numpy as np

from . import fp8
from . import quantize as Q

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32_10(ctr: np.ndarray, key) -> np.ndarray:
    """Philox-4x32-10 of counters ctr [N, 4] (uint32) under key (k0, k1);
    returns [N, 4] uint32. Each round: the products M0 * c0 and M1 * c2 (64-bit)
    give c = (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
    the key advances by the Weyl constants between rounds."""
    c = np.asarray(ctr, dtype=np.uint32).reshape(-1, 4).astype(np.uint64)
    c0, c1, c2, c3 = c[:, 0], c[:, 1], c[:, 2], c[:, 3]
    k0, k1 = np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF)
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = (p1 >> _S32) ^ c1 ^ k0, p1 & _LO32, (p0 >> _S32) ^ c3 ^ k1, p0 & _LO32
        k0 = (k0 + _W0) & _LO32
        k1 = (k1 + _W1) & _LO32
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def uniforms(seed: int, index: np.ndarray) -> np.ndarray:
    """u in [0, 1) for flat element indices (reading S1), float64."""
    idx = np.asarray(index, dtype=np.uint64).reshape(-1)
    blk = idx >> np.uint64(2)
    ctr = np.zeros((idx.size, 4), dtype=np.uint32)
    ctr[:, 0] = (blk & _LO32).astype(np.uint32)
    ctr[:, 1] = (blk >> _S32).astype(np.uint32)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    w = words[np.arange(idx.size), (idx & np.uint64(3)).astype(np.int64)]
    return (w >> np.uint32(8)).astype(np.float64) * 2.0 ** -24


def encode_e5m2_stochastic(y: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Codes of float32 values y with uniforms u (reading S2)."""
    y = np.asarray(y, dtype=np.float32)
    u = np.asarray(u, dtype=np.float64).reshape(y.shape)
    table = fp8.decode_table(fp8.E5M2)
    mags = np.unique(table[(table >= 0) & np.isfinite(table)])       # 0, 2^-16, ..., 57344 ascending
    a = np.abs(y.astype(np.float64))
    fmax = fp8.fmax(fp8.E5M2)
    inside = np.isfinite(a) & (a < fmax)
    j = np.searchsorted(mags, np.where(inside, a, 0.0), side="right") - 1
    lo = mags[j]
    hi = mags[np.minimum(j + 1, mags.size - 1)]
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(hi > lo, (a - lo) / (hi - lo), 0.0)
    mag = np.where(u < p, hi, lo)
    mag = np.where(inside, mag, fmax)
    signed = np.where(np.signbit(y), -mag, mag).astype(np.float32)
    codes = fp8.encode(signed, fp8.E5M2)                            # exact values: their own codes
    return np.where(np.isnan(y), np.uint8(0x7F), codes).astype(np.uint8)


def quantize_stochastic(x: np.ndarray, dtype: int, gran: int, seed: int):
    """Dynamic E5M2 quantization with stochastic rounding (readings S1-S3).
    Returns (q, scale, amax) as quantize_dynamic does."""
    x32 = Q.widen(x, dtype)
    amax, _ = Q.group_amax(x32, gran)
    s = Q.scale_from_amax(amax, fp8.E5M2)
    r = Q.reciprocal(s)
    y = (x32 * Q._broadcast(r, gran)).astype(np.float32)
    u = uniforms(seed, np.arange(y.size, dtype=np.uint64)).reshape(y.shape)
    return encode_e5m2_stochastic(y, u), s, amax


def quantize_delayed_stochastic(x: np.ndarray, dtype: int, state: np.ndarray, idx: int, margin: int, seed: int,
                                flag: int = 0):
    """Delayed (ring) E5M2 quantization with stochastic rounding: the ring
    arithmetic of quantize_delayed, the cast of reading S2."""
    x32 = Q.widen(x, dtype)
    st = np.asarray(state, dtype=np.float32)
    length = st.size - 2
    s_t = np.float32(st[length])
    r = Q.reciprocal(np.array([s_t]))
    y = (x32 * r[0]).astype(np.float32)
    u = uniforms(seed, np.arange(y.size, dtype=np.uint64)).reshape(y.shape)
    q = encode_e5m2_stochastic(y, u)
    amax, nonfinite = Q.group_amax(x32, Q.PER_TENSOR)
    new_state, new_flag = Q.ring_update(st, idx, margin, amax[0], bool(nonfinite[0]), fp8.E5M2, flag)
    return q, np.array([s_t], dtype=np.float32), amax, new_state, new_flag


def quantize_with_scale_stochastic(x: np.ndarray, dtype: int, s, seed: int):
    """Given-scale E5M2 quantization with stochastic rounding (the given-scale
    mode of the fused layouts, reading R18, with the cast of reading S2):
    y = fl32(x * fl32(1/s)), element i draws u from its row-major index.
    Returns (q, s as float32 [1])."""
    x32 = Q.widen(x, dtype)
    s = np.asarray(s, dtype=np.float32).reshape(1)
    r = Q.reciprocal(s)
    y = (x32 * r[0]).astype(np.float32)
    u = uniforms(seed, np.arange(y.size, dtype=np.uint64)).reshape(y.shape)
    return encode_e5m2_stochastic(y, u), s
