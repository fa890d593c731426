"""Block-wise FP8 scaling and the block-scaled a8w8 GEMM.

Oracle (test infrastructure only; see the package docstring).

What is computed (hip-quant README, "Block-wise FP8 Scaling" and "Block-scaled
Linear and Adafactor Kernel Helpers"): FP8 bytes plus one float32 dequant scale
per block of `block_size` consecutive elements along the last dimension, so
value ~= fp8_value * block_scale and an input [rows, K] has scales
[rows, ceil(K / block_size)]; the block-scaled linear consumes FP8 bytes and
the two scale tensors directly.

Readings where the README leaves a step open:
  B1  A block's scale follows the per-group rule of the other granularities:
      amax over the block's finite elements, s = max(fl32(amax / fmax), 2^-126),
      r = fl32(1 / s), q = saturating RNE cast of fl32(x * r). The last block
      of a row holds K mod block_size elements when that is not zero.
  B2  The block-scaled GEMM is
        out[m, n] = sum_b xs[m, b] * ws[n, b] * sum_{k in block b} dec(XQ[m,k]) * dec(WQ[n,k])
      with both operands blocked along K with the same block size, written as
      bf16.
  B3  Stochastic block-wise E5M2 (quantize_e5m2_blockwise_stochastic) is the
      block scale of B1 with the stochastic cast of oracle/stochastic.py.
  B4  The optional bias of the block-scaled linear is bf16, one value per
      output column, in output units: it is added to the block sum (in
      float32 on the device), before the bf16 rounding of the output.
"""
from __future__ import annotations

import numpy as np

from . import fp8, gemm as G, quantize as Q, stochastic as S


def block_count(cols: int, block_size: int) -> int:
    return -(-cols // block_size)


def quantize_blockwise(x: np.ndarray, dtype: int, fmt: int, block_size: int, stochastic: bool = False,
                       seed: int = 0):
    """Returns (q uint8 [rows, cols], scales float32 [rows, nb], amax float32 [rows, nb])."""
    x32 = Q.widen(x, dtype)
    if x32.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x32.shape
    nb = block_count(cols, block_size)
    a = np.abs(x32.astype(np.float64))
    a = np.where(np.isfinite(a), a, 0.0)
    pad = np.zeros((rows, nb * block_size))
    pad[:, :cols] = a
    amax = pad.reshape(rows, nb, block_size).max(axis=2).astype(np.float32)
    s = Q.scale_from_amax(amax, fmt)
    r = Q.reciprocal(s)
    r_el = np.repeat(r, block_size, axis=1)[:, :cols]
    y = (x32 * r_el).astype(np.float32)
    if stochastic:
        if fmt != fp8.E5M2:
            raise ValueError("stochastic rounding produces E5M2")
        u = S.uniforms(seed, np.arange(y.size, dtype=np.uint64)).reshape(y.shape)
        q = S.encode_e5m2_stochastic(y, u)
    else:
        q = fp8.encode(y, fmt)
    return q, s, amax


def gemm_blockscaled(xq, xf: int, wq, wf: int, x_scales, w_scales, block_size: int, bias=None) -> np.ndarray:
    """float64 reference [M, N] of readings B2 and B4 (bias: bf16 bits [N] or None)."""
    a = fp8.decode(xq, xf)
    b = fp8.decode(wq, wf)
    m, k = a.shape
    n = b.shape[0]
    nb = block_count(k, block_size)
    xs = np.asarray(x_scales, dtype=np.float32).reshape(m, nb).astype(np.float64)
    ws = np.asarray(w_scales, dtype=np.float32).reshape(n, nb).astype(np.float64)
    out = np.zeros((m, n))
    for blk in range(nb):
        sl = slice(blk * block_size, min(k, (blk + 1) * block_size))
        out += (a[:, sl] @ b[:, sl].T) * xs[:, blk, None] * ws[None, :, blk]
    if bias is not None:
        out += G.bf16_bits_to_f64(bias)[None, :]
    return out


def gemm_blockscaled_rows(xq, xf: int, wq, wf: int, x_scales, w_scales, block_size: int, pairs, bias=None):
    """Reference and sum of |terms| (the bias one of them) at selected (m, n)
    positions."""
    ta, tb = fp8.decode_table(xf), fp8.decode_table(wf)
    xq = np.asarray(xq, dtype=np.uint8)
    wq = np.asarray(wq, dtype=np.uint8)
    m, k = xq.shape
    n = wq.shape[0]
    nb = block_count(k, block_size)
    xs = np.asarray(x_scales, dtype=np.float32).reshape(m, nb).astype(np.float64)
    ws = np.asarray(w_scales, dtype=np.float32).reshape(n, nb).astype(np.float64)
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    a = ta[xq[pairs[:, 0]]]
    b = tb[wq[pairs[:, 1]]]
    blk = np.arange(k) // block_size
    sc = xs[pairs[:, 0]][:, blk] * ws[pairs[:, 1]][:, blk]
    t = a * b * sc
    ref, at = t.sum(axis=1), np.abs(t).sum(axis=1)
    if bias is not None:
        bv = G.bf16_bits_to_f64(bias)[pairs[:, 1]]
        ref, at = ref + bv, at + np.abs(bv)
    return ref, at


def tolerance_blockscaled(ref, absterms, nblocks: int):
    """Allowed |out - ref|: the plain GEMM bound plus one float32 rounding of
    the block scale product and of the rescaling FMA per block, each at most
    2^-24 of the running sum of |terms|."""
    return G.tolerance(ref, absterms) + (nblocks + 2) * 2.0 ** -24 * np.asarray(absterms, dtype=np.float64)
