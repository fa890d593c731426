"""Byte map of the pre-shuffled FP8 weight layout.

Oracle (test infrastructure only; see the package docstring).

The aiter PR "gemm_a8w8_bpreshuffle_out" (Technical Details, Test Plan) has
the GEMM read a weight WQ [N, K] that was pre-shuffled into a kernel-friendly
order, and allows a K-padded WQ; it does not print the order. The order below
is this library's own, written from its specification (not from kernel code):

  * N is padded with zero rows to NP = ceil(N / 32) * 32 and K with zero
    columns to KP = ceil(K / 128) * 128.
  * Each group of 32 rows (output channels) n = 32*G + n32 is split over two
    fragments of 16 "slots": with n32 = 8*g + 4*p + r (g in 0..3, p in 0..1,
    r in 0..3) the row goes to fragment nb = 2*G + p, slot s = 4*g + r.
  * Fragment (nb, kb) covers slots 0..15 and columns kb*128 .. kb*128+127 and
    starts at byte (nb * (KP / 128) + kb) * 2048, so one fragment row block is
    contiguous along K.
  * Inside a fragment, the byte of slot s and column k_in (0..127) sits at
        h * 1024 + (q * 16 + s) * 16 + b
    with q = k_in // 32, h = (k_in % 32) // 16, b = k_in % 16. A 64-lane
    wavefront reads one half-fragment as 64 consecutive 16-byte pieces.

Padding bytes are 0x00 (+0.0 in both FP8 formats).
"""
from __future__ import annotations

import numpy as np

FRAG_N = 16
GROUP_N = 32
FRAG_K = 128
FRAG_BYTES = FRAG_N * FRAG_K


def padded_dims(n: int, k: int):
    np_ = -(-n // GROUP_N) * GROUP_N
    kp = -(-k // FRAG_K) * FRAG_K
    return np_, kp


def preshuffled_bytes(n: int, k: int) -> int:
    np_, kp = padded_dims(n, k)
    return np_ * kp


def offset_of(n_idx, k_idx, k: int):
    """Byte offset of element (n, k) of WQ in the pre-shuffled buffer."""
    n_idx = np.asarray(n_idx, dtype=np.int64)
    k_idx = np.asarray(k_idx, dtype=np.int64)
    _, kp = padded_dims(1, k)
    kblocks = kp // FRAG_K
    grp, n32 = n_idx // GROUP_N, n_idx % GROUP_N
    g, p, r = n32 // 8, (n32 // 4) % 2, n32 % 4
    nb = 2 * grp + p
    slot = 4 * g + r
    kb, k_in = k_idx // FRAG_K, k_idx % FRAG_K
    q = k_in // 32
    h = (k_in % 32) // 16
    b = k_in % 16
    return (nb * kblocks + kb) * FRAG_BYTES + h * 1024 + (q * 16 + slot) * 16 + b


def preshuffle(wq: np.ndarray) -> np.ndarray:
    """uint8 [N, K] -> uint8 [preshuffled_bytes(N, K)]."""
    wq = np.asarray(wq, dtype=np.uint8)
    n, k = wq.shape
    out = np.zeros(preshuffled_bytes(n, k), dtype=np.uint8)
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    out[offset_of(nn, kk, k).reshape(-1)] = wq.reshape(-1)
    return out


def unshuffle(buf: np.ndarray, n: int, k: int) -> np.ndarray:
    """Inverse of preshuffle: uint8 [preshuffled_bytes(N, K)] -> uint8 [N, K]."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    return buf[offset_of(nn, kk, k)].reshape(n, k)
