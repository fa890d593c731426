"""Byte map of the pre-shuffled FP8 weight layout.

Oracle (test infrastructure only; see the package docstring).

The aiter PR "gemm_a8w8_bpreshuffle_out" (Technical Details, Test Plan) has
the GEMM read a weight WQ [N, K] that was pre-shuffled into a kernel-friendly
order, and allows a K-padded WQ; it does not print the order. The order below
is this library's own, written from its specification (not from kernel code):

  * N is padded with zero rows to NP = ceil(N / 16) * 16 and K with zero
    columns to KP = ceil(K / 128) * 128.
  * The padded matrix is cut into fragments of 16 rows x 128 columns
    (2048 bytes). Fragment (nb, kb) starts at byte (nb * (KP / 128) + kb) * 2048,
    so one 16-row block is contiguous along K.
  * Inside a fragment, the byte of row n_in (0..15) and column k_in (0..127)
    sits at   h * 1024 + lane * 16 + b   where
        g    = k_in // 32          (which quarter of the 128 columns)
        h    = (k_in % 32) // 16   (which 16-byte half of that quarter)
        b    = k_in % 16
        lane = g * 16 + n_in.
    A 64-lane wavefront therefore reads one half-fragment as 64 consecutive
    16-byte pieces, lane l getting row l % 16 and columns 32*(l//16) + 16*h ..+15.

Padding bytes are 0x00 (+0.0 in both FP8 formats).
"""
from __future__ import annotations

import numpy as np

FRAG_N = 16
FRAG_K = 128
FRAG_BYTES = FRAG_N * FRAG_K


def padded_dims(n: int, k: int):
    np_ = -(-n // FRAG_N) * FRAG_N
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
    nb, n_in = n_idx // FRAG_N, n_idx % FRAG_N
    kb, k_in = k_idx // FRAG_K, k_idx % FRAG_K
    g = k_in // 32
    h = (k_in % 32) // 16
    b = k_in % 16
    lane = g * 16 + n_in
    return (nb * kblocks + kb) * FRAG_BYTES + h * 1024 + lane * 16 + b


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
