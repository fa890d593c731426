"""Pins for the oracle's pre-shuffled weight byte map.

The layout is this library's own (the aiter PR only says the weight is
pre-shuffled and may be K-padded). It is pinned by bijectivity, zero padding,
positions worked out by hand from the layout's specification, and (in the GPU
tests) by the GEMM on pre-shuffled weights matching the plain oracle GEMM.
"""
import numpy as np
import pytest

from oracle import preshuffle as P


@pytest.mark.parametrize("n,k", [(16, 128), (40, 300), (1, 16), (33, 4096 + 16), (64, 128)])
def test_round_trip_and_padding(n, k):
    rng = np.random.default_rng(n * 1000 + k)
    w = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    buf = P.preshuffle(w)
    np_, kp = P.padded_dims(n, k)
    assert buf.size == np_ * kp == P.preshuffled_bytes(n, k)
    assert np.array_equal(P.unshuffle(buf, n, k), w)
    # every byte of the buffer is either an element of W or a zero pad byte
    nn, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    used = np.zeros(buf.size, dtype=bool)
    used[P.offset_of(nn, kk, k).reshape(-1)] = True
    assert used.sum() == n * k
    assert np.all(buf[~used] == 0)


def test_hand_derived_positions():
    k = 256  # two 128-column blocks per 16-row block
    cases = {
        (0, 0): 0,
        (1, 0): 16,            # next lane
        (0, 1): 1,             # next byte in the lane
        (0, 16): 1024,         # second 16-byte half of the first quarter
        (0, 32): 256,          # quarter 1 -> lane 16
        (0, 96): 768,          # quarter 3 -> lane 48
        (15, 127): 2047,       # last byte of a fragment
        (0, 128): 2048,        # next K block of the same rows
        (16, 0): 4096,         # next 16-row block (after 2 K blocks)
        (17, 130): 4096 + 2048 + 16 + 2,
    }
    for (n, kk), off in cases.items():
        assert int(P.offset_of(n, kk, k)) == off, (n, kk)
