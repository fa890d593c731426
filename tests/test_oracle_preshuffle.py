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
    k = 256  # two 128-column blocks per fragment row block
    cases = {
        (0, 0): 0,
        (1, 0): 16,            # next slot
        (0, 1): 1,             # next byte in the slot's piece
        (0, 16): 1024,         # second 16-byte half of the first quarter
        (0, 32): 256,          # quarter 1 -> piece 16
        (0, 96): 768,          # quarter 3 -> piece 48
        (8, 0): 64,            # n32 = 8: g = 1 -> slot 4
        (4, 0): 4096,          # n32 = 4: p = 1 -> second fragment of the group
        (31, 127): 6143,       # g 3, p 1, r 3 -> fragment 1 slot 15, last byte
        (0, 128): 2048,        # next K block of the same fragment
        (32, 0): 8192,         # next 32-row group -> fragment 2
        (13, 130): 6226,       # g 1, p 1, r 1 -> fragment 1 slot 5, K block 1, byte 2
    }
    for (n, kk), off in cases.items():
        assert int(P.offset_of(n, kk, k)) == off, (n, kk)


def test_fragment_pair_holds_eight_consecutive_rows_per_slot_quad():
    """Slots 4g..4g+3 of the two fragments of a 32-row group hold rows
    8g .. 8g+7 of the group: first 4 in fragment 0, next 4 in fragment 1."""
    k = 128
    for g in range(4):
        rows = []
        for p_ in range(2):
            for r in range(4):
                slot = 4 * g + r
                off = p_ * 2048 + slot * 16     # k = 0 of fragment p_
                n = [n for n in range(32) if int(P.offset_of(n, 0, k)) == off]
                rows.append(n[0])
        assert rows == list(range(8 * g, 8 * g + 8))
