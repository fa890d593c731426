"""Pins for the block-wise quantization and block-scaled GEMM oracle.

Pinned by: a plain-loop restatement of the block rule on small inputs (every
block's amax, scale and codes, ragged last block included), the reduction to
per-token quantization when one block spans the row, block locality, the
reduction of the block-scaled GEMM to the plain GEMM when the scales are
constant along K, and exact rational brute force on tiny block-scaled GEMMs.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import blockwise as B, fp8, gemm as G, quantize as Q, stochastic as S
import workloads


@pytest.mark.parametrize("bs", [16, 32, 64])
@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_block_rule_by_plain_loops(bs, fmt):
    rng = np.random.default_rng(bs + fmt)
    x = (rng.standard_normal((3, 80)) * np.exp(rng.standard_normal((3, 80)) * 3)).astype(np.float32)
    x[1, 5] = np.nan
    x[2, 70] = np.inf
    q, s, a = B.quantize_blockwise(x, Q.F32, fmt, bs)
    nb = -(-80 // bs)
    assert s.shape == (3, nb) and a.shape == (3, nb)
    fmax = fp8.fmax(fmt)
    for i in range(3):
        for b in range(nb):
            vals = [float(v) for v in x[i, b * bs:min(80, (b + 1) * bs)]]
            fin = [abs(v) for v in vals if v == v and abs(v) != float("inf")]
            amax = np.float32(max(fin, default=0.0))
            assert a[i, b] == amax
            sc = max(np.float32(amax / np.float32(fmax)), np.float32(2.0 ** -126))
            assert s[i, b] == sc
            r = np.float32(np.float32(1.0) / sc)
            for c in range(b * bs, min(80, (b + 1) * bs)):
                assert q[i, c] == fp8.encode(np.array([np.float32(x[i, c] * r)], np.float32), fmt)[0]


def test_one_block_per_row_is_per_token():
    rng = np.random.default_rng(4)
    bits = workloads.random_bf16(rng, (9, 64), std=2.0)
    for bs in (64, 128):
        q, s, a = B.quantize_blockwise(bits, Q.BF16, fp8.E4M3, bs)
        q_t, s_t, a_t = Q.quantize_dynamic(bits, Q.BF16, fp8.E4M3, Q.PER_TOKEN)
        assert np.array_equal(q, q_t)
        assert np.array_equal(s[:, 0], s_t) and np.array_equal(a[:, 0], a_t)


def test_blocks_are_independent():
    rng = np.random.default_rng(5)
    x1 = rng.standard_normal((4, 64)).astype(np.float32)
    x2 = (rng.standard_normal((4, 48)) * 1e3).astype(np.float32)
    q, s, _ = B.quantize_blockwise(np.concatenate([x1, x2], axis=1), Q.F32, fp8.E4M3, 32)
    q1, s1, _ = B.quantize_blockwise(x1, Q.F32, fp8.E4M3, 32)
    q2, s2, _ = B.quantize_blockwise(x2, Q.F32, fp8.E4M3, 32)
    assert np.array_equal(q, np.concatenate([q1, q2], axis=1))
    assert np.array_equal(s, np.concatenate([s1, s2], axis=1))


def test_stochastic_blockwise_uses_the_block_scale():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((5, 96)) * 1e-3).astype(np.float32)
    q, s, _ = B.quantize_blockwise(x, Q.F32, fp8.E5M2, 32, stochastic=True, seed=77)
    _, s_d, _ = B.quantize_blockwise(x, Q.F32, fp8.E5M2, 32)
    assert np.array_equal(s, s_d)
    r = Q.reciprocal(s)
    y = (x * np.repeat(r, 32, axis=1)).astype(np.float32)
    u = S.uniforms(77, np.arange(x.size, dtype=np.uint64)).reshape(x.shape)
    assert np.array_equal(q, S.encode_e5m2_stochastic(y, u))


def test_gemm_with_constant_block_scales_is_the_plain_gemm():
    rng = np.random.default_rng(7)
    t = fp8.decode_table(fp8.E4M3)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    xq, wq = rng.choice(finite, (6, 96)), rng.choice(finite, (5, 96))
    xs = rng.uniform(0.1, 2, 6).astype(np.float32)
    ws = rng.uniform(0.1, 2, 5).astype(np.float32)
    ref = B.gemm_blockscaled(xq, fp8.E4M3, wq, fp8.E4M3, np.repeat(xs[:, None], 3, 1), np.repeat(ws[:, None], 3, 1),
                             32)
    plain = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    at = G.abs_terms(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    assert np.all(np.abs(ref - plain) <= 2.0 ** -45 * at)


@pytest.mark.parametrize("k,bs", [(64, 32), (80, 32), (96, 64), (48, 16)])
def test_gemm_exact_rationals(k, bs):
    rng = np.random.default_rng(k + bs)
    ta, tb = fp8.decode_table(fp8.E4M3), fp8.decode_table(fp8.E5M2)
    fa = np.array([c for c in range(256) if np.isfinite(ta[c])], dtype=np.uint8)
    fb = np.array([c for c in range(256) if np.isfinite(tb[c])], dtype=np.uint8)
    m, n = 3, 4
    xq, wq = rng.choice(fa, (m, k)), rng.choice(fb, (n, k))
    nb = -(-k // bs)
    xs = rng.uniform(1e-3, 1.0, (m, nb)).astype(np.float32)
    ws = rng.uniform(1e-3, 1.0, (n, nb)).astype(np.float32)
    ref = B.gemm_blockscaled(xq, fp8.E4M3, wq, fp8.E5M2, xs, ws, bs)
    rows, at = B.gemm_blockscaled_rows(xq, fp8.E4M3, wq, fp8.E5M2, xs, ws, bs,
                                       np.array([[i, j] for i in range(m) for j in range(n)]))
    for i in range(m):
        for j in range(n):
            exact = Fraction(0)
            for c in range(k):
                exact += (Fraction(float(ta[xq[i, c]])) * Fraction(float(tb[wq[j, c]])) *
                          Fraction(float(xs[i, c // bs])) * Fraction(float(ws[j, c // bs])))
            assert abs(Fraction(float(ref[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 300)
            assert rows[i * n + j] == pytest.approx(float(exact), rel=2.0 ** -45, abs=1e-300)


def _bf16_value(bits16: int) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits16) << 16))[0]


def test_gemm_bias_exact_rationals():
    """Reading B4: the bias is one more term in output units, exactly."""
    rng = np.random.default_rng(31)
    ta, tb = fp8.decode_table(fp8.E4M3), fp8.decode_table(fp8.E4M3)
    fa = np.array([c for c in range(256) if np.isfinite(ta[c])], dtype=np.uint8)
    m, n, k, bs = 2, 5, 64, 32
    xq, wq = rng.choice(fa, (m, k)), rng.choice(fa, (n, k))
    xs = rng.uniform(1e-3, 1.0, (m, 2)).astype(np.float32)
    ws = rng.uniform(1e-3, 1.0, (n, 2)).astype(np.float32)
    bias = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    bias[(bias & 0x7F80) == 0x7F80] = 0x3F80  # finite values only (1.0 for Inf/NaN patterns)
    ref = B.gemm_blockscaled(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bs, bias=bias)
    rows, at = B.gemm_blockscaled_rows(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bs,
                                       np.array([[i, j] for i in range(m) for j in range(n)]), bias=bias)
    for i in range(m):
        for j in range(n):
            exact = Fraction(_bf16_value(bias[j]))
            for c in range(k):
                exact += (Fraction(float(ta[xq[i, c]])) * Fraction(float(tb[wq[j, c]])) *
                          Fraction(float(xs[i, c // bs])) * Fraction(float(ws[j, c // bs])))
            assert abs(Fraction(float(ref[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 300)
            assert rows[i * n + j] == pytest.approx(float(exact), rel=2.0 ** -45, abs=1e-300)
            assert at[i * n + j] >= abs(_bf16_value(bias[j]))


def test_gemm_zero_codes_return_the_bias():
    bias = np.array([0x3F80, 0xC040, 0x0000, 0x8000, 0x4B00], dtype=np.uint16)  # 1, -3, 0, -0, 2^23
    xq = np.zeros((3, 96), np.uint8)
    wq = np.zeros((5, 96), np.uint8)
    xs, ws = np.ones((3, 3), np.float32), np.ones((5, 3), np.float32)
    ref = B.gemm_blockscaled(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, 32, bias=bias)
    assert np.array_equal(ref, np.tile([1.0, -3.0, 0.0, 0.0, 2.0 ** 23], (3, 1)))
