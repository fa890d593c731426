"""Pins for the oracle's float64 a8w8 GEMM, its grouped variant and the tolerance.

Pinned by exact rational brute force (fractions.Fraction) on tiny shapes and on
the 16x64x128 tiny per-tensor workload, by one-hot operands that reproduce the
scales exactly, by the grouped result equalling per-expert brute force, and by
closed-form values of the bf16 ulp.
"""
import numpy as np
import pytest

from oracle import fp8, gemm as G, quantize as Q
import workloads


def _rand_codes(rng, shape, fmt):
    t = fp8.decode_table(fmt)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    return rng.choice(finite, size=shape)


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (4, 2, 33), (2, 3, 130)])
def test_float64_gemm_matches_exact_rationals(fmt, shape):
    m, n, k = shape
    rng = np.random.default_rng(sum(shape) + fmt)
    xq = _rand_codes(rng, (m, k), fmt)
    wq = _rand_codes(rng, (n, k), fmt)
    xs = rng.uniform(0.01, 2, size=m).astype(np.float32)
    ws = rng.uniform(0.01, 2, size=n).astype(np.float32)
    ref = G.gemm_a8w8(xq, fmt, wq, fmt, xs, ws)
    exact = G.gemm_a8w8_exact(xq, fmt, wq, fmt, xs, ws)
    for i in range(m):
        for j in range(n):
            e = float(exact[i][j])
            assert abs(ref[i, j] - e) <= 2.0 ** -50 * max(abs(e), 1e-300)


def test_tiny_per_tensor_workload_exact():
    x, w = workloads.tiny_per_tensor(0)
    xq, xs, _ = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, Q.PER_TENSOR)
    wq, ws, _ = Q.quantize_dynamic(w, Q.F32, fp8.E4M3, Q.PER_TENSOR)
    ref = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    exact = G.gemm_a8w8_exact(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    e = np.array([[float(v) for v in row] for row in exact])
    assert ref.shape == (16, 64)
    assert np.all(np.abs(ref - e) <= 2.0 ** -50 * np.abs(e))
    # and the scaled result is close to the float product of the inputs
    approx = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.max(np.abs(ref - approx)) < 0.1 * np.max(np.abs(approx))


def test_one_hot_operands_reproduce_scales():
    m, n, k = 5, 6, 64
    xq = np.zeros((m, k), dtype=np.uint8)
    wq = np.zeros((n, k), dtype=np.uint8)
    one = 0x38  # 1.0 in E4M3
    for i in range(m):
        xq[i, i] = one
    for j in range(n):
        wq[j, j % m] = one
    xs = np.array([0.5, 3.0, 7.25, 1e-3, 2.0], dtype=np.float32)
    ws = np.array([1.5, 0.25, 4.0, 9.0, 1e-2, 3.0], dtype=np.float32)
    ref = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    for i in range(m):
        for j in range(n):
            want = float(xs[i]) * float(ws[j]) if j % m == i else 0.0
            assert ref[i, j] == want


def test_broadcast_scalar_scales():
    rng = np.random.default_rng(3)
    xq = _rand_codes(rng, (4, 32), fp8.E4M3)
    wq = _rand_codes(rng, (3, 32), fp8.E4M3)
    a = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, np.float32(0.5), np.float32(2.0))
    b = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, np.full(4, 0.5, np.float32), np.full(3, 2.0, np.float32))
    assert np.array_equal(a, b)


def test_mixed_format_pair():
    rng = np.random.default_rng(4)
    xq = _rand_codes(rng, (3, 40), fp8.E5M2)
    wq = _rand_codes(rng, (2, 40), fp8.E4M3)
    ref = G.gemm_a8w8(xq, fp8.E5M2, wq, fp8.E4M3, np.float32(1), np.float32(1))
    exact = G.gemm_a8w8_exact(xq, fp8.E5M2, wq, fp8.E4M3, np.float32(1), np.float32(1))
    for i in range(3):
        for j in range(2):
            assert ref[i, j] == float(exact[i][j])


def test_sampled_positions_match_full_reference():
    rng = np.random.default_rng(5)
    xq = _rand_codes(rng, (20, 96), fp8.E4M3)
    wq = _rand_codes(rng, (30, 96), fp8.E4M3)
    xs = rng.uniform(0.1, 1, 20).astype(np.float32)
    ws = rng.uniform(0.1, 1, 30).astype(np.float32)
    full = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    fat = G.abs_terms(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    pairs = np.array([[0, 0], [19, 29], [7, 13], [3, 0]])
    ref, at = G.gemm_a8w8_rows(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, pairs)
    assert np.array_equal(ref, full[pairs[:, 0], pairs[:, 1]])
    assert np.allclose(at, fat[pairs[:, 0], pairs[:, 1]], rtol=1e-15, atol=0)


def test_ulp_bf16_closed_forms():
    u = G.ulp_bf16(np.array([1.0, 1.5, 1.99, 2.0, -3.0, 0.0, 2.0 ** -140, 448.0]))
    assert list(u) == [2.0 ** -7, 2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6,
                       2.0 ** -133, 2.0 ** -133, 2.0 ** 1]


def test_tolerance_rejects_one_wrong_term():
    """Dropping a single product term is outside the tolerance."""
    rng = np.random.default_rng(6)
    xq = _rand_codes(rng, (8, 256), fp8.E4M3)
    wq = _rand_codes(rng, (8, 256), fp8.E4M3)
    xs = np.float32(0.01)
    ws = np.float32(0.02)
    ref = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    at = G.abs_terms(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    bad = G.gemm_a8w8(xq[:, 1:], fp8.E4M3, wq[:, 1:], fp8.E4M3, xs, ws)
    term = fp8.decode(xq[:, :1], fp8.E4M3) * fp8.decode(wq[:, :1], fp8.E4M3).T * 0.01 * 0.02
    big = np.abs(term) > 4 * G.tolerance(ref, at)
    assert big.any()
    assert np.all(np.abs(bad - ref)[big] > G.tolerance(ref, at)[big])


def test_grouped_equals_per_expert_brute_force():
    rng = np.random.default_rng(7)
    e, n, k = 4, 5, 48
    counts = [3, 0, 1, 4]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t = int(offsets[-1])
    xq = _rand_codes(rng, (t, k), fp8.E4M3)
    wq = _rand_codes(rng, (e, n, k), fp8.E4M3)
    xs = rng.uniform(0.1, 1, t).astype(np.float32)
    ws = rng.uniform(0.1, 1, (e, n)).astype(np.float32)
    ref, at, covered = G.grouped_gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, offsets)
    assert covered.all()
    for ex in range(e):
        lo, hi = offsets[ex], offsets[ex + 1]
        if hi == lo:
            continue
        exact = G.gemm_a8w8_exact(xq[lo:hi], fp8.E4M3, wq[ex], fp8.E4M3, xs[lo:hi], ws[ex])
        for i in range(hi - lo):
            for j in range(n):
                v = float(exact[i][j])
                assert abs(ref[lo + i, j] - v) <= 2.0 ** -50 * abs(v)


def test_grouped_rows_outside_groups_are_uncovered():
    rng = np.random.default_rng(8)
    xq = _rand_codes(rng, (6, 16), fp8.E4M3)
    wq = _rand_codes(rng, (2, 3, 16), fp8.E4M3)
    offsets = np.array([0, 2, 4], dtype=np.int32)
    ref, _, covered = G.grouped_gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, np.float32(1),
                                          np.ones((2, 3), np.float32), offsets)
    assert list(covered) == [True] * 4 + [False] * 2
    assert np.isnan(ref[4:]).all() and not np.isnan(ref[:4]).any()


def test_workload_generators_are_deterministic():
    a = workloads.grouped_moe(3, tokens=64, n=16, k=32)
    b = workloads.grouped_moe(3, tokens=64, n=16, k=32)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    offsets = a[2]
    counts = np.diff(offsets)
    assert offsets[0] == 0 and offsets[-1] == 64
    assert counts[1] == 0 and counts[5] == 0


# ---- epilogue variants (bias, FP8 output) ----------------------------------------

def test_bias_values_closed_forms():
    import torch
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000], dtype=np.uint16)   # 1, -2, 0.25, 0, -0
    assert np.array_equal(G.bias_values(bits, G.BIAS_BF16),
                          torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy())
    # E4M3: 0x38 = 1, 0x40 = 2, 0x30 = 0.5, 0xB8 = -1, 0x7E = 448; scale 0.25 keeps them exact
    e4 = np.array([0x38, 0x40, 0x30, 0xB8, 0x7E], dtype=np.uint8)
    assert G.bias_values(e4, G.BIAS_E4M3, np.float32(0.25)).tolist() == [0.25, 0.5, 0.125, -0.25, 112.0]
    # E5M2: 0x3C = 1, 0x40 = 2, 0x7B = 57344, 0x01 = 2^-16
    e5 = np.array([0x3C, 0x40, 0x7B, 0x01], dtype=np.uint8)
    assert G.bias_values(e5, G.BIAS_E5M2, np.float32(2.0)).tolist() == [2.0, 4.0, 114688.0, 2.0 ** -15]
    with pytest.raises(ValueError):
        G.bias_values(bits, G.BIAS_BF16, np.float32(1.0))


def test_epilogue_bf16_closed_forms():
    # exact products, then one value exactly halfway between two bf16 numbers (ties to even)
    acc = np.array([3.0, 5.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    out = G.epilogue_f32(acc, np.float32(0.5), np.float32(4.0))
    got = G.bf16_bits_to_f64(out)
    assert got.tolist() == [6.0, 10.0, 2.0, 2.0 + 2.0 ** -5]
    # bias added in float32 after the scales
    out = G.epilogue_f32(np.array([1.0], np.float32), np.float32(1.0), np.float32(1.0), bias_f32=np.float32(-3.0))
    assert G.bf16_bits_to_f64(out).tolist() == [-2.0]


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_epilogue_fp8_output_closed_forms(fmt):
    table = fp8.decode_table(fmt)
    finite = np.array([c for c in range(256) if np.isfinite(table[c])], dtype=np.uint8)
    # every finite code value times a power-of-two out_scale comes back as its own code
    out_scale = np.float32(0.125)
    vals = (table[finite] * 0.125).astype(np.float32)
    codes = G.epilogue_f32(vals, np.float32(1.0), np.float32(1.0), out_scale=out_scale, out_fmt=fmt)
    want = finite.copy()
    want[table[finite] == 0] = np.where(np.signbit(table[finite][table[finite] == 0]), 0x80, 0x00)
    assert np.array_equal(codes, want)
    # saturation and NaN
    big = np.array([1e30, -1e30, np.nan], dtype=np.float32)
    codes = G.epilogue_f32(big, np.float32(1.0), np.float32(1.0), out_scale=np.float32(1.0), out_fmt=fmt)
    mx = 0x7E if fmt == fp8.E4M3 else 0x7B
    assert codes.tolist() == [mx, 0x80 | mx, 0x7F]
