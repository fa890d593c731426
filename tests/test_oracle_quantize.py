"""Pins for the oracle's amax / scale / code computation at the three granularities.

Pinned by: the scale counts and names fuel-ir's quant_scale.rs prints (golden
fixture), the E4M3 half-ulp error bound the method implies, the invariant that
every group with a non-zero amax holds a +-fmax code, the per-channel /
per-token transpose identity, brute-force amax on small inputs, torch's bf16
widening, and closed-form scales for special amax values.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8, quantize as Q
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scale_granularity.json")


def test_scale_count_and_names_match_fuel_ir():
    with open(GOLDEN) as f:
        g = json.load(f)
    for case in g["scale_count"]:
        gran = g["names"][case["granularity"]]
        assert Q.scale_count(gran, case["rows"], case["cols"]) == case["count"]
        assert Q.granularity_name(gran) == case["granularity"]
    for p in g["pairs"]:
        a, w = g["names"][p["activation"]], g["names"][p["weight"]]
        assert f"act_{Q.granularity_name(a)}_weight_{Q.granularity_name(w)}" == p["symbol"]


def test_bf16_widening_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = Q.widen(bits, Q.BF16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_amax_brute_force_small():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 9)).astype(np.float32)
    x[2, 3] = np.nan
    x[4, 0] = -np.inf
    x[5, :] = 0.0
    for gran in (Q.PER_TENSOR, Q.PER_TOKEN, Q.PER_CHANNEL):
        amax, nonfinite = Q.group_amax(x, gran)
        if gran == Q.PER_TENSOR:
            groups = [[float(v) for v in x.reshape(-1)]]
        elif gran == Q.PER_TOKEN:
            groups = [[float(v) for v in row] for row in x]
        else:
            groups = [[float(v) for v in col] for col in x.T]
        for i, grp in enumerate(groups):
            fin = [abs(v) for v in grp if v == v and abs(v) != float("inf")]
            assert amax[i] == max(fin, default=0.0)
            assert nonfinite[i] == (len(fin) != len(grp))


def test_scale_closed_forms():
    amax = np.array([448.0, 896.0, 0.0, 1.0, 3.0e-39, 448.0 * 2.0 ** -140], dtype=np.float32)
    s = Q.scale_from_amax(amax, fp8.E4M3)
    assert s[0] == 1.0 and s[1] == 2.0
    assert s[2] == np.float32(2.0 ** -126)           # floor for an all-zero group
    assert s[3] == np.float32(1.0) / np.float32(448.0)
    assert s[4] == np.float32(2.0 ** -126) and s[5] == np.float32(2.0 ** -126)
    s5 = Q.scale_from_amax(np.array([57344.0], dtype=np.float32), fp8.E5M2)
    assert s5[0] == 1.0


def _ulp_fp8(v: np.ndarray, fmt: int) -> np.ndarray:
    mbits, bias = (3, 7) if fmt == fp8.E4M3 else (2, 15)
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, 1 - bias)
    return np.ldexp(1.0, (e - mbits).astype(np.int64))


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
@pytest.mark.parametrize("gran", [Q.PER_TENSOR, Q.PER_TOKEN, Q.PER_CHANNEL])
def test_half_ulp_error_bound(fmt, gran):
    rng = np.random.default_rng(11)
    x = rng.standard_t(4, size=(33, 160)).astype(np.float32)
    bits = workloads.to_bf16_bits(x)
    q, s, amax = Q.quantize_dynamic(bits, Q.BF16, fmt, gran)
    x32 = Q.widen(bits, Q.BF16).astype(np.float64)
    sb = s.astype(np.float64)
    sb = sb.reshape(1, 1) if gran == Q.PER_TENSOR else (sb.reshape(-1, 1) if gran == Q.PER_TOKEN else sb.reshape(1, -1))
    v = x32 / sb
    dec = fp8.decode(q, fmt)
    bound = 0.5 * _ulp_fp8(v, fmt) + 2.0 ** -22 * np.abs(v)
    inside = np.abs(v) <= fp8.fmax(fmt)
    assert np.all(np.abs(dec - v)[inside] <= bound[inside])
    assert np.all(np.abs(dec[~inside]) == fp8.fmax(fmt))


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
@pytest.mark.parametrize("gran", [Q.PER_TENSOR, Q.PER_TOKEN, Q.PER_CHANNEL])
def test_every_nonzero_group_hits_fmax(fmt, gran):
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((40, 48)) * np.exp(rng.standard_normal((40, 1)) * 3)).astype(np.float32)
    x[3] = 0.0
    q, s, amax = Q.quantize_dynamic(x, Q.F32, fmt, gran)
    mags = q & 0x7F
    top = fp8.max_code(fmt)
    if gran == Q.PER_TENSOR:
        hits = [np.any(mags == top)]
    elif gran == Q.PER_TOKEN:
        hits = np.any(mags == top, axis=1)
    else:
        hits = np.any(mags == top, axis=0)
    for i, h in enumerate(hits):
        assert h == (amax[i] > 0)


def test_per_channel_is_transposed_per_token():
    rng = np.random.default_rng(13)
    x = workloads.to_bf16_bits(rng.standard_normal((24, 40)).astype(np.float32) * 3)
    for fmt in (fp8.E4M3, fp8.E5M2):
        qc, sc, ac = Q.quantize_dynamic(x, Q.BF16, fmt, Q.PER_CHANNEL)
        qt, st, at = Q.quantize_dynamic(np.ascontiguousarray(x.T), Q.BF16, fmt, Q.PER_TOKEN)
        assert np.array_equal(qc, qt.T)
        assert np.array_equal(sc, st) and np.array_equal(ac, at)


def test_per_tensor_equals_per_token_for_one_row():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((1, 300)).astype(np.float32)
    a = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, Q.PER_TENSOR)
    b = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, Q.PER_TOKEN)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_requantizing_the_dequantized_tensor_is_idempotent():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    q, s, _ = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, Q.PER_TOKEN)
    deq = (fp8.decode(q, fp8.E4M3) * s.reshape(-1, 1).astype(np.float64)).astype(np.float32)
    q2 = Q.cast_scaled(deq, Q.reciprocal(s), Q.PER_TOKEN, fp8.E4M3)
    assert np.array_equal(q, q2)


def test_zero_and_nonfinite_groups():
    x = np.zeros((3, 32), dtype=np.float32)
    x[0, 0] = -0.0
    x[1, :] = 1.0
    x[1, 5] = np.nan
    x[1, 6] = np.inf
    x[1, 7] = -np.inf
    q, s, amax = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, Q.PER_TOKEN)
    assert amax[0] == 0 and s[0] == np.float32(2.0 ** -126)
    assert q[0, 0] == 0x80 and np.all(q[0, 1:] == 0) and np.all(q[2] == 0)
    assert amax[1] == 1.0 and s[1] == np.float32(1.0) / np.float32(448.0)
    assert q[1, 5] == 0x7F and q[1, 6] == 0x7E and q[1, 7] == 0xFE
    assert q[1, 0] == 0x7E


def test_planted_mistake_is_caught():
    """A dropped rounding step (truncation instead of RNE) breaks the bound."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    q, s, _ = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, Q.PER_TOKEN)
    v = x.astype(np.float64) / s.reshape(-1, 1)
    t = fp8.decode_table(fp8.E4M3)
    # truncating encoder: largest table value <= |v|
    mags = t[:0x7F]
    trunc = np.searchsorted(mags, np.abs(v), side="right") - 1
    dec_bad = np.sign(v) * mags[np.clip(trunc, 0, 0x7E)]
    bound = 0.5 * _ulp_fp8(v, fp8.E4M3) + 2.0 ** -22 * np.abs(v)
    assert not np.all(np.abs(dec_bad - v) <= bound)


# ---- per-tensor quantization with a given scale (backward re-quantization) ----

@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_given_scale_equal_to_dynamic_scale_reproduces_dynamic_codes(fmt):
    rng = np.random.default_rng(31)
    bits = workloads.random_bf16(rng, (33, 48), std=3.0)
    q_dyn, s_dyn, a_dyn = Q.quantize_dynamic(bits, Q.BF16, fmt, Q.PER_TENSOR)
    q, s, a = Q.quantize_with_scale(bits, Q.BF16, fmt, s_dyn)
    assert np.array_equal(q, q_dyn)
    assert s.view(np.uint32)[0] == s_dyn.view(np.uint32)[0]
    assert a.view(np.uint32)[0] == a_dyn.view(np.uint32)[0]


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_given_scale_saturates_above_fmax_and_rounds_within_half_ulp_below(fmt):
    """A scale a quarter of the dynamic one pushes the largest values past fmax:
    they must encode to +-max, the rest to within half an FP8 ulp (plus the
    float32 rounding of x * r) of x / s, measured with the decode table."""
    rng = np.random.default_rng(32)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    fmax = fp8.fmax(fmt)
    s = np.float32(np.abs(x).max() / fmax / 4.0)
    q, s_out, amax = Q.quantize_with_scale(x, Q.F32, fmt, s)
    assert s_out[0] == s and amax[0] == np.float32(np.abs(x).max())
    table = fp8.decode_table(fmt)
    v = x.astype(np.float64) / float(s)
    dec = table[q]
    max_code = 0x7E if fmt == fp8.E4M3 else 0x7B
    big = np.abs(v) > fmax * (1 + 2.0 ** -20)
    assert big.any()
    assert np.all(q[big] == np.where(v[big] > 0, max_code, 0x80 | max_code))
    small = np.abs(v) < fmax * (1 - 2.0 ** -20)
    mant = 3 if fmt == fp8.E4M3 else 2
    emin = -6 if fmt == fp8.E4M3 else -14
    e = np.floor(np.log2(np.maximum(np.abs(v[small]), 2.0 ** emin)))
    half_ulp = np.ldexp(0.5, (e - mant).astype(np.int64))
    assert np.all(np.abs(dec[small] - v[small]) <= half_ulp + 2.0 ** -22 * np.abs(v[small]))
