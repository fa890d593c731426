"""Pins for the stochastic-rounding E5M2 oracle.

Pinned by: the Philox-4x32-10 known-answer vectors published with the
generator (golden fixture), closed forms of the rounding rule (representable
values never move, u = 0 rounds every inexact value up, the result is always one
of the two neighbours), unbiasedness in expectation (the README's reason for the
method), the saturation / NaN / sign rules shared with the deterministic cast,
and equality of the scales with the deterministic quantization.
"""
import json
import os

import numpy as np
import pytest

from oracle import fp8, quantize as Q, stochastic as S
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_philox_known_answer_vectors():
    with open(GOLDEN) as f:
        kat = json.load(f)["vectors"]
    for v in kat:
        ctr = np.array([[int(w, 16) for w in v["ctr"]]], dtype=np.uint32)
        key = [int(w, 16) for w in v["key"]]
        out = S.philox4x32_10(ctr, key)[0]
        assert [f"{int(w):08x}" for w in out] == v["out"]


def test_uniforms_layout_and_range():
    """Element i takes word i % 4 of the counter i // 4 (reading S1)."""
    seed = (7 << 32) | 99
    u = S.uniforms(seed, np.arange(12, dtype=np.uint64))
    words = S.philox4x32_10(np.array([[0, 0, 0, 0], [1, 0, 0, 0], [2, 0, 0, 0]], dtype=np.uint32), (99, 7))
    assert np.array_equal(u, (words.reshape(-1) >> 8).astype(np.float64) * 2.0 ** -24)
    big = S.uniforms(5, np.array([2 ** 34 + 6], dtype=np.uint64))
    w = S.philox4x32_10(np.array([[(2 ** 32 + 1) & 0xFFFFFFFF, 1, 0, 0]], dtype=np.uint32), (5, 0))[0, 2]
    assert big[0] == (int(w) >> 8) * 2.0 ** -24
    many = S.uniforms(1, np.arange(1 << 16, dtype=np.uint64))
    assert many.min() >= 0.0 and many.max() < 1.0 and abs(many.mean() - 0.5) < 0.01


def test_representable_values_never_move():
    t = fp8.decode_table(fp8.E5M2)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    y = t[finite].astype(np.float32)
    for u in (0.0, 0.5, 1.0 - 2.0 ** -24):
        codes = S.encode_e5m2_stochastic(y, np.full(y.shape, u))
        # +-0 keep their sign bit; every other value its own code
        assert np.array_equal(codes, finite)


def test_result_is_always_a_neighbour_and_u_zero_rounds_up():
    rng = np.random.default_rng(2)
    y = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-6, 4, 20000)).astype(np.float32)
    t = fp8.decode_table(fp8.E5M2)
    mags = np.unique(t[(t >= 0) & np.isfinite(t)])
    a = np.abs(y.astype(np.float64))
    j = np.searchsorted(mags, a, side="right") - 1
    lo, hi = mags[j], mags[np.minimum(j + 1, mags.size - 1)]
    for u in (0.0, rng.uniform(size=y.size)):
        dec = np.abs(t[S.encode_e5m2_stochastic(y, np.broadcast_to(u, y.shape))])
        assert np.all((dec == lo) | (dec == hi))
        assert np.array_equal(np.signbit(t[S.encode_e5m2_stochastic(y, np.broadcast_to(u, y.shape))]), np.signbit(y))
    dec0 = np.abs(t[S.encode_e5m2_stochastic(y, np.zeros(y.shape))])
    assert np.array_equal(dec0, np.where(a > lo, hi, lo))


def test_unbiased_in_expectation():
    """Mean of the decoded codes over 2^16 draws within 4 standard errors of
    the value, for values in the normal and the subnormal E5M2 range."""
    t = fp8.decode_table(fp8.E5M2)
    for v in (1.1, 3.3e-5, 7.0e-6, 1000.7, -0.37):
        n = 1 << 16
        u = S.uniforms(12345, np.arange(n, dtype=np.uint64))
        dec = t[S.encode_e5m2_stochastic(np.full(n, v, np.float32), u)]
        a = abs(float(np.float32(v)))
        j = np.searchsorted(np.unique(t[(t >= 0) & np.isfinite(t)]), a, side="right") - 1
        mags = np.unique(t[(t >= 0) & np.isfinite(t)])
        gap = mags[j + 1] - mags[j]
        se = gap / 2 / np.sqrt(n)
        assert abs(dec.mean() - float(np.float32(v))) < 4 * se


def test_saturation_nan_and_zero():
    y = np.array([57344.0, 60000.0, np.inf, -np.inf, np.nan, 0.0, -0.0], dtype=np.float32)
    codes = S.encode_e5m2_stochastic(y, np.zeros(y.shape))
    assert codes.tolist() == [0x7B, 0x7B, 0x7B, 0xFB, 0x7F, 0x00, 0x80]


@pytest.mark.parametrize("gran", [Q.PER_TENSOR, Q.PER_TOKEN, Q.PER_CHANNEL])
def test_scales_equal_deterministic_quantization(gran):
    rng = np.random.default_rng(8)
    bits = workloads.random_bf16(rng, (24, 48), std=1e-3)
    q, s, a = S.quantize_stochastic(bits, Q.BF16, gran, seed=3)
    q_d, s_d, a_d = Q.quantize_dynamic(bits, Q.BF16, fp8.E5M2, gran)
    assert np.array_equal(s.view(np.uint32), s_d.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), a_d.view(np.uint32))
    # codes differ from round-to-nearest by at most one step in magnitude
    t = fp8.decode_table(fp8.E5M2)
    mags = np.unique(t[(t >= 0) & np.isfinite(t)])
    step = np.abs(np.searchsorted(mags, np.abs(t[q])) - np.searchsorted(mags, np.abs(t[q_d])))
    assert step.max() <= 1 and (step == 1).any()


def test_given_scale_stochastic_with_the_dynamic_scale_is_the_dynamic_stochastic():
    rng = np.random.default_rng(61)
    x = (rng.standard_normal((12, 64)) * 3).astype(np.float32)
    q_dyn, s_dyn, _ = S.quantize_stochastic(x, Q.F32, Q.PER_TENSOR, seed=99)
    q_giv, s_giv = S.quantize_with_scale_stochastic(x, Q.F32, s_dyn, seed=99)
    assert np.array_equal(q_giv, q_dyn) and s_giv[0] == s_dyn[0]


def test_given_scale_stochastic_codes_neighbour_the_deterministic_ones():
    """With a scale that saturates part of the tensor: saturated values keep
    the saturated code, the rest lie at most one E5M2 step from round-to-nearest,
    on the side of the exact value."""
    rng = np.random.default_rng(62)
    x = (rng.standard_normal((16, 128)) * 10).astype(np.float32)
    s = np.float32(np.abs(x).max() / fp8.fmax(fp8.E5M2) / 4)
    q_sr, _ = S.quantize_with_scale_stochastic(x, Q.F32, s, seed=7)
    q_rn, _, _ = Q.quantize_with_scale(x, Q.F32, fp8.E5M2, s)
    t = fp8.decode_table(fp8.E5M2)
    y = (x * np.float32(np.float32(1) / s)).astype(np.float32).astype(np.float64)
    d_sr, d_rn = t[q_sr], t[q_rn]
    sat = np.abs(y) >= fp8.fmax(fp8.E5M2)
    assert np.array_equal(q_sr[sat], q_rn[sat])
    lo = np.minimum(d_sr, d_rn)[~sat]
    hi = np.maximum(d_sr, d_rn)[~sat]
    # both codes bracket y: the stochastic one is a neighbour of y, never farther
    assert np.all((d_sr[~sat] == d_rn[~sat]) | ((lo <= y[~sat]) & (y[~sat] <= hi)))
