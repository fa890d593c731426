"""Pins for the oracle's FP8 decode tables and saturating RNE encoder.

The oracle is checked against what the format definitions fix (bit layout,
bias, maximum, special values: hip-quant README, "FP8 Formats (both APIs)"),
against torch's float8 types as an independent library routine, and against a
second encoder written here with integer round-half-even arithmetic.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_formats.json")
FMTS = {"E4M3": fp8.E4M3, "E5M2": fp8.E5M2}
TORCH_T = {fp8.E4M3: torch.float8_e4m3fn, fp8.E5M2: torch.float8_e5m2}


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# decode table
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["E4M3", "E5M2"])
def test_table_matches_format_definition(name):
    spec = _golden()[name]
    fmt = FMTS[name]
    t = fp8.decode_table(fmt)
    e, m, bias = spec["exponent_bits"], spec["mantissa_bits"], spec["bias"]
    assert 1 + e + m == 8
    finite = t[np.isfinite(t)]
    assert finite.max() == spec["max"] and finite.min() == -spec["max"]
    assert fp8.fmax(fmt) == spec["max"]
    assert t[fp8.max_code(fmt)] == spec["max"]
    assert t[0x80 | fp8.max_code(fmt)] == -spec["max"]
    # smallest subnormal 2^(1-bias-m), smallest normal 2^(1-bias)
    assert t[0x01] == 2.0 ** (1 - bias - m)
    assert t[1 << m] == 2.0 ** (1 - bias)
    assert t[0x00] == 0.0 and not math.copysign(1, t[0x00]) < 0
    assert t[0x80] == 0.0 and math.copysign(1, t[0x80]) < 0
    assert np.isinf(t).any() == spec["has_inf"]
    assert np.isnan(t).any() == spec["has_nan"]


def test_e4m3_special_codes():
    t = fp8.decode_table(fp8.E4M3)
    nan_codes = [c for c in range(256) if np.isnan(t[c])]
    assert nan_codes == [0x7F, 0xFF]
    assert np.isfinite(t).sum() == 254
    assert t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6


def test_e5m2_special_codes():
    t = fp8.decode_table(fp8.E5M2)
    assert t[0x7B] == 57344.0
    assert t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert all(np.isnan(t[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert t[0x01] == 2.0 ** -16 and t[0x04] == 2.0 ** -14


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_table_matches_torch_float8(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TORCH_T[fmt]).to(torch.float64).numpy()
    t = fp8.decode_table(fmt)
    same = (ref == t) | (np.isnan(ref) & np.isnan(t))
    assert same.all()
    # sign of zero too
    assert np.signbit(ref[0x80]) and np.signbit(t[0x80])


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_magnitude_strictly_increasing(fmt):
    t = fp8.decode_table(fmt)
    pos = t[: fp8.max_code(fmt) + 1]
    assert np.all(np.diff(pos) > 0)
    neg = t[0x80: 0x80 + fp8.max_code(fmt) + 1]
    assert np.all(np.diff(neg) < 0)


# --------------------------------------------------------------------------
# encoder
# --------------------------------------------------------------------------

_SPEC = {fp8.E4M3: (3, 7, 0x7E, 0x43E00000), fp8.E5M2: (2, 15, 0x7B, 0x47600000)}


def int_encode(v: np.ndarray, fmt: int) -> np.ndarray:
    """Independent encoder: integer round-half-even on the float32 bit fields."""
    mbits, bias, top, fmax_bits = _SPEC[fmt]
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.int64)
    sign = ((u >> 31) & 1) << 7
    a = u & 0x7FFFFFFF
    ef = a >> 23
    mf = a & 0x7FFFFF
    sig = np.where(ef > 0, mf | (1 << 23), mf)          # significand
    exp2 = np.where(ef > 0, ef - 150, -149)             # value = sig * 2^exp2
    emin = 1 - bias                                      # smallest normal exponent
    # floor(log2|v|) for normal float32 (ef-127); subnormal float32 are far below emin
    e = np.where(ef > 0, ef - 127, -200)
    e_t = np.maximum(e, emin)                           # exponent of the target grid
    p = e_t - mbits                                      # grid spacing 2^p
    sh = p - exp2                                        # right shift of sig
    sh_c = np.clip(sh, 1, 62)
    q_shift = sig >> sh_c
    rem = sig & ((np.int64(1) << sh_c) - 1)
    half = np.int64(1) << (sh_c - 1)
    up = (rem > half) | ((rem == half) & (q_shift & 1 == 1))
    q_right = q_shift + up
    q_left = sig << np.clip(-sh, 0, 62)
    q = np.where(sh > 0, q_right, q_left)
    q = np.where(sh > 62, 0, q)
    normal = e >= emin
    code = np.where(normal, ((e_t + bias) << mbits) + q - (1 << mbits), q)
    code = np.where(a >= fmax_bits, top, code)
    code = np.minimum(code, top)
    code = code | sign
    code = np.where(a > 0x7F800000, 0x7F, code)
    return code.astype(np.uint8)


def _all_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32)


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_encoder_matches_integer_encoder_on_all_bf16(fmt):
    v = _all_bf16_as_f32()
    for mult in (1.0, 3.0, 2.0 ** -20, 2.0 ** 10, 0.7):
        vv = (v * np.float32(mult)).astype(np.float32)
        assert np.array_equal(fp8.encode(vv, fmt), int_encode(vv, fmt))


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_encoder_matches_integer_encoder_on_random_f32(fmt):
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    assert np.array_equal(fp8.encode(v, fmt), int_encode(v, fmt))
    # values concentrated in the format's range
    w = (rng.standard_normal(1 << 20) * fp8.fmax(fmt) / 3).astype(np.float32)
    assert np.array_equal(fp8.encode(w, fmt), int_encode(w, fmt))


def _boundary_values(fmt):
    t = fp8.decode_table(fmt)
    pos = t[: fp8.max_code(fmt) + 1]
    vals = []
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # midpoints are exact in float32
        for x in (np.float32(lo), mid, np.float32(hi)):
            vals += [x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))]
    top = pos[-1]
    ulp_top = top - pos[-2]
    for x in (top, top + ulp_top / 2, top + ulp_top, 2 * top, 1e30):
        x = np.float32(x)
        vals += [x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0))]
    vals = np.array(vals, dtype=np.float32)
    return np.concatenate([vals, -vals])


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_encoder_boundaries(fmt):
    v = _boundary_values(fmt)
    assert np.array_equal(fp8.encode(v, fmt), int_encode(v, fmt))


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_encoder_matches_torch_inside_range(fmt):
    rng = np.random.default_rng(7)
    v = np.concatenate([
        _boundary_values(fmt),
        (rng.standard_normal(1 << 20) * fp8.fmax(fmt) / 4).astype(np.float32),
        _all_bf16_as_f32(),
    ])
    inside = np.isfinite(v) & (np.abs(v.astype(np.float64)) < fp8.fmax(fmt))
    v = v[inside]
    ref = torch.from_numpy(v).to(TORCH_T[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(v, fmt), ref)


def test_saturation_and_specials_e4m3():
    f = fp8.E4M3
    v = np.array([448, 464, 479.9, 480, 1e6, np.inf, -448, -464, -np.inf, np.nan, -np.nan],
                 dtype=np.float32)
    assert list(fp8.encode(v, f)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E,
                                       0xFE, 0xFE, 0xFE, 0x7F, 0x7F]


def test_saturation_and_specials_e5m2():
    f = fp8.E5M2
    v = np.array([57344, 61440, 65536, np.inf, -np.inf, np.nan], dtype=np.float32)
    assert list(fp8.encode(v, f)) == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0x7F]


def test_ties_go_to_even_code():
    f = fp8.E4M3
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A
    assert fp8.encode(np.float32(1.0625), f) == 0x38
    assert fp8.encode(np.float32(1.1875), f) == 0x3A
    # subnormal grid 2^-9: half of the smallest subnormal rounds to zero
    assert fp8.encode(np.float32(2.0 ** -10), f) == 0x00
    assert fp8.encode(np.float32(3 * 2.0 ** -10), f) == 0x02
    assert fp8.encode(np.float32(-(2.0 ** -10)), f) == 0x80
    # binade crossing: halfway between 0x0F (15*2^-9) and 0x10 (2^-5 ... ) picks 0x10
    t = fp8.decode_table(f)
    assert fp8.encode(np.float32((t[0x0F] + t[0x10]) / 2), f) == 0x10


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_round_trip_of_every_finite_code(fmt):
    t = fp8.decode_table(fmt)
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    assert np.array_equal(fp8.encode(t[codes].astype(np.float32), fmt), codes)
