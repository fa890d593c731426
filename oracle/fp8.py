"""OCP FP8 formats: closed-form decode tables and the saturating RNE encoder.

Oracle (test infrastructure only; see the package docstring).

Formats, as the hip-quant 0.6.0 README states them ("Supported Quantization
Formats", table "FP8 Formats (both APIs)"):
  E4M3: 1 sign, 4 exponent, 3 mantissa bits, bias 7, largest magnitude 448,
        NaN but no infinities; used for forward activations and weights.
  E5M2: 1 sign, 5 exponent, 2 mantissa bits, bias 15, largest magnitude 57344,
        +-Inf and NaN; used for backward gradients.
The same README says the default conversion follows OCP semantics with
round-to-nearest-even; the method statement asks for a *saturating* cast.

Readings where the pages are silent:
  * NaN encodes to the canonical 0x7F for both formats (the sign of a NaN is
    not meaningful on a GPU, so it is dropped).
  * Magnitudes at or above the format maximum, +-Inf included, saturate to the
    signed maximum code (E4M3 0x7E / 0xFE = +-448, E5M2 0x7B / 0xFB = +-57344).
  * A tie between two representable neighbours goes to the code with an even
    mantissa LSB, i.e. the even code.
  * The sign of the input is kept, so -0.0 and negatives that round to zero
    encode to 0x80.
"""
from __future__ import annotations

import numpy as np

E4M3 = 0
E5M2 = 1

# (exponent bits, mantissa bits, bias, largest finite code, largest finite value)
_SPEC = {
    E4M3: (4, 3, 7, 0x7E, 448.0),
    E5M2: (5, 2, 15, 0x7B, 57344.0),
}

NAN_CODE = 0x7F


def fmax(fmt: int) -> float:
    """Largest finite magnitude of the format (448 for E4M3, 57344 for E5M2)."""
    return _SPEC[fmt][4]


def max_code(fmt: int) -> int:
    """Code of the largest finite positive value."""
    return _SPEC[fmt][3]


def _decode_one(code: int, fmt: int) -> float:
    """Value of one FP8 code, written out from the bit-field definition."""
    ebits, mbits, bias, _, _ = _SPEC[fmt]
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    e_all_ones = (1 << ebits) - 1
    if fmt == E4M3:
        # No infinities: only exponent 1111 with mantissa 111 is NaN; exponent
        # 1111 with other mantissas holds ordinary normal numbers.
        if e == e_all_ones and m == (1 << mbits) - 1:
            return float("nan")
    else:
        # IEEE-like: exponent all ones is Inf (mantissa 0) or NaN.
        if e == e_all_ones:
            return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        # subnormal: m * 2^(1 - bias - mbits)
        return sign * m * 2.0 ** (1 - bias - mbits)
    # normal: (2^mbits + m) * 2^(e - bias - mbits)
    return sign * ((1 << mbits) + m) * 2.0 ** (e - bias - mbits)


_TABLES: dict[int, np.ndarray] = {}


def decode_table(fmt: int) -> np.ndarray:
    """float64[256]: value of every code (exact in float64)."""
    if fmt not in _TABLES:
        _TABLES[fmt] = np.array([_decode_one(c, fmt) for c in range(256)], dtype=np.float64)
    return _TABLES[fmt]


def decode(codes: np.ndarray, fmt: int) -> np.ndarray:
    """Decode uint8 codes to float64 values."""
    return decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def encode(v: np.ndarray, fmt: int) -> np.ndarray:
    """Saturating round-to-nearest-even cast of float32 values to FP8 codes.

    The magnitude is matched against the table of non-negative finite values
    (all exact in float64), the nearer neighbour wins, a tie goes to the even
    code, and magnitudes >= the format maximum (Inf included) saturate.
    """
    v = np.asarray(v, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        return _encode(v, fmt)


def _encode(v: np.ndarray, fmt: int) -> np.ndarray:
    table = decode_table(fmt)
    top = max_code(fmt)
    mags = table[: top + 1]                       # codes 0..top, strictly increasing
    a = np.abs(v.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    hi = np.searchsorted(mags, a, side="left")   # first code with value >= a
    hi = np.minimum(hi, top)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= fmax(fmt), top, code).astype(np.uint8)
    code = code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0)).astype(np.uint8)
    code = np.where(nan, np.uint8(NAN_CODE), code).astype(np.uint8)
    return code
