"""Dynamic and delayed FP8 quantization: amax, scale, codes, amax-history ring.

Oracle (test infrastructure only; see the package docstring).

What is computed, and where the pages say so:
  * Granularity and scale count (fuel-ir 0.22.4 ``quant_scale.rs``, the module
    table and ``ScaleGranularity::scale_count``): per-tensor -> 1 scale,
    per-token -> one per row, per-channel -> one per column of a [rows, cols]
    tensor.
  * amax per group, then scale = amax / fmax (448 for E4M3), then a saturating
    round-to-nearest-even cast of the scaled value (the method statement; the
    hip-quant README "Scale / amax tracking" section: "scaled, then
    quantized"; its "Training-path numerical guards" treat the quant scale as a
    pre-quant multiplier whose reciprocal is the dequant scale).
  * Delayed scaling (AstrAI ``ops.cu`` commit message "finalize fp8 scale rings
    inside quantize kernels", and ``pack_quantize_params``): a float32 ring
    [hist[len] | scale | counter]; the quantize folds this step's amax into
    hist[idx], reduces the window and publishes the next scale. hip-quant's
    ``Fp8TensorMeta`` uses a 16-entry history and ignores NaN/Inf amax samples,
    keeping the last valid scale with a sticky ``found_nonfinite`` flag.

Readings taken where the pages leave a step open:
  A1  q = cast(fl32(x * r)) with r = fl32(1 / s) computed once per group.
  A2  per-channel means one scale per *column*; the GEMM's per-output-channel
      weight scale for W [N, K] is the per-row (per-token) call on W.
  A3  amax is the largest |x| over the group's finite elements; s is floored at
      2^-126 (the smallest normal float32) so r stays finite and an all-zero
      group encodes to zeros.
  A6  the ring window is reduced with max; next scale = max * 2^margin / fmax;
      an all-zero window keeps the scale; the initial state is hist = 0,
      scale = 1, counter = 0; idx is the caller's slot for this step.
  A7  in delayed mode the codes use the scale held in the ring when the call
      starts (s_t), which is also what the call reports as its scale; the ring
      then holds s_{t+1}.
"""
from __future__ import annotations

import numpy as np

from . import fp8

PER_TENSOR = 0
PER_TOKEN = 1
PER_CHANNEL = 2

F32 = 0
BF16 = 1

SCALE_FLOOR = np.float32(2.0 ** -126)

_GRAN_NAMES = {PER_TENSOR: "per_tensor", PER_TOKEN: "per_token", PER_CHANNEL: "per_channel"}


def scale_count(gran: int, rows: int, cols: int) -> int:
    """Number of float32 scales for a [rows, cols] tensor (1 / rows / cols)."""
    if gran == PER_TENSOR:
        return 1
    if gran == PER_TOKEN:
        return rows
    if gran == PER_CHANNEL:
        return cols
    raise ValueError(f"unknown granularity {gran}")


def granularity_name(gran: int) -> str:
    return _GRAN_NAMES[gran]


def widen(x: np.ndarray, dtype: int) -> np.ndarray:
    """Load and widen: bf16 bit patterns (uint16) or float32 -> float32, exactly."""
    if dtype == BF16:
        bits = np.asarray(x, dtype=np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32)
    if dtype == F32:
        return np.asarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def group_amax(x32: np.ndarray, gran: int):
    """amax over the finite elements of each group, and whether the group held a
    non-finite element. Returns (amax float32 [count], nonfinite bool [count])."""
    a = np.abs(x32.astype(np.float64))
    finite = np.isfinite(a)
    a = np.where(finite, a, 0.0)
    if gran == PER_TENSOR:
        amax = np.array([a.max(initial=0.0)])
        nonfinite = np.array([not finite.all()])
    elif gran == PER_TOKEN:
        amax = a.max(axis=1, initial=0.0)
        nonfinite = ~finite.all(axis=1)
    elif gran == PER_CHANNEL:
        amax = a.max(axis=0, initial=0.0)
        nonfinite = ~finite.all(axis=0)
    else:
        raise ValueError(f"unknown granularity {gran}")
    # every |x| of a float32 is a float32, so the max converts back exactly
    return amax.astype(np.float32), nonfinite


def scale_from_amax(amax: np.ndarray, fmt: int) -> np.ndarray:
    """s = max(fl32(amax / fmax), 2^-126), float32 division (correctly rounded)."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(fp8.fmax(fmt))).astype(np.float32)
    return np.maximum(s, SCALE_FLOOR).astype(np.float32)


def reciprocal(s: np.ndarray) -> np.ndarray:
    """r = fl32(1 / s), float32 division."""
    return (np.float32(1.0) / np.asarray(s, dtype=np.float32)).astype(np.float32)


def _broadcast(vals: np.ndarray, gran: int) -> np.ndarray:
    if gran == PER_TENSOR:
        return vals.reshape(1, 1)
    if gran == PER_TOKEN:
        return vals.reshape(-1, 1)
    return vals.reshape(1, -1)


def cast_scaled(x32: np.ndarray, r: np.ndarray, gran: int, fmt: int) -> np.ndarray:
    """Codes = encode(fl32(x * r)) with r broadcast over its group."""
    scaled = (x32 * _broadcast(np.asarray(r, dtype=np.float32), gran)).astype(np.float32)
    return fp8.encode(scaled, fmt)


def quantize_dynamic(x: np.ndarray, dtype: int, fmt: int, gran: int):
    """Dynamic quantization of a 2-D tensor.

    Returns (q uint8 [rows, cols], scale float32 [count], amax float32 [count]).
    ``scale`` is the dequant scale s: x ~= decode(q) * s.
    """
    x32 = widen(x, dtype)
    if x32.ndim != 2:
        raise ValueError("x must be 2-D")
    amax, _ = group_amax(x32, gran)
    s = scale_from_amax(amax, fmt)
    r = reciprocal(s)
    q = cast_scaled(x32, r, gran, fmt)
    return q, s, amax


def quantize_with_scale(x: np.ndarray, dtype: int, fmt: int, s):
    """Per-tensor quantization with a given dequant scale s (no reduction
    decides it): q = encode(fl32(x * fl32(1 / s))). This is the backward
    re-quantization of AstrAI ``ops.cu`` (``linear_backward_fp8`` quantizes the
    weight and the input again with their forward scales, no ring update).

    Returns (q uint8, s float32 [1], amax float32 [1]) with amax over the finite
    elements, as the other forms report it.
    """
    x32 = widen(x, dtype)
    if x32.ndim != 2:
        raise ValueError("x must be 2-D")
    s = np.asarray(s, dtype=np.float32).reshape(1)
    q = cast_scaled(x32, reciprocal(s), PER_TENSOR, fmt)
    amax, _ = group_amax(x32, PER_TENSOR)
    return q, s, amax


# ---------------------------------------------------------------------------
# delayed scaling: the amax-history ring
# ---------------------------------------------------------------------------

def ring_new(length: int = 16) -> np.ndarray:
    """Initial ring state: float32 [length + 2] = [hist = 0 | scale = 1 | counter = 0]."""
    if length < 1:
        raise ValueError("ring length must be >= 1")
    st = np.zeros(length + 2, dtype=np.float32)
    st[length] = 1.0
    return st


def ring_update(state: np.ndarray, idx: int, margin: int, amax: float,
                nonfinite: bool, fmt: int, flag: int = 0):
    """Fold one amax sample into the ring and publish the next scale.

    Returns (new_state, new_flag). The rules, in order:
      * a non-finite sample (or a tensor that held a non-finite element) leaves
        history and scale unchanged and sets the sticky flag;
      * otherwise hist[idx] = amax, w = max(hist);
        - w == 0 keeps the scale;
        - else cand = fl32(fl32(w * 2^margin) / fmax); a finite cand becomes the
          scale (floored at 2^-126); a non-finite cand keeps the scale and sets
          the flag;
      * the counter slot is always left at 0.
    """
    st = np.array(state, dtype=np.float32, copy=True)
    length = st.size - 2
    if not 0 <= idx < length:
        raise ValueError("ring idx out of range")
    amax = np.float32(amax)
    if nonfinite or not np.isfinite(amax):
        flag = 1
    else:
        st[idx] = amax
        w = np.float32(st[:length].max())
        if w > 0:
            shifted = np.ldexp(w, np.int32(margin)).astype(np.float32)
            cand = np.float32(shifted / np.float32(fp8.fmax(fmt)))
            if np.isfinite(cand):
                st[length] = max(cand, SCALE_FLOOR)
            else:
                flag = 1
    st[length + 1] = 0.0
    return st, flag


def quantize_delayed(x: np.ndarray, dtype: int, fmt: int, state: np.ndarray,
                     idx: int, margin: int, flag: int = 0):
    """Per-tensor quantization with the scale taken from the ring (delayed).

    Returns (q, scale_used float32 [1], amax float32 [1], new_state, new_flag):
    the codes use s_t = state[len] as read at the call, r = fl32(1 / s_t); the
    tensor's amax (finite elements) is then folded into the ring.
    """
    x32 = widen(x, dtype)
    st = np.asarray(state, dtype=np.float32)
    length = st.size - 2
    s_t = np.float32(st[length])
    r = reciprocal(np.array([s_t]))
    q = cast_scaled(x32, r, PER_TENSOR, fmt)
    amax, nonfinite = group_amax(x32, PER_TENSOR)
    new_state, new_flag = ring_update(st, idx, margin, amax[0], bool(nonfinite[0]), fmt, flag)
    return q, np.array([s_t], dtype=np.float32), amax, new_state, new_flag
