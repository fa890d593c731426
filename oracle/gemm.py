"""The scaled FP8 (a8w8) GEMM and its grouped (per-expert) variant, in float64.

Oracle (test infrastructure only; see the package docstring).

What is computed:
  out[m, n] = x_scale[m] * w_scale[n] * sum_k dec(XQ[m, k]) * dec(WQ[n, k])
with XQ [M, K] and WQ [N, K] FP8 codes, per-token (or one) activation scales and
per-output-channel (or one) weight scales, written as bf16. This is the method
statement; the aiter PR "gemm_a8w8_bpreshuffle_out" (Technical Details) gives
the operand shapes XQ [M, K], WQ [N, K], x_scale (M), w_scale (N) and a bf16
[M, N] output, and AstrAI's ``linear_forward_fp8`` the NT layout x @ w^T.
hip-quant's README ("Hardware Status", validated test system) fixes the rule
used here for checking: compare with the *decoded FP8 operands actually
consumed*, not with the original floats.

The grouped variant follows the megablocks-hip grouped-GEMM notes ("Current
mitigation", "hipify & zero-initialisation fix"): per expert, the rows
[off[e], off[e+1]) of the concatenated tokens times that expert's weight,
written over (not accumulated into) the output.

Rounding and tolerance (reading A9): the float32 accumulation order is free;
the reference is float64. An output element passes when
  |out - ref| <= 2 * ulp_bf16(ref) + 2^-22 * sum_k |x_s * w_s * dec * dec|
with ulp_bf16(v) = 2^(floor(log2|v|) - 7), floored at 2^-133.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import fp8


def _scales(vals, count: int) -> np.ndarray:
    v = np.asarray(vals, dtype=np.float32).reshape(-1).astype(np.float64)
    if v.size == 1:
        return np.full(count, v[0])
    if v.size != count:
        raise ValueError(f"scale has {v.size} entries, expected 1 or {count}")
    return v


def gemm_a8w8(xq, xf: int, wq, wf: int, x_scale, w_scale) -> np.ndarray:
    """float64 reference [M, N] on the decoded operands (float64 matmul)."""
    a = fp8.decode(xq, xf)
    b = fp8.decode(wq, wf)
    m, k = a.shape
    n, k2 = b.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    acc = a @ b.T
    return acc * _scales(x_scale, m)[:, None] * _scales(w_scale, n)[None, :]


def abs_terms(xq, xf: int, wq, wf: int, x_scale, w_scale) -> np.ndarray:
    """sum_k |x_s * w_s * dec(XQ) * dec(WQ)| per output element (float64)."""
    a = np.abs(fp8.decode(xq, xf))
    b = np.abs(fp8.decode(wq, wf))
    m, n = a.shape[0], b.shape[0]
    acc = a @ b.T
    return acc * np.abs(_scales(x_scale, m))[:, None] * np.abs(_scales(w_scale, n))[None, :]


def gemm_a8w8_exact(xq, xf: int, wq, wf: int, x_scale, w_scale) -> list:
    """Exact rational result for tiny shapes (brute force with Fraction)."""
    ta = fp8.decode_table(xf)
    tb = fp8.decode_table(wf)
    xq = np.asarray(xq, dtype=np.uint8)
    wq = np.asarray(wq, dtype=np.uint8)
    m, k = xq.shape
    n = wq.shape[0]
    xs = _scales(x_scale, m)
    ws = _scales(w_scale, n)
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += Fraction(float(ta[xq[i, kk]])) * Fraction(float(tb[wq[j, kk]]))
            row.append(acc * Fraction(float(xs[i])) * Fraction(float(ws[j])))
        out.append(row)
    return out


def gemm_a8w8_rows(xq, xf: int, wq, wf: int, x_scale, w_scale, pairs):
    """Reference and abs-terms for selected (m, n) output positions only.

    For very large problems: each element is one float64 dot product."""
    ta = fp8.decode_table(xf)
    tb = fp8.decode_table(wf)
    xq = np.asarray(xq, dtype=np.uint8)
    wq = np.asarray(wq, dtype=np.uint8)
    xs = _scales(x_scale, xq.shape[0])
    ws = _scales(w_scale, wq.shape[0])
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    a = ta[xq[pairs[:, 0]]]
    b = tb[wq[pairs[:, 1]]]
    ref = (a * b).sum(axis=1) * xs[pairs[:, 0]] * ws[pairs[:, 1]]
    at = (np.abs(a) * np.abs(b)).sum(axis=1) * np.abs(xs[pairs[:, 0]]) * np.abs(ws[pairs[:, 1]])
    return ref, at


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """2^(floor(log2|v|) - 7), floored at 2^-133 (one bf16 ulp at |v|)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    u = np.ldexp(1.0, (e - 7).astype(np.int64))
    u = np.where(a > 0, u, 0.0)
    return np.maximum(u, 2.0 ** -133)


def tolerance(ref: np.ndarray, absterms: np.ndarray) -> np.ndarray:
    """Allowed |out - ref| per element."""
    return 2.0 * ulp_bf16(ref) + 2.0 ** -22 * np.asarray(absterms, dtype=np.float64)


def grouped_gemm_a8w8(xq, xf: int, wq_experts, wf: int, x_scale, w_scale, offsets):
    """Grouped reference: out[off[e]:off[e+1]] = gemm(XQ rows, WQ[e], x_s rows, w_s[e]).

    Returns (ref float64 [T, N], absterms [T, N], covered bool [T]); rows of no
    group are NaN in ref and False in covered."""
    xq = np.asarray(xq, dtype=np.uint8)
    wq_experts = np.asarray(wq_experts, dtype=np.uint8)
    offsets = np.asarray(offsets, dtype=np.int64)
    t = xq.shape[0]
    e_count, n, _ = wq_experts.shape
    xs = _scales(x_scale, t)
    ws = np.asarray(w_scale, dtype=np.float32).reshape(e_count, n)
    ref = np.full((t, n), np.nan)
    at = np.full((t, n), np.nan)
    covered = np.zeros(t, dtype=bool)
    for e in range(e_count):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        ref[lo:hi] = gemm_a8w8(xq[lo:hi], xf, wq_experts[e], wf, xs[lo:hi], ws[e])
        at[lo:hi] = abs_terms(xq[lo:hi], xf, wq_experts[e], wf, xs[lo:hi], ws[e])
        covered[lo:hi] = True
    return ref, at, covered


# ---------------------------------------------------------------------------
# epilogue variants (AstrAI ops.cu: linear_forward_fp8 adds a bias in the GEMM
# epilogue, bf16 as is or FP8 codes times bias_scale; mm_fp8 can emit FP8
# E4M3 output, which requires out_scale, "the output quantization step")
# ---------------------------------------------------------------------------
BIAS_BF16 = 0
BIAS_E4M3 = 1
BIAS_E5M2 = 2


def bias_values(bias, kind: int, bias_scale=None) -> np.ndarray:
    """The bias as float64: bf16 bit patterns widened exactly, or FP8 codes
    decoded and multiplied by the float32 bias_scale in float32."""
    if kind == BIAS_BF16:
        if bias_scale is not None:
            raise ValueError("a bf16 bias takes no bias_scale")
        return bf16_bits_to_f64(bias)
    fmt = {BIAS_E4M3: fp8.E4M3, BIAS_E5M2: fp8.E5M2}[kind]
    dec = fp8.decode(np.asarray(bias, dtype=np.uint8), fmt).astype(np.float32)
    return (dec * np.float32(np.asarray(bias_scale, dtype=np.float32).reshape(-1)[0])).astype(np.float32).astype(
        np.float64)


def epilogue_f32(acc, x_scale, w_scale, bias_f32=None, out_scale=None, out_fmt=None):
    """The epilogue's float32 arithmetic on float32 accumulators acc [P]
    (one per output element, with its row's x_scale and column's w_scale and
    bias): v = fl32(fl32(acc * x_s) * w_s); with a bias v = fl32(v + b); then
    the bf16 output (round to nearest even) or, with out_scale, the FP8 code
    of fl32(v * fl32(1 / out_scale)) (the output quantization, read as the
    input quantization reads its scale: a reciprocal once, then a multiply).
    Returns uint16 bf16 bits or uint8 codes."""
    v = (np.asarray(acc, dtype=np.float32) * np.asarray(x_scale, dtype=np.float32)).astype(np.float32)
    v = (v * np.asarray(w_scale, dtype=np.float32)).astype(np.float32)
    if bias_f32 is not None:
        v = (v + np.asarray(bias_f32, dtype=np.float32)).astype(np.float32)
    if out_scale is None:
        import torch
        return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    r = (np.float32(1.0) / np.float32(np.asarray(out_scale, dtype=np.float32).reshape(-1)[0])).astype(np.float32)
    return fp8.encode((v * r).astype(np.float32), out_fmt)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) of a GEMM output to float64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
