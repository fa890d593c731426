"""Helpers for the GPU parity tests (not collected: no test_ prefix).

Tolerance for GEMM outputs (written here, used by every GEMM test):

  strict(m, n) = 2 * ulp_bf16(ref) + 2^-22 * sum_k |x_s w_s dec(XQ) dec(WQ)|
      the bound the method statement gives for the GEMM.

  run_term(m, n) = |x_s w_s| * sum over runs g of 8 consecutive k of
                   sum_{k in g} min(|t_k|, q_g) * [t_k is not a multiple of q_g],
                   q_g = 2^(floor(log2 max_{k in g} |t_k|) - 13)
      the gfx950 FP8 MFMA adds each run of 8 consecutive-k products in a fixed-
      point window whose last kept bit is 2^-13 of the run's largest product
      (measured on the device: a product 2^-14 below the run maximum is dropped,
      one 2^-13 below is kept; runs 8 apart are independent; adding to the fp32
      accumulator is exact to fp32). The term bounds what that window can drop.

A GEMM test asserts |out - ref| <= strict + run_term on every element, and that
the share of elements outside `strict` alone stays below a small fraction. On
operands whose products all lie within 2^5 of each other the window drops
nothing, and those tests assert `strict` alone on every element.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import fp8, gemm as G


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X; none is visible"
    import fp8_dynamic_quantization_amd as hq
    hq.load()  # raises if libhq.so is missing: no fallback path exists
    return hq


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run_term_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """MFMA run term (unscaled) for decoded operand rows a [P, K] and b [P, K]
    (one output element per row pair)."""
    t = np.abs(a * b)
    p, k = t.shape
    kp = -(-k // 8) * 8
    if kp != k:
        t = np.concatenate([t, np.zeros((p, kp - k))], axis=1)
    runs = t.reshape(p, kp // 8, 8)
    mx = runs.max(axis=2, keepdims=True)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
    q = np.ldexp(1.0, (e - 13).astype(np.int64))
    frac = np.mod(runs, q)
    lost = np.where(frac != 0, np.minimum(runs, q), 0.0)
    lost = np.where(mx > 0, lost, 0.0)
    return lost.sum(axis=(1, 2))


def _scale_vec(s, count):
    s = np.asarray(s, dtype=np.float32).reshape(-1).astype(np.float64)
    return np.full(count, s[0]) if s.size == 1 else s


def check_gemm(out_bits, xq, xf, wq, wf, xs, ws, pairs=None, strict_only=False, max_strict_frac=0.01):
    """Compare a GPU bf16 output with the oracle. ``pairs`` (P x 2) samples
    positions; None checks every element. Returns a stats dict."""
    xq = np.asarray(xq, np.uint8)
    wq = np.asarray(wq, np.uint8)
    m, n = xq.shape[0], wq.shape[0]
    xsv, wsv = _scale_vec(xs, m), _scale_vec(ws, n)
    if pairs is None:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        pairs = np.stack([ii.reshape(-1), jj.reshape(-1)], axis=1)
    pairs = np.asarray(pairs, dtype=np.int64)
    got = G.bf16_bits_to_f64(np.asarray(out_bits)[pairs[:, 0], pairs[:, 1]])
    ref_all, at_all, run_all = [], [], []
    ta, tb = fp8.decode_table(xf), fp8.decode_table(wf)
    for c0 in range(0, len(pairs), 4096):
        pc = pairs[c0:c0 + 4096]
        ref, at = G.gemm_a8w8_rows(xq, xf, wq, wf, xsv, wsv, pc)
        ref_all.append(ref)
        at_all.append(at)
        if not strict_only:
            a = ta[xq[pc[:, 0]]]
            b = tb[wq[pc[:, 1]]]
            run_all.append(run_term_rows(a, b) * np.abs(xsv[pc[:, 0]] * wsv[pc[:, 1]]))
    ref = np.concatenate(ref_all)
    at = np.concatenate(at_all)
    strict = G.tolerance(ref, at)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), "non-finite GEMM output"
    outside = err > strict
    stats = {"n": len(ref), "strict_violations": int(outside.sum()),
             "max_err_over_strict": float(np.max(err / strict))}
    if strict_only:
        bad = np.nonzero(outside)[0]
        assert bad.size == 0, (f"{bad.size} elements outside the strict bound; first at "
                               f"{pairs[bad[0]].tolist()}: got {got[bad[0]]}, ref {ref[bad[0]]}, "
                               f"tol {strict[bad[0]]}")
        return stats
    run = np.concatenate(run_all)
    bound = strict + run
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{bad.size} elements outside strict + MFMA-run bound; first at "
                           f"{pairs[bad[0]].tolist()}: got {got[bad[0]]}, ref {ref[bad[0]]}, "
                           f"bound {bound[bad[0]]}")
    assert outside.mean() <= max_strict_frac, f"{outside.mean():.4%} of elements outside the strict bound"
    stats["max_err_over_bound"] = float(np.max(err / bound))
    return stats


def narrow_codes(rng, shape, fmt, zero_frac=0.1):
    """Codes with |value| in [1, 2) (and some zeros), both signs: every product of
    two such values is a multiple of 2^-6 in [1, 4), so MFMA runs are exact."""
    lo = 0x38 if fmt == fp8.E4M3 else 0x3C
    hi = 0x3F
    c = rng.integers(lo, hi + 1, size=shape).astype(np.uint8)
    c |= (rng.random(shape) < 0.5).astype(np.uint8) << 7
    c[rng.random(shape) < zero_frac] = 0
    return c
