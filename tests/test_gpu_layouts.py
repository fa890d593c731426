"""GPU parity of hq_quantize_fp8_layouts: per-tensor codes written row-major,
transposed and pre-shuffled (of either) in one pass, with a given, a delayed
(ring) or a dynamic scale. Every layout must equal, byte for byte, the oracle's
codes moved by a plain transpose and the oracle's pre-shuffle index map."""
import numpy as np
import pytest
import torch

import workloads
from oracle import fp8, gemm as G, preshuffle as P, quantize as Q
from tests.gpu_helpers import allowed_share, check_gemm, dev_bf16, dev_f32, host, require_gpu

pytestmark = pytest.mark.gpu

ALL = dict(q=True, q_t=True, q_pre=True, q_t_pre=True)


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _check_layouts(out, q_ref):
    if "q" in out:
        assert np.array_equal(host(out["q"]), q_ref)
    if "q_t" in out:
        assert np.array_equal(host(out["q_t"]), np.ascontiguousarray(q_ref.T))
    if "q_pre" in out:
        assert np.array_equal(host(out["q_pre"]), P.preshuffle(q_ref))
    if "q_t_pre" in out:
        assert np.array_equal(host(out["q_t_pre"]), P.preshuffle(np.ascontiguousarray(q_ref.T)))


def _input(rng, shape, dtype, specials=False):
    if dtype == Q.BF16:
        x = workloads.random_bf16(rng, shape, std=float(10.0 ** rng.integers(-2, 3)))
        dev = dev_bf16(x)
    else:
        x = (rng.standard_normal(shape) * 10.0 ** rng.integers(-2, 3)).astype(np.float32)
        if specials:
            flat = x.reshape(-1)
            flat[rng.choice(flat.size, 3, replace=False)] = [np.nan, np.inf, -np.inf]
        dev = dev_f32(x)
    return x, dev


# (rows, cols): one tile, ragged tiles and N padding, several tiles, rows % 16 != 0
SHAPES = [(16, 16), (64, 128), (48, 160), (144, 4112), (256, 384), (1040, 272)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
@pytest.mark.parametrize("dtype", [Q.BF16, Q.F32])
def test_given_scale_all_layouts(hq, shape, fmt, dtype):
    rng = np.random.default_rng(shape[0] * 7 + shape[1] + fmt * 3 + dtype)
    x, xd = _input(rng, shape, dtype)
    # a scale that saturates the largest values, as a stale forward scale may
    s = np.float32(np.abs(Q.widen(x, dtype)).max() / fp8.fmax(fmt) / 2.0)
    out = hq.hq_quantize_fp8_layouts(xd, fmt, scale_in=dev_f32(np.array([s])), **ALL)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = Q.quantize_with_scale(x, dtype, fmt, s)
    _check_layouts(out, q_ref)
    assert host(out["scale"]).view(np.uint32)[0] == s_ref.view(np.uint32)[0]
    assert out["amax"] is None


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_dynamic_all_layouts(hq, shape, fmt):
    rng = np.random.default_rng(shape[0] + 3 * shape[1] + fmt)
    x, xd = _input(rng, shape, Q.BF16)
    out = hq.hq_quantize_fp8_layouts(xd, fmt, **ALL)
    torch.cuda.synchronize()
    q_ref, s_ref, a_ref = Q.quantize_dynamic(x, Q.BF16, fmt, Q.PER_TENSOR)
    _check_layouts(out, q_ref)
    assert host(out["scale"]).view(np.uint32)[0] == s_ref.view(np.uint32)[0]
    assert host(out["amax"]).view(np.uint32)[0] == a_ref.view(np.uint32)[0]


def test_rows_not_multiple_of_16_row_major_layouts_only(hq):
    rng = np.random.default_rng(3)
    x, xd = _input(rng, (300, 272), Q.F32)
    out = hq.hq_quantize_fp8_layouts(xd, fp8.E4M3, q=True, q_pre=True)
    torch.cuda.synchronize()
    q_ref, _, _ = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, Q.PER_TENSOR)
    _check_layouts(out, q_ref)


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_special_values_given_scale(hq, fmt):
    rng = np.random.default_rng(9)
    x, xd = _input(rng, (64, 96), Q.F32, specials=True)
    s = np.float32(0.01)
    out = hq.hq_quantize_fp8_layouts(xd, fmt, scale_in=dev_f32(np.array([s])), **ALL)
    torch.cuda.synchronize()
    q_ref, _, _ = Q.quantize_with_scale(x, Q.F32, fmt, s)
    _check_layouts(out, q_ref)


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_ring_sequence_matches_hq_quantize_and_oracle(hq, fmt):
    """Six delayed steps (ring of 4, margin 1), one with a NaN: the layouts
    call and the oracle agree on codes, ring state and the sticky flag."""
    rng = np.random.default_rng(21 + fmt)
    ring = hq.Ring(4, margin=1)
    st, flag = Q.ring_new(4), 0
    for t in range(6):
        x = (rng.standard_normal((128, 256)) * np.exp(rng.standard_normal())).astype(np.float32)
        if t == 3:
            x[5, 7] = np.nan
        out = hq.hq_quantize_fp8_layouts(dev_f32(x), fmt, ring=ring, ring_idx=t % 4, **ALL)
        torch.cuda.synchronize()
        q_ref, s_ref, a_ref, st, flag = Q.quantize_delayed(x, Q.F32, fmt, st, t % 4, 1, flag)
        _check_layouts(out, q_ref)
        assert host(out["scale"]).view(np.uint32)[0] == s_ref.view(np.uint32)[0]
        assert np.array_equal(host(ring.state).view(np.uint32), st.view(np.uint32)), t
        assert int(host(ring.flag)[0]) == flag


def test_training_backward_operands_fused(hq):
    """One backward step of a training-linear layer with every GEMM operand
    produced by the fused pass: G (E5M2, ring) row-major for dgrad and
    transposed for wgrad; W and X (E5M2, their forward scales) straight into
    the pre-shuffled transposed layouts the GEMMs take. Codes and scales
    byte-exact; both GEMMs within tolerance of the oracle on sampled outputs."""
    base, factors = workloads.training_linear(4, layers=1, steps=1)
    xb, wb, gb = workloads.training_step_inputs(base, factors, 0, 0)
    m, k = xb.shape
    n = wb.shape[0]
    # forward scales (dynamic per tensor, E4M3) as the forward pass would have made them
    _, sx, _ = Q.quantize_dynamic(xb, Q.BF16, fp8.E4M3, Q.PER_TENSOR)
    _, sw, _ = Q.quantize_dynamic(wb, Q.BF16, fp8.E4M3, Q.PER_TENSOR)
    ring = hq.Ring(16)
    g_out = hq.hq_quantize_fp8_layouts(dev_bf16(gb), fp8.E5M2, ring=ring, ring_idx=0, q=True, q_t=True)
    w_out = hq.hq_quantize_fp8_layouts(dev_bf16(wb), fp8.E5M2, scale_in=dev_f32(sw), q_t_pre=True)
    x_out = hq.hq_quantize_fp8_layouts(dev_bf16(xb), fp8.E5M2, scale_in=dev_f32(sx), q_t_pre=True)
    dx = hq.hq_gemm_a8w8(g_out["q"], fp8.E5M2, w_out["q_t_pre"], fp8.E5M2, g_out["scale"], w_out["scale"], k)
    dw = hq.hq_gemm_a8w8(g_out["q_t"], fp8.E5M2, x_out["q_t_pre"], fp8.E5M2, g_out["scale"], x_out["scale"], k)
    torch.cuda.synchronize()
    gq, gs, _, _, _ = Q.quantize_delayed(gb, Q.BF16, fp8.E5M2, Q.ring_new(16), 0, 0, 0)
    wq, _, _ = Q.quantize_with_scale(wb, Q.BF16, fp8.E5M2, sw)
    xq, _, _ = Q.quantize_with_scale(xb, Q.BF16, fp8.E5M2, sx)
    _check_layouts(g_out, gq)
    _check_layouts(w_out, wq)
    _check_layouts(x_out, xq)
    rng = np.random.default_rng(4)
    wt, xt, gt = (np.ascontiguousarray(a.T) for a in (wq, xq, gq))
    pairs = np.stack([rng.integers(0, m, 4000), rng.integers(0, k, 4000)], axis=1)
    check_gemm(host(dx), gq, fp8.E5M2, wt, fp8.E5M2, gs, sw, pairs=pairs,
               max_strict_frac=allowed_share("layouts dgrad", len(pairs)), label="layouts dgrad")
    pairs = np.stack([rng.integers(0, n, 4000), rng.integers(0, k, 4000)], axis=1)
    check_gemm(host(dw), gt, fp8.E5M2, xt, fp8.E5M2, gs, sx, pairs=pairs,
               max_strict_frac=allowed_share("layouts wgrad", len(pairs)), label="layouts wgrad")


# ---- stochastic rounding (E5M2) -----------------------------------------------------

from oracle import stochastic as S  # noqa: E402


@pytest.mark.parametrize("shape", [(64, 128), (144, 4112), (1040, 272)])
@pytest.mark.parametrize("dtype", [Q.BF16, Q.F32])
def test_stochastic_dynamic_all_layouts(hq, shape, dtype):
    """Dynamic scale: every layout carries the oracle's stochastic codes (drawn
    from the row-major index of x), equal to hq_quantize_fp8_stochastic's
    per-tensor codes for the same seed."""
    rng = np.random.default_rng(shape[0] + shape[1] + dtype + 1000)
    x, xd = _input(rng, shape, dtype)
    seed = 0xC0FFEE + shape[0]
    out = hq.hq_quantize_fp8_layouts_stochastic(xd, seed, **ALL)
    q2, s2, _ = hq.hq_quantize_fp8_stochastic(xd, Q.PER_TENSOR, seed)
    torch.cuda.synchronize()
    q_ref, s_ref, a_ref = S.quantize_stochastic(x, dtype, Q.PER_TENSOR, seed)
    _check_layouts(out, q_ref)
    assert np.array_equal(host(q2), q_ref)
    assert host(out["scale"]).view(np.uint32)[0] == s_ref.view(np.uint32)[0]
    assert host(out["amax"]).view(np.uint32)[0] == a_ref.view(np.uint32)[0]


@pytest.mark.parametrize("shape", [(16, 16), (256, 384)])
def test_stochastic_given_scale_all_layouts(hq, shape):
    rng = np.random.default_rng(shape[0] * 3 + shape[1])
    x, xd = _input(rng, shape, Q.BF16)
    s = np.float32(np.abs(Q.widen(x, Q.BF16)).max() / fp8.fmax(fp8.E5M2) / 3.0)
    out = hq.hq_quantize_fp8_layouts_stochastic(xd, 2 ** 63 + 11, scale_in=dev_f32(np.array([s])), **ALL)
    torch.cuda.synchronize()
    q_ref, s_ref = S.quantize_with_scale_stochastic(x, Q.BF16, s, 2 ** 63 + 11)
    _check_layouts(out, q_ref)
    assert host(out["scale"]).view(np.uint32)[0] == s_ref.view(np.uint32)[0]


def test_stochastic_ring_sequence(hq):
    """Delayed (ring) steps, one with a NaN: codes in every layout, the scale
    used and the ring state match the oracle after each step."""
    rng = np.random.default_rng(77)
    ring = hq.Ring(4, margin=1)
    st, flag = Q.ring_new(4), 0
    for t in range(5):
        x = (rng.standard_normal((128, 256)) * np.exp(rng.standard_normal())).astype(np.float32)
        if t == 2:
            x[3, 9] = np.nan
        out = hq.hq_quantize_fp8_layouts_stochastic(dev_f32(x), 1234 + t, ring=ring, ring_idx=t % 4, **ALL)
        torch.cuda.synchronize()
        q_ref, s_ref, a_ref, st, flag = S.quantize_delayed_stochastic(x, Q.F32, st, t % 4, 1, 1234 + t, flag)
        _check_layouts(out, q_ref)
        assert host(out["scale"]).view(np.uint32)[0] == s_ref.view(np.uint32)[0]
        assert np.array_equal(host(ring.state).view(np.uint32), st.view(np.uint32)), t
        assert int(host(ring.flag)[0]) == flag
