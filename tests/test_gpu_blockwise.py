"""GPU parity of the block-wise path: hq_quantize_fp8_blockwise (codes, block
scales and block amax byte-exact with the oracle, deterministic and stochastic
E5M2) and hq_gemm_a8w8_blockscaled (within the block-scaled tolerance of the
float64 oracle).

Tolerance of the block-scaled GEMM (written here, from the arithmetic): each
block's partial sum is formed by FP8 MFMAs as in the plain GEMM, then folded
into the float32 sum with one FMA by the float32 product xs * ws. On top of the
plain GEMM bound (2 bf16 ulp + 2^-22 of the sum of |terms|) that adds one
rounding of the scale product and one of the FMA per block, each at most 2^-24
of the running sum of |terms| (oracle.blockwise.tolerance_blockscaled). Narrow
operands (every product a multiple of 2^-6 in [1, 4)) keep every partial exact
and are held to that bound alone; full-range operands add, per block, what the
FP8 matrix cores' run window drops (tests/mfma_model.py), scaled by that
block's scale product."""
import zlib

import numpy as np
import pytest
import torch

import workloads
from oracle import blockwise as B, fp8, gemm as G, quantize as Q
from tests.gpu_helpers import allowed_share, dev_bf16, dev_f32, dev_u8, host, narrow_codes, require_gpu
from tests.mfma_model import window_drop

pytestmark = pytest.mark.gpu

FORMATS = [fp8.E4M3, fp8.E5M2]


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _seed(*key):
    return zlib.crc32(repr(key).encode())


def _input(rng, shape, dtype, specials=False):
    std = float(10.0 ** rng.integers(-3, 3))
    if dtype == Q.BF16:
        x = workloads.random_bf16(rng, shape, std=std)
        return x, dev_bf16(x)
    x = workloads.random_f32(rng, shape, std=std)
    if specials:
        flat = x.reshape(-1)
        pos = rng.choice(flat.size, 5, replace=False)
        flat[pos] = [np.nan, np.inf, -np.inf, 0.0, 1e-40]
    return x, dev_f32(x)


def _check_quant(got, want):
    q, s, a = got
    q_ref, s_ref, a_ref = want
    assert host(s).shape == s_ref.shape
    bad = np.argwhere(host(q) != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0].tolist()}"
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))


# (rows, cols): one block, ragged last block for every block size, several row
# passes of the pipelined loop, more rows than resident wavefronts
QSHAPES = [(1, 16), (3, 144), (64, 128), (37, 4112), (5, 2064), (3500, 48)]


@pytest.mark.parametrize("shape", QSHAPES)
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("dtype", [Q.BF16, Q.F32])
def test_blockwise_quantize_byte_exact(hq, shape, bs, fmt, dtype):
    rng = np.random.default_rng(_seed(shape, bs, fmt, dtype))
    x, xd = _input(rng, shape, dtype, specials=dtype == Q.F32)
    got = hq.hq_quantize_fp8_blockwise(xd, fmt, bs)
    torch.cuda.synchronize()
    _check_quant(got, B.quantize_blockwise(x, dtype, fmt, bs))


@pytest.mark.parametrize("shape", [(3, 144), (37, 4112), (700, 272)])
@pytest.mark.parametrize("bs", [16, 128])
@pytest.mark.parametrize("dtype", [Q.BF16, Q.F32])
@pytest.mark.parametrize("seed", [0, 0xDEADBEEF12345678])
def test_blockwise_stochastic_byte_exact(hq, shape, bs, dtype, seed):
    rng = np.random.default_rng(_seed(shape, bs, dtype, seed, "sr"))
    x, xd = _input(rng, shape, dtype)
    got = hq.hq_quantize_fp8_blockwise(xd, fp8.E5M2, bs, stochastic=True, seed=seed)
    torch.cuda.synchronize()
    _check_quant(got, B.quantize_blockwise(x, dtype, fp8.E5M2, bs, stochastic=True, seed=seed))


def test_blockwise_outlier_block_isolated(hq):
    """A single large entry sets only its own block's scale: the other blocks
    of its row keep the fine scale of their own values."""
    x = np.full((4, 512), 0.01, dtype=np.float32)
    x[2, 300] = 1000.0
    got = hq.hq_quantize_fp8_blockwise(dev_f32(x), fp8.E4M3, 128)
    torch.cuda.synchronize()
    _check_quant(got, B.quantize_blockwise(x, Q.F32, fp8.E4M3, 128))
    s = host(got[1])
    assert s[2, 2] == np.float32(np.float32(1000.0) / np.float32(448.0))
    assert np.all(np.delete(s.reshape(-1), 2 * 4 + 2) == s[0, 0])


def test_blockwise_quantize_bench_size_sampled_rows(hq):
    """The benchmark's activation (bf16 [4096, 4096] with outliers, blocks of
    128): codes and scales of 64 sampled rows, whole, byte-exact."""
    xb, _ = workloads.ptpc_square()
    q, s, a = hq.hq_quantize_fp8_blockwise(dev_bf16(xb), fp8.E4M3, 128)
    torch.cuda.synchronize()
    rows = np.random.default_rng(11).choice(xb.shape[0], 64, replace=False)
    rows = np.concatenate([rows, [0, xb.shape[0] - 1]])
    q_ref, s_ref, a_ref = B.quantize_blockwise(xb[rows], Q.BF16, fp8.E4M3, 128)
    assert np.array_equal(host(q)[rows], q_ref)
    assert np.array_equal(host(s)[rows].view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(a)[rows].view(np.uint32), a_ref.view(np.uint32))


# ---------------------------------------------------------------------------
# block-scaled GEMM
# ---------------------------------------------------------------------------
def _block_scales(rng, rows, nb):
    return rng.uniform(1e-3, 2.0, (rows, nb)).astype(np.float32)


def _check_bs_gemm(out_bits, xq, xf, wq, wf, xs, ws, bs, pairs=None, strict_only=False, tag=""):
    m, k = xq.shape
    n = wq.shape[0]
    nb = B.block_count(k, bs)
    if pairs is None:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        pairs = np.stack([ii.reshape(-1), jj.reshape(-1)], axis=1)
    pairs = np.asarray(pairs, dtype=np.int64)
    got = G.bf16_bits_to_f64(np.asarray(out_bits)[pairs[:, 0], pairs[:, 1]])
    assert np.all(np.isfinite(got)), "non-finite GEMM output"
    xs64, ws64 = xs.astype(np.float64), ws.astype(np.float64)
    worst_strict, worst_bound, outside = 0.0, 0.0, 0
    for c0 in range(0, len(pairs), 2048):
        pc = pairs[c0:c0 + 2048]
        ref, at = B.gemm_blockscaled_rows(xq, xf, wq, wf, xs, ws, bs, pc)
        strict = B.tolerance_blockscaled(ref, at, nb)
        err = np.abs(got[c0:c0 + len(pc)] - ref)
        if strict_only:
            bad = np.nonzero(err > strict)[0]
            assert bad.size == 0, (f"{bad.size} outside the strict bound; first at {pc[bad[0]].tolist()}: "
                                   f"got {got[c0 + bad[0]]}, ref {ref[bad[0]]}, tol {strict[bad[0]]}")
        else:
            xa, wb = xq[pc[:, 0]], wq[pc[:, 1]]
            run = np.zeros(len(pc))
            for blk in range(nb):
                sl = slice(blk * bs, min(k, (blk + 1) * bs))
                run += window_drop(xa[:, sl], xf, wb[:, sl], wf) * np.abs(xs64[pc[:, 0], blk] * ws64[pc[:, 1], blk])
            bound = strict + run
            bad = np.nonzero(err > bound)[0]
            assert bad.size == 0, (f"{bad.size} outside strict + window bound; first at {pc[bad[0]].tolist()}: "
                                   f"got {got[c0 + bad[0]]}, ref {ref[bad[0]]}, bound {bound[bad[0]]}")
            worst_bound = max(worst_bound, float(np.max(err / bound)))
        outside += int((err > strict).sum())
        worst_strict = max(worst_strict, float(np.max(err / strict)))
    stats = {"n": len(pairs), "outside_strict": outside, "strict_share": outside / len(pairs),
             "max_err_over_strict": worst_strict, "max_err_over_bound": worst_bound}
    key = f"bs{tag} {bs} {tuple(xq.shape)}x{tuple(wq.shape)} {xf}{wf}"
    print(f"[gemm check] {key}: {stats}", flush=True)
    if not strict_only:
        allowed = allowed_share(key, len(pairs))
        assert outside <= allowed * len(pairs), f"{outside} of {len(pairs)} outside the strict bound"
    return stats


# (m, n, k): one tile and one K step; ragged M, N and K (partial last K step
# and partial last block); a single row; several K steps over many tiles
GSHAPES = [(128, 128, 128), (300, 520, 1040), (1, 96, 256), (130, 260, 272), (520, 384, 2048)]
PAIRS = [(fp8.E4M3, fp8.E4M3), (fp8.E4M3, fp8.E5M2), (fp8.E5M2, fp8.E4M3), (fp8.E5M2, fp8.E5M2)]


@pytest.mark.parametrize("shape", GSHAPES)
@pytest.mark.parametrize("bs", [32, 64, 128])
@pytest.mark.parametrize("formats", PAIRS)
def test_blockscaled_gemm_narrow_strict(hq, shape, bs, formats):
    m, n, k = shape
    xf, wf = formats
    rng = np.random.default_rng(_seed(shape, bs, formats, "narrow"))
    xq, wq = narrow_codes(rng, (m, k), xf), narrow_codes(rng, (n, k), wf)
    nb = B.block_count(k, bs)
    xs, ws = _block_scales(rng, m, nb), _block_scales(rng, n, nb)
    out = hq.hq_gemm_a8w8_blockscaled(dev_u8(xq), xf, dev_u8(wq), wf, dev_f32(xs), dev_f32(ws), bs)
    torch.cuda.synchronize()
    _check_bs_gemm(host(out), xq, xf, wq, wf, xs, ws, bs, strict_only=True)


@pytest.mark.parametrize("shape", [(300, 520, 1040), (64, 4000, 512)])
@pytest.mark.parametrize("bs", [32, 128])
@pytest.mark.parametrize("formats", [(fp8.E4M3, fp8.E4M3), (fp8.E5M2, fp8.E4M3)])
def test_blockscaled_gemm_full_range(hq, shape, bs, formats):
    m, n, k = shape
    xf, wf = formats
    rng = np.random.default_rng(_seed(shape, bs, formats, "full"))
    finite = [np.array([c for c in range(256) if np.isfinite(fp8.decode_table(f)[c])], np.uint8) for f in formats]
    xq, wq = rng.choice(finite[0], (m, k)), rng.choice(finite[1], (n, k))
    nb = B.block_count(k, bs)
    xs = (_block_scales(rng, m, nb) * 1e-3).astype(np.float32)
    ws = (_block_scales(rng, n, nb) * 1e-3).astype(np.float32)
    out = hq.hq_gemm_a8w8_blockscaled(dev_u8(xq), xf, dev_u8(wq), wf, dev_f32(xs), dev_f32(ws), bs)
    torch.cuda.synchronize()
    pairs = np.stack([rng.integers(0, m, 6000), rng.integers(0, n, 6000)], axis=1)
    _check_bs_gemm(host(out), xq, xf, wq, wf, xs, ws, bs, pairs=pairs)


def test_blockscaled_gemm_exact_small_case(hq):
    """Exact block partials and power-of-two scales in a narrow range: every
    partial, product and sum is exact in float32, so the output is the bf16
    rounding of the oracle's value, bit for bit."""
    rng = np.random.default_rng(3)
    m, n, k, bs = 40, 72, 96, 32
    xq, wq = narrow_codes(rng, (m, k), fp8.E4M3), narrow_codes(rng, (n, k), fp8.E4M3)
    nb = B.block_count(k, bs)
    xs = np.ldexp(1.0, rng.integers(-2, 2, (m, nb))).astype(np.float32)
    ws = np.ldexp(1.0, rng.integers(-2, 2, (n, nb))).astype(np.float32)
    out = hq.hq_gemm_a8w8_blockscaled(dev_u8(xq), fp8.E4M3, dev_u8(wq), fp8.E4M3, dev_f32(xs), dev_f32(ws), bs)
    torch.cuda.synchronize()
    ref = B.gemm_blockscaled(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bs)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)  # exact in float32
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(host(out), want)


def test_blockscaled_pipeline_bench_size(hq):
    """The benchmark's pass at full size: X bf16 [4096, 4096] with outliers and
    W bf16 [4096, 4096], both quantized in blocks of 128 along K (E4M3), then the
    block-scaled GEMM. Codes and scales of sampled rows byte-exact; the GEMM
    within tolerance on 4096 sampled outputs (taken on the GPU's own codes, which
    the row checks have tied to the oracle's)."""
    xb, wb = workloads.ptpc_square()
    xq, xs, _ = hq.hq_quantize_fp8_blockwise(dev_bf16(xb), fp8.E4M3, 128)
    wq, ws, _ = hq.hq_quantize_fp8_blockwise(dev_bf16(wb), fp8.E4M3, 128)
    out = hq.hq_gemm_a8w8_blockscaled(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, 128)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    xq_h, xs_h, wq_h, ws_h = host(xq), host(xs), host(wq), host(ws)
    for src, codes, sc in ((xb, xq_h, xs_h), (wb, wq_h, ws_h)):
        rows = rng.choice(src.shape[0], 24, replace=False)
        q_ref, s_ref, _ = B.quantize_blockwise(src[rows], Q.BF16, fp8.E4M3, 128)
        assert np.array_equal(codes[rows], q_ref)
        assert np.array_equal(sc[rows].view(np.uint32), s_ref.view(np.uint32))
    pairs = np.stack([rng.integers(0, 4096, 4096), rng.integers(0, 4096, 4096)], axis=1)
    pairs[:4] = [[0, 0], [4095, 4095], [0, 4095], [4095, 0]]
    _check_bs_gemm(host(out), xq_h, fp8.E4M3, wq_h, fp8.E4M3, xs_h, ws_h, 128, pairs=pairs)


def test_blockscaled_equals_plain_gemm_for_uniform_scales(hq):
    """With every block scale of a row equal (the per-token / per-channel case)
    the block-scaled GEMM and the plain a8w8 GEMM both stay within the plain
    GEMM's bound of the same float64 reference."""
    rng = np.random.default_rng(8)
    m, n, k, bs = 200, 264, 512, 64
    xq, wq = narrow_codes(rng, (m, k), fp8.E4M3), narrow_codes(rng, (n, k), fp8.E5M2)
    xr = rng.uniform(0.01, 1.0, m).astype(np.float32)
    wr = rng.uniform(0.01, 1.0, n).astype(np.float32)
    nb = B.block_count(k, bs)
    xs, ws = np.repeat(xr[:, None], nb, axis=1), np.repeat(wr[:, None], nb, axis=1)
    out = hq.hq_gemm_a8w8_blockscaled(dev_u8(xq), fp8.E4M3, dev_u8(wq), fp8.E5M2, dev_f32(xs), dev_f32(ws), bs)
    plain = hq.hq_gemm_a8w8(dev_u8(xq), fp8.E4M3, hq.hq_preshuffle_weight(dev_u8(wq)), fp8.E5M2, dev_f32(xr),
                            dev_f32(wr), n)
    torch.cuda.synchronize()
    ref = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E5M2, xr, wr)
    at = G.abs_terms(xq, fp8.E4M3, wq, fp8.E5M2, xr, wr)
    tol = B.tolerance_blockscaled(ref, at, nb)
    for o in (out, plain):
        assert np.all(np.abs(G.bf16_bits_to_f64(host(o)) - ref) <= tol)


def _bf16_bias(rng, n, scale):
    return workloads.to_bf16_bits((rng.standard_normal(n) * scale).astype(np.float32))


@pytest.mark.parametrize("shape", [(130, 260, 272), (300, 520, 1040)])
@pytest.mark.parametrize("bs", [32, 128])
def test_blockscaled_gemm_bias_narrow_strict(hq, shape, bs):
    """Reading B4: the bf16 bias added to the block sum before the output
    rounding; ragged N covers the bias of the last, partial column tile."""
    m, n, k = shape
    rng = np.random.default_rng(_seed(shape, bs, "bias"))
    xq, wq = narrow_codes(rng, (m, k), fp8.E4M3), narrow_codes(rng, (n, k), fp8.E5M2)
    nb = B.block_count(k, bs)
    xs, ws = _block_scales(rng, m, nb), _block_scales(rng, n, nb)
    bias = _bf16_bias(rng, n, 50.0)
    out = hq.hq_gemm_a8w8_blockscaled(dev_u8(xq), fp8.E4M3, dev_u8(wq), fp8.E5M2, dev_f32(xs), dev_f32(ws), bs,
                                      bias=dev_bf16(bias))
    torch.cuda.synchronize()
    ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    pairs = np.stack([ii.reshape(-1), jj.reshape(-1)], axis=1)
    got = G.bf16_bits_to_f64(host(out)[pairs[:, 0], pairs[:, 1]])
    ref, at = B.gemm_blockscaled_rows(xq, fp8.E4M3, wq, fp8.E5M2, xs, ws, bs, pairs, bias=bias)
    bad = np.nonzero(np.abs(got - ref) > B.tolerance_blockscaled(ref, at, nb))[0]
    assert bad.size == 0, f"{bad.size} outside; first at {pairs[bad[0]].tolist()}: got {got[bad[0]]}, ref {ref[bad[0]]}"


def test_blockscaled_gemm_bias_exact(hq):
    """Exact partials, power-of-two scales and integer biases: every sum is exact
    in float32, so the output is the bf16 rounding of the oracle value, bit for
    bit."""
    rng = np.random.default_rng(41)
    m, n, k, bs = 48, 100, 128, 64
    xq, wq = narrow_codes(rng, (m, k), fp8.E4M3), narrow_codes(rng, (n, k), fp8.E4M3)
    xs = np.ldexp(1.0, rng.integers(-2, 2, (m, 2))).astype(np.float32)
    ws = np.ldexp(1.0, rng.integers(-2, 2, (n, 2))).astype(np.float32)
    bias = workloads.to_bf16_bits(rng.integers(-64, 65, n).astype(np.float32))
    out = hq.hq_gemm_a8w8_blockscaled(dev_u8(xq), fp8.E4M3, dev_u8(wq), fp8.E4M3, dev_f32(xs), dev_f32(ws), bs,
                                      bias=dev_bf16(bias))
    torch.cuda.synchronize()
    ref = B.gemm_blockscaled(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bs, bias=bias)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(host(out), want)


# ---------------------------------------------------------------------------
# block-scaled GEMM over the pre-shuffled weight (blocks of 128)
# ---------------------------------------------------------------------------
def _bs_pre(hq, xq, xf, wq, wf, xs, ws, bs=128, bias=None):
    n = wq.shape[0]
    pre = hq.hq_preshuffle_weight(dev_u8(wq))
    return hq.hq_gemm_a8w8_blockscaled_preshuffled(dev_u8(xq), xf, pre, wf, dev_f32(xs), dev_f32(ws), n, bs,
                                                   bias=None if bias is None else dev_bf16(bias))


# (m, n, k): one tile; ragged M, N and K (a partial last block); a single row
# (the 64 x 128 tile); the 128 x 128 and 256 x 128 tiles over several K blocks
PSHAPES = [(128, 128, 128), (300, 520, 1040), (1, 96, 256), (130, 260, 272), (520, 384, 2048), (1100, 700, 640)]


@pytest.mark.parametrize("shape", PSHAPES)
@pytest.mark.parametrize("bs", [32, 64, 128])
@pytest.mark.parametrize("formats", PAIRS)
def test_blockscaled_preshuffled_narrow_strict(hq, shape, bs, formats):
    m, n, k = shape
    xf, wf = formats
    rng = np.random.default_rng(_seed(shape, bs, formats, "pre-narrow"))
    xq, wq = narrow_codes(rng, (m, k), xf), narrow_codes(rng, (n, k), wf)
    nb = B.block_count(k, bs)
    xs, ws = _block_scales(rng, m, nb), _block_scales(rng, n, nb)
    out = _bs_pre(hq, xq, xf, wq, wf, xs, ws, bs)
    torch.cuda.synchronize()
    pairs = None
    if m * n > 300 * 600:  # sampled, tile edges included
        pairs = np.stack([rng.integers(0, m, 8192), rng.integers(0, n, 8192)], axis=1)
        pairs[:16] = [[r, c] for r in (0, 63, 64, m - 1) for c in (0, 127, 128, n - 1)]
    _check_bs_gemm(host(out), xq, xf, wq, wf, xs, ws, bs, pairs=pairs, strict_only=True)


@pytest.mark.parametrize("shape", [(300, 520, 1040), (64, 4000, 512), (1030, 1030, 1152)])
@pytest.mark.parametrize("bs", [32, 64, 128])
def test_blockscaled_preshuffled_full_range(hq, shape, bs):
    m, n, k = shape
    rng = np.random.default_rng(_seed(shape, bs, "pre-full"))
    finite = np.array([c for c in range(256) if np.isfinite(fp8.decode_table(fp8.E4M3)[c])], np.uint8)
    xq, wq = rng.choice(finite, (m, k)), rng.choice(finite, (n, k))
    nb = B.block_count(k, bs)
    xs = (_block_scales(rng, m, nb) * 1e-3).astype(np.float32)
    ws = (_block_scales(rng, n, nb) * 1e-3).astype(np.float32)
    out = _bs_pre(hq, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bs)
    torch.cuda.synchronize()
    pairs = np.stack([rng.integers(0, m, 6000), rng.integers(0, n, 6000)], axis=1)
    _check_bs_gemm(host(out), xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bs, pairs=pairs, tag="pre")


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_blockscaled_preshuffled_exact_with_bias(hq, bs):
    """Exact block partials, power-of-two scales and integer biases: every sum
    is exact in float32, so the output is the bf16 rounding of the oracle's
    value, bit for bit (for blocks of 32 and 64 this also shows that the chunks
    scaled out of each block's MFMA contribute exactly nothing)."""
    rng = np.random.default_rng(43 + bs)
    m, n, k = 200, 136, 400
    xq, wq = narrow_codes(rng, (m, k), fp8.E4M3), narrow_codes(rng, (n, k), fp8.E5M2)
    nb = B.block_count(k, bs)
    xs = np.ldexp(1.0, rng.integers(-2, 2, (m, nb))).astype(np.float32)
    ws = np.ldexp(1.0, rng.integers(-2, 2, (n, nb))).astype(np.float32)
    bias = workloads.to_bf16_bits(rng.integers(-64, 65, n).astype(np.float32))
    out = _bs_pre(hq, xq, fp8.E4M3, wq, fp8.E5M2, xs, ws, bs, bias=bias)
    torch.cuda.synchronize()
    ref = B.gemm_blockscaled(xq, fp8.E4M3, wq, fp8.E5M2, xs, ws, bs, bias=bias)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(host(out), want)


def test_blockscaled_preshuffled_bench_size(hq):
    """The benchmark's 4096^3 block-scaled pass (blocks of 128, the PTPC
    operands) through the pre-shuffled weight: 4096 sampled outputs against the
    oracle; and, as the same arithmetic in the same order, the same bits as the
    row-major entry point."""
    xb, wb = workloads.ptpc_square()
    xq, xs, _ = hq.hq_quantize_fp8_blockwise(dev_bf16(xb), fp8.E4M3, 128)
    wq, ws, _ = hq.hq_quantize_fp8_blockwise(dev_bf16(wb), fp8.E4M3, 128)
    pre = hq.hq_preshuffle_weight(wq)
    out = hq.hq_gemm_a8w8_blockscaled_preshuffled(xq, fp8.E4M3, pre, fp8.E4M3, xs, ws, 4096)
    row_major = hq.hq_gemm_a8w8_blockscaled(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, 128)
    torch.cuda.synchronize()
    rng = np.random.default_rng(14)
    pairs = np.stack([rng.integers(0, 4096, 4096), rng.integers(0, 4096, 4096)], axis=1)
    pairs[:4] = [[0, 0], [4095, 4095], [0, 4095], [4095, 0]]
    _check_bs_gemm(host(out), host(xq), fp8.E4M3, host(wq), fp8.E4M3, host(xs), host(ws), 128, pairs=pairs,
                   tag="pre")
    assert torch.equal(out.view(torch.int16), row_major.view(torch.int16))


@pytest.mark.parametrize("shape", [(4096, 1024, 384), (2560, 2560, 272)])
@pytest.mark.parametrize("bs", [32, 64, 128])
def test_blockscaled_preshuffled_large_tiles_sampled(hq, shape, bs):
    """Shapes whose launch takes the 128 x 128 tile (4096 x 1024) and the
    256 x 128 tile (2560 x 2560, with a partial last block): narrow codes, 8192
    sampled outputs within the strict bound, tile edges included."""
    m, n, k = shape
    rng = np.random.default_rng(_seed(shape, bs, "pre-large"))
    xq, wq = narrow_codes(rng, (m, k), fp8.E4M3), narrow_codes(rng, (n, k), fp8.E4M3)
    nb = B.block_count(k, bs)
    xs, ws = _block_scales(rng, m, nb), _block_scales(rng, n, nb)
    out = _bs_pre(hq, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bs)
    torch.cuda.synchronize()
    pairs = np.stack([rng.integers(0, m, 8192), rng.integers(0, n, 8192)], axis=1)
    edges = np.array([[r, c] for r in (0, 127, 128, 255, 256, m - 1) for c in (0, 127, 128, n - 1)])
    pairs[:len(edges)] = edges
    _check_bs_gemm(host(out), xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bs, pairs=pairs, strict_only=True)
