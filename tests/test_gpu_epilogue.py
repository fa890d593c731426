"""GPU parity of hq_gemm_a8w8_epilogue and hq_grouped_gemm_a8w8_epilogue: the bias (bf16, or FP8 codes times a
bias scale) and the FP8 output (codes of v * 1/out_scale) of the GEMM epilogue.

With operands whose products are multiples of 2^-6 in [1, 4) (narrow codes)
the float32 accumulator is exact, so the kernel's epilogue chain and the
oracle's (epilogue_f32 on the exact accumulator) must agree bit for bit, for
every output element, bf16 or FP8. Full-range operands are checked against the
float64 reference within the GEMM tolerance (bf16 output) or within half an FP8
step plus that tolerance (FP8 output)."""
import zlib

import numpy as np
import pytest
import torch

from oracle import fp8, gemm as G
from tests.gpu_helpers import check_gemm, dev_f32, dev_u8, host, narrow_codes, require_gpu
from tests.mfma_model import window_drop

pytestmark = pytest.mark.gpu

BIASES = ["none", "bf16", "e4m3", "e5m2"]
OUTS = ["bf16", "e4m3", "e5m2"]
FMT = {"e4m3": fp8.E4M3, "e5m2": fp8.E5M2}
KIND = {"bf16": G.BIAS_BF16, "e4m3": G.BIAS_E4M3, "e5m2": G.BIAS_E5M2}


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _bias(rng, n, kind):
    """(device bias, device bias_scale or None, float64 bias values)."""
    if kind == "bf16":
        b = (rng.standard_normal(n) * 8).astype(np.float32)
        bits = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return torch.from_numpy(bits.view(np.int16)).cuda(), None, G.bias_values(bits, G.BIAS_BF16)
    table = fp8.decode_table(FMT[kind])
    finite = np.array([c for c in range(256) if np.isfinite(table[c])], dtype=np.uint8)
    codes = rng.choice(finite, n)
    bsc = np.float32(rng.uniform(0.01, 0.1))
    return dev_u8(codes), dev_f32(np.array([bsc])), G.bias_values(codes, KIND[kind], bsc)


def _run(hq, xq, xf, wq, wf, xs, ws, bias_kind, out_kind, rng, out_scale_val):
    m, n = xq.shape[0], wq.shape[0]
    pre = hq.hq_preshuffle_weight(dev_u8(wq))
    kw = {}
    bvals = None
    if bias_kind != "none":
        bd, bs, bvals = _bias(rng, n, bias_kind)
        kw.update(bias=bd, bias_type=KIND[bias_kind], bias_scale=bs)
    if out_kind != "bf16":
        kw.update(out_scale=dev_f32(np.array([out_scale_val])), out_fmt=FMT[out_kind])
    out = hq.hq_gemm_a8w8_epilogue(dev_u8(xq), xf, pre, wf, dev_f32(np.atleast_1d(xs)), dev_f32(np.atleast_1d(ws)),
                                   n, **kw)
    torch.cuda.synchronize()
    return host(out), bvals


# (m, n, k): decode path (M <= 64, ragged N), and the 64x128, 128x256 and
# 256x256 tile configurations
SHAPES = [(1, 96, 256), (33, 200, 400), (300, 520, 1040), (2000, 4000, 272), (3600, 3700, 400),
          (1000, 1088, 512)]  # 64 x 128 tiles with K split inside the workgroup


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bias_kind", BIASES)
@pytest.mark.parametrize("out_kind", OUTS)
def test_epilogue_bit_exact_on_exact_accumulators(hq, shape, bias_kind, out_kind):
    if bias_kind == "none" and out_kind == "bf16":
        pytest.skip("plain GEMM: covered by the GEMM tests")
    m, n, k = shape
    rng = np.random.default_rng(zlib.crc32(repr((shape, bias_kind, out_kind)).encode()))
    xq = narrow_codes(rng, (m, k), fp8.E4M3)
    wq = narrow_codes(rng, (n, k), fp8.E5M2)
    xs = rng.uniform(1e-3, 2.0, m).astype(np.float32)
    ws = rng.uniform(1e-3, 2.0, n).astype(np.float32)
    out_scale = np.float32(rng.uniform(0.5, 4.0))
    got, bvals = _run(hq, xq, fp8.E4M3, wq, fp8.E5M2, xs, ws, bias_kind, out_kind, rng, out_scale)
    # rows / columns to compare: all for small shapes, edges plus a random sample for large ones
    if m * n <= 300 * 520:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        ii, jj = ii.reshape(-1), jj.reshape(-1)
    else:
        ii = np.concatenate([rng.integers(0, m, 6000), np.array([0, m - 1, 255, 256] * 3)])
        jj = np.concatenate([rng.integers(0, n, 6000), np.array([0, n - 1, n - 8, 257] * 3)])
    if m * n <= 300 * 520:
        acc = (fp8.decode(xq, fp8.E4M3) @ fp8.decode(wq, fp8.E5M2).T)[ii, jj]  # exact: integers times 2^-5
    else:
        acc = (fp8.decode(xq[ii], fp8.E4M3) * fp8.decode(wq[jj], fp8.E5M2)).sum(axis=1)
    acc32 = acc.astype(np.float32)
    assert np.array_equal(acc32.astype(np.float64), acc)  # exact in float32
    want = G.epilogue_f32(acc32, xs[ii], ws[jj], None if bvals is None else bvals[jj].astype(np.float32),
                          None if out_kind == "bf16" else out_scale, FMT.get(out_kind))
    have = got[ii, jj]
    bad = np.nonzero(have != want)[0]
    assert bad.size == 0, (f"{bad.size} of {len(ii)} differ; first at ({ii[bad[0]]}, {jj[bad[0]]}): "
                           f"got {have[bad[0]]:#x} want {want[bad[0]]:#x}")


@pytest.mark.parametrize("shape", [(8, 300, 512), (700, 640, 1024)])
@pytest.mark.parametrize("bias_kind", ["bf16", "e4m3"])
def test_bias_full_range_operands_within_tolerance(hq, shape, bias_kind):
    m, n, k = shape
    rng = np.random.default_rng(zlib.crc32(repr((shape, bias_kind, "full")).encode()))
    t = fp8.decode_table(fp8.E4M3)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    xq, wq = rng.choice(finite, (m, k)), rng.choice(finite, (n, k))
    xs = rng.uniform(1e-4, 1e-3, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-3, n).astype(np.float32)
    got, bvals = _run(hq, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bias_kind, "bf16", rng, 1.0)
    ii, jj = rng.integers(0, m, 5000), rng.integers(0, n, 5000)
    ref, at = G.gemm_a8w8_rows(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, np.stack([ii, jj], axis=1))
    ref = ref + bvals[jj]
    run = window_drop(xq[ii], fp8.E4M3, wq[jj], fp8.E4M3) * np.abs(xs[ii] * ws[jj])
    err = np.abs(G.bf16_bits_to_f64(got[ii, jj]) - ref)
    assert np.all(err <= G.tolerance(ref, at) + run)


@pytest.mark.parametrize("out_kind", ["e4m3", "e5m2"])
def test_fp8_output_full_range_within_half_step(hq, out_kind):
    """Codes of full-range products: each decodes to within half an FP8 step of
    ref / out_scale, widened by the GEMM's own error bound; values past the
    format's maximum saturate."""
    m, n, k = 520, 384, 768
    rng = np.random.default_rng(77 + len(out_kind))
    t = fp8.decode_table(fp8.E4M3)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    xq, wq = rng.choice(finite, (m, k)), rng.choice(finite, (n, k))
    xs = rng.uniform(1e-4, 1e-3, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-3, n).astype(np.float32)
    fmt = FMT[out_kind]
    ii, jj = rng.integers(0, m, 6000), rng.integers(0, n, 6000)
    ref, at = G.gemm_a8w8_rows(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, np.stack([ii, jj], axis=1))
    # an output scale (from the oracle's values) that saturates about a tenth of the outputs
    out_scale = np.float32(np.quantile(np.abs(ref), 0.9) / fp8.fmax(fmt))
    got, _ = _run(hq, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, "none", out_kind, rng, out_scale)
    run = window_drop(xq[ii], fp8.E4M3, wq[jj], fp8.E4M3) * np.abs(xs[ii] * ws[jj])
    v = ref / float(out_scale)
    slack = (2.0 ** -22 * at + run) / float(out_scale) + 2.0 ** -21 * np.abs(v)
    dec = fp8.decode_table(fmt)[got[ii, jj]]
    fmax = fp8.fmax(fmt)
    mant, emin = (3, -6) if fmt == fp8.E4M3 else (2, -14)
    sat = np.abs(v) > fmax * (1 + 2.0 ** -10) + slack
    mx = 0x7E if fmt == fp8.E4M3 else 0x7B
    assert np.all(got[ii, jj][sat] == np.where(v[sat] > 0, mx, 0x80 | mx))
    inner = np.abs(v) < fmax * (1 - 2.0 ** -10)
    e = np.floor(np.log2(np.maximum(np.abs(v[inner]), 2.0 ** emin)))
    half = np.ldexp(0.5, (e - mant).astype(np.int64))
    assert np.all(np.abs(dec[inner] - v[inner]) <= half + slack[inner])
    assert sat.any() and inner.any()


def test_plain_epilogue_equals_hq_gemm_a8w8(hq):
    """No bias, bf16 output: the same bits as hq_gemm_a8w8."""
    rng = np.random.default_rng(5)
    m, n, k = 300, 520, 1040
    xq = rng.integers(0, 0x7E, (m, k), dtype=np.uint8)
    wq = rng.integers(0, 0x7E, (n, k), dtype=np.uint8)
    xs = dev_f32(rng.uniform(0.1, 1.0, m).astype(np.float32))
    ws = dev_f32(rng.uniform(0.1, 1.0, n).astype(np.float32))
    pre = hq.hq_preshuffle_weight(dev_u8(wq))
    a = hq.hq_gemm_a8w8(dev_u8(xq), fp8.E4M3, pre, fp8.E4M3, xs, ws, n)
    b = hq.hq_gemm_a8w8_epilogue(dev_u8(xq), fp8.E4M3, pre, fp8.E4M3, xs, ws, n)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---- grouped ---------------------------------------------------------------------

def _grouped_bias(rng, e_count, n, kind):
    """(device bias [E, n], device bias_scale [E] or None, float64 values [E, n])."""
    if kind == "bf16":
        b = (rng.standard_normal((e_count, n)) * 8).astype(np.float32)
        bits = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return (torch.from_numpy(bits.view(np.int16)).cuda(), None,
                np.stack([G.bias_values(bits[i], G.BIAS_BF16) for i in range(e_count)]))
    table = fp8.decode_table(FMT[kind])
    finite = np.array([c for c in range(256) if np.isfinite(table[c])], dtype=np.uint8)
    codes = rng.choice(finite, (e_count, n))
    bsc = rng.uniform(0.01, 0.1, e_count).astype(np.float32)
    vals = np.stack([G.bias_values(codes[i], KIND[kind], bsc[i]) for i in range(e_count)])
    return dev_u8(codes), dev_f32(bsc), vals


@pytest.mark.parametrize("bias_kind", BIASES)
@pytest.mark.parametrize("out_kind", OUTS)
def test_grouped_epilogue_bit_exact_on_exact_accumulators(hq, bias_kind, out_kind):
    """Per-expert bias rows and a shared output scale over ragged groups (two
    empty experts, rows past the last offset left untouched): on exact
    accumulators every covered element equals epilogue_f32 bit for bit."""
    rng = np.random.default_rng(zlib.crc32(repr(("grouped", bias_kind, out_kind)).encode()))
    counts = [5, 0, 130, 1, 0, 257, 64]
    e_count = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t, n, k = int(offsets[-1]) + 7, 144, 400
    xq = narrow_codes(rng, (t, k), fp8.E4M3)
    wq = narrow_codes(rng, (e_count, n, k), fp8.E5M2)
    xs = rng.uniform(1e-3, 2.0, t).astype(np.float32)
    ws = rng.uniform(1e-3, 2.0, (e_count, n)).astype(np.float32)
    out_scale = np.float32(rng.uniform(0.5, 4.0))
    kw = {}
    bvals = None
    if bias_kind != "none":
        bd, bs, bvals = _grouped_bias(rng, e_count, n, bias_kind)
        kw.update(bias=bd, bias_type=KIND[bias_kind], bias_scale=bs)
    if out_kind != "bf16":
        kw.update(out_scale=dev_f32(np.array([out_scale])), out_fmt=FMT[out_kind])
        sentinel = 0x55
        out = torch.full((t, n), sentinel, dtype=torch.uint8, device="cuda")
    else:
        sentinel = 0x7FC1
        out = torch.full((t, n), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    pre = torch.cat([hq.hq_preshuffle_weight(dev_u8(wq[i])) for i in range(e_count)])
    off = torch.from_numpy(offsets).cuda()
    hq.hq_grouped_gemm_a8w8_epilogue(dev_u8(xq), fp8.E4M3, pre, fp8.E5M2, dev_f32(xs), dev_f32(ws.reshape(-1)), off,
                                     e_count, n, out=out, **kw)
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(got[offsets[-1]:] == sentinel)
    dx, dw = fp8.decode(xq, fp8.E4M3), fp8.decode(wq, fp8.E5M2)
    for e in range(e_count):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        acc = dx[lo:hi] @ dw[e].T
        acc32 = acc.astype(np.float32)
        assert np.array_equal(acc32.astype(np.float64), acc)
        b = None if bvals is None else np.broadcast_to(bvals[e], acc.shape).astype(np.float32)
        want = G.epilogue_f32(acc32, xs[lo:hi, None], ws[e][None, :], b,
                              None if out_kind == "bf16" else out_scale, FMT.get(out_kind))
        bad = np.argwhere(got[lo:hi] != want)
        assert bad.size == 0, (f"expert {e}: {len(bad)} differ; first at row {lo + bad[0][0]}, col {bad[0][1]}: "
                               f"got {got[lo + bad[0][0], bad[0][1]]:#x} want {want[bad[0][0], bad[0][1]]:#x}")


def test_grouped_plain_epilogue_equals_hq_grouped_gemm_a8w8(hq):
    """No bias, bf16 output: the same bits as hq_grouped_gemm_a8w8 (full-range codes)."""
    rng = np.random.default_rng(9)
    counts = [300, 0, 77, 513]
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    t, n, k = sum(counts), 520, 1040
    xq = dev_u8(rng.integers(0, 0x7E, (t, k), dtype=np.uint8))
    wq = rng.integers(0, 0x7E, (len(counts), n, k), dtype=np.uint8)
    pre = torch.cat([hq.hq_preshuffle_weight(dev_u8(wq[i])) for i in range(len(counts))])
    xs = dev_f32(rng.uniform(0.1, 1.0, t).astype(np.float32))
    ws = dev_f32(rng.uniform(0.1, 1.0, len(counts) * n).astype(np.float32))
    a = hq.hq_grouped_gemm_a8w8(xq, fp8.E4M3, pre, fp8.E4M3, xs, ws, offsets, len(counts), n)
    b = hq.hq_grouped_gemm_a8w8_epilogue(xq, fp8.E4M3, pre, fp8.E4M3, xs, ws, offsets, len(counts), n)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("shape", [(3601, 3648, 400),    # 256 x 256
                                   (2001, 1088, 272),    # 128 x 128
                                   (1000, 1088, 400),    # 64 x 128
                                   (1000, 1088, 512)])   # 64 x 128, K split inside the workgroup
@pytest.mark.parametrize("bias_kind", ["none", "bf16"])
def test_full_line_stores_every_element(hq, shape, bias_kind):
    """bf16 outputs go out as whole 128-byte lines when N % 64 == 0: the
    256 x 256 tile swaps pieces between lanes of rows r and r + 8 of each
    16-row block (blocks with all 16 rows present), the 32-column-per-wavefront
    tiles stage the tile through LDS (tiles whose columns all exist). M = 3601,
    2001, 1000 end in a partial row tile; N = 3648 leaves three of the last
    256-column tile's wavefront columns empty, N = 1088 ends in a half 128-column
    tile (per-lane stores). Every element is compared with the oracle's
    epilogue on exact accumulators."""
    m, n, k = shape
    rng = np.random.default_rng(zlib.crc32(repr(("full lines", shape, bias_kind)).encode()))
    xq = narrow_codes(rng, (m, k), fp8.E4M3)
    wq = narrow_codes(rng, (n, k), fp8.E4M3)
    xs = rng.uniform(1e-3, 2.0, m).astype(np.float32)
    ws = rng.uniform(1e-3, 2.0, n).astype(np.float32)
    got, bvals = _run(hq, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, bias_kind, "bf16", rng, 1.0)
    acc = fp8.decode(xq, fp8.E4M3) @ fp8.decode(wq, fp8.E4M3).T
    acc32 = acc.astype(np.float32)
    assert np.array_equal(acc32.astype(np.float64), acc)  # exact in float32
    want = G.epilogue_f32(acc32, xs[:, None], ws[None, :],
                          None if bvals is None else bvals[None, :].astype(np.float32), None, None)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} differ; first at {tuple(bad[0])}: got {got[tuple(bad[0])]:#x}"


@pytest.mark.parametrize("out_kind", ["e4m3", "e5m2"])
@pytest.mark.parametrize("bias_kind", ["none", "e4m3"])
def test_fp8_output_staged_every_element(hq, out_kind, bias_kind):
    """FP8 output codes of the 256 x 256 tile go through LDS and out as whole
    row segments when N % 16 == 0 and the tile's 256 columns all exist; the
    last column tile of N = 3648 (64 columns) and the ragged last row tile of
    M = 3601 take the per-lane stores or the row mask. Every code is compared
    with the oracle's epilogue on exact accumulators."""
    m, n, k = 3601, 3648, 400
    rng = np.random.default_rng(zlib.crc32(repr(("fp8 staged", out_kind, bias_kind)).encode()))
    xq = narrow_codes(rng, (m, k), fp8.E4M3)
    wq = narrow_codes(rng, (n, k), fp8.E5M2)
    xs = rng.uniform(1e-3, 2.0, m).astype(np.float32)
    ws = rng.uniform(1e-3, 2.0, n).astype(np.float32)
    out_scale = np.float32(rng.uniform(0.5, 4.0))
    got, bvals = _run(hq, xq, fp8.E4M3, wq, fp8.E5M2, xs, ws, bias_kind, out_kind, rng, out_scale)
    acc = fp8.decode(xq, fp8.E4M3) @ fp8.decode(wq, fp8.E5M2).T
    acc32 = acc.astype(np.float32)
    assert np.array_equal(acc32.astype(np.float64), acc)  # exact in float32
    want = G.epilogue_f32(acc32, xs[:, None], ws[None, :],
                          None if bvals is None else bvals[None, :].astype(np.float32), out_scale, FMT[out_kind])
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} differ; first at {tuple(bad[0])}: got {got[tuple(bad[0])]:#x}"
