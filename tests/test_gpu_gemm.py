"""GPU parity of hq_preshuffle_weight, hq_gemm_a8w8 and hq_grouped_gemm_a8w8 (and
their strict forms) with the oracle: pre-shuffle bit-exact; strict GEMMs within
the method's bound on every element; FP8-path GEMMs within that bound plus the
matrix cores' window drop on every element, with the share of elements outside
the method's bound alone at most the share measured for the test
(gpu_helpers.MEASURED_SHARE).
"""
import zlib

import numpy as np
import pytest
import torch

import workloads
from oracle import fp8, gemm as G, preshuffle as P, quantize as Q
from tests.gpu_helpers import (allowed_share, check_gemm, dev_bf16, dev_f32, dev_u8, host, narrow_codes,
                               require_gpu)

pytestmark = pytest.mark.gpu

PAIRS = [(fp8.E4M3, fp8.E4M3), (fp8.E5M2, fp8.E5M2), (fp8.E4M3, fp8.E5M2), (fp8.E5M2, fp8.E4M3)]


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _finite_codes(rng, shape, fmt):
    t = fp8.decode_table(fmt)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    return rng.choice(finite, size=shape)


def _gemm(hq, xq, xf, wq, wf, xs, ws, strict=False):
    n = wq.shape[0]
    pre = hq.hq_preshuffle_weight(dev_u8(wq))
    out = hq.hq_gemm_a8w8(dev_u8(xq), xf, pre, wf, dev_f32(np.atleast_1d(xs)), dev_f32(np.atleast_1d(ws)), n,
                          strict=strict)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("nk", [(16, 128), (40, 304), (1, 16), (33, 4112), (2048, 1024)])
def test_preshuffle_bit_exact(hq, nk):
    n, k = nk
    rng = np.random.default_rng(n + k)
    w = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    got = host(hq.hq_preshuffle_weight(dev_u8(w)))
    assert np.array_equal(got, P.preshuffle(w))


# M <= 64 runs the weight-streaming kernel (one block per 16-column fragment,
# K split over 16 wavefronts, chunks of 4 or 2 K blocks), larger M the tiles.
SHAPES = [(1, 16, 16), (16, 64, 128), (17, 33, 144), (130, 200, 400), (256, 256, 256), (300, 520, 1040),
          (129, 130, 2064),
          (4, 64, 16384),      # several K chunks per wavefront
          (33, 48, 2064),      # 4 activation blocks, ragged K
          (64, 100, 1040),     # largest skinny M, ragged N
          (65, 96, 256),       # smallest tiled M
          (8, 7, 304),         # N not a multiple of 4: element stores
          (2, 2050, 384)]      # many fragments, ragged last group


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("pair", PAIRS)
@pytest.mark.parametrize("scales", ["vector", "scalar"])
def test_gemm_narrow_operands_strict(hq, shape, pair, scales):
    """Every output element within the strict bound (MFMA runs exact here)."""
    m, n, k = shape
    xf, wf = pair
    rng = np.random.default_rng(zlib.crc32(repr((shape, pair, scales)).encode()))
    xq = narrow_codes(rng, (m, k), xf)
    wq = narrow_codes(rng, (n, k), wf)
    if scales == "vector":
        xs = rng.uniform(1e-3, 2.0, m).astype(np.float32)
        ws = rng.uniform(1e-3, 2.0, n).astype(np.float32)
    else:
        xs, ws = np.float32(0.37), np.float32(1.9)
    out = _gemm(hq, xq, xf, wq, wf, xs, ws)
    check_gemm(out, xq, xf, wq, wf, xs, ws, strict_only=True)
    strict = _gemm(hq, xq, xf, wq, wf, xs, ws, strict=True)
    assert np.array_equal(strict, out)  # exact partial sums: the same bits either way


def _edge_pairs(rng, m, n, count):
    """Random output positions plus every combination of tile-edge rows and
    columns (first, 255/256 and 127/128 boundaries, last)."""
    rows = sorted({0, 127, 128, 255, 256, m // 2, m - 2, m - 1})
    cols = sorted({0, 7, 8, 127, 128, 255, 256, n // 2, n - 9, n - 8, n - 1})
    edge = np.array([(r, c) for r in rows for c in cols if 0 <= r < m and 0 <= c < n], dtype=np.int64)
    rnd = np.stack([rng.integers(0, m, count), rng.integers(0, n, count)], axis=1)
    return np.concatenate([edge, rnd])


# One shape per tile configuration the launcher's cost model picks (ragged M,
# N and K): 256 x 256 (eight wavefronts), 128 x 256, 128 x 128 and
# 64 x 128 (the small test shapes above all take 64 x 128 as well).
@pytest.mark.parametrize("shape", [(3600, 3700, 400), (3841, 3330, 1024),   # 256 x 256
                                   (3601, 3648, 400),                       # 256 x 256, whole-line stores
                                   (2000, 4000, 272),                       # 128 x 256
                                   (4000, 1000, 272),                       # 128 x 128
                                   (2001, 1088, 272),                       # 128 x 128, staged stores
                                   (1000, 1000, 400),                       # 64 x 128
                                   (1000, 1088, 400),                       # 64 x 128, staged stores
                                   (1000, 1088, 512)])                      # 64 x 128, K split in the workgroup
@pytest.mark.parametrize("pair", PAIRS)
def test_gemm_tile_configs_narrow_strict(hq, shape, pair):
    m, n, k = shape
    xf, wf = pair
    rng = np.random.default_rng(zlib.crc32(repr((shape, pair, "tiles")).encode()))
    xq = narrow_codes(rng, (m, k), xf)
    wq = narrow_codes(rng, (n, k), wf)
    xs = rng.uniform(1e-3, 2.0, m).astype(np.float32)
    ws = rng.uniform(1e-3, 2.0, n).astype(np.float32)
    out = _gemm(hq, xq, xf, wq, wf, xs, ws)
    pairs = _edge_pairs(rng, m, n, 3000)
    check_gemm(out, xq, xf, wq, wf, xs, ws, pairs=pairs, strict_only=True)
    strict = _gemm(hq, xq, xf, wq, wf, xs, ws, strict=True)
    check_gemm(strict, xq, xf, wq, wf, xs, ws, pairs=pairs, strict_only=True)


@pytest.mark.parametrize("shape", [(16, 64, 128), (130, 200, 400), (64, 96, 1024)])
@pytest.mark.parametrize("pair", PAIRS)
def test_gemm_full_range_codes(hq, shape, pair):
    """Every finite code, both formats: the FP8 path within the bound plus the
    window drop, the strict path within the bound, on every element."""
    m, n, k = shape
    xf, wf = pair
    rng = np.random.default_rng(hash((shape, pair, 7)) % 2**32)
    xq = _finite_codes(rng, (m, k), xf)
    wq = _finite_codes(rng, (n, k), wf)
    xs = rng.uniform(1e-4, 1e-2, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    out = _gemm(hq, xq, xf, wq, wf, xs, ws)
    key = f"full_range {shape} {pair}"
    check_gemm(out, xq, xf, wq, wf, xs, ws, max_strict_frac=allowed_share(key, m * n), label=key)
    strict = _gemm(hq, xq, xf, wq, wf, xs, ws, strict=True)
    check_gemm(strict, xq, xf, wq, wf, xs, ws, strict_only=True, label=key + " strict")


def test_one_hot_reproduces_scales(hq):
    m, n, k = 40, 48, 256
    xq = np.zeros((m, k), np.uint8)
    wq = np.zeros((n, k), np.uint8)
    for i in range(m):
        xq[i, (7 * i) % k] = 0x38
    for j in range(n):
        wq[j, (7 * (j % m)) % k] = 0x38
    xs = (np.arange(m) + 1).astype(np.float32) / 8
    ws = (np.arange(n) + 1).astype(np.float32) / 16
    out = _gemm(hq, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    ref = G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
    # every product x_s * w_s is exact in float32 (at most 11 significant bits);
    # the kernel's only rounding is then the final round-to-nearest-even to bf16
    ref_bf16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref_bf16)


def test_tiny_per_tensor_workload(hq):
    x, w = workloads.tiny_per_tensor(0)
    xq, xs, _ = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, Q.PER_TENSOR)
    wq, ws, _ = Q.quantize_dynamic(w, Q.F32, fp8.E4M3, Q.PER_TENSOR)
    # quantize on the GPU too, and feed the GPU's own codes and scales
    gx, gxs, _ = hq.hq_quantize_fp8(dev_f32(x), fp8.E4M3, Q.PER_TENSOR)
    gw, gws, _ = hq.hq_quantize_fp8(dev_f32(w), fp8.E4M3, Q.PER_TENSOR)
    pre = hq.hq_preshuffle_weight(gw)
    out = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, 64))
    strict = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, 64, strict=True))
    assert np.array_equal(host(gx), xq) and np.array_equal(host(gw), wq)
    check_gemm(out, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, max_strict_frac=allowed_share("tiny", 16 * 64),
               label="tiny")
    check_gemm(strict, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, strict_only=True, label="tiny strict")


def _sample_pairs(rng, m, n, count):
    pairs = np.stack([rng.integers(0, m, count), rng.integers(0, n, count)], axis=1)
    corners = np.array([[0, 0], [m - 1, n - 1], [0, n - 1], [m - 1, 0]])
    return np.concatenate([pairs, corners])


def test_output_past_2_31_elements(hq):
    """M = 65540, N = 32768, K = 128: the bf16 output holds 2^31 + 131072
    elements (4.3 GB), so its row offsets must be carried in 64 bits; sampled
    outputs on both sides of element 2^31 (rows 65535 .. 65539 included)
    against the oracle."""
    m, n, k = 65540, 32768, 128
    rng = np.random.default_rng(2031)
    xq = _finite_codes(rng, (m, k), fp8.E4M3)
    wq = _finite_codes(rng, (n, k), fp8.E5M2)
    xs = rng.uniform(1e-3, 1e-1, m).astype(np.float32)
    ws = rng.uniform(1e-3, 1e-1, n).astype(np.float32)
    out = _gemm(hq, xq, fp8.E4M3, wq, fp8.E5M2, xs, ws)
    edge = np.array([[r, c] for r in (0, 65535, 65536, 65537, m - 1) for c in (0, 255, 256, n - 1)])
    pairs = np.concatenate([_sample_pairs(rng, m, n, 6000), edge])
    check_gemm(out, xq, fp8.E4M3, wq, fp8.E5M2, xs, ws, pairs=pairs,
               max_strict_frac=allowed_share("past_2_31", len(pairs)), label="past_2_31")
    del out


def test_ptpc_square_full_size(hq):
    """4096^3 with per-token X and per-output-channel W, in the launch
    configuration the benchmark times (the weight quantized straight into the
    pre-shuffled layout); every output element against the oracle, for the
    FP8 path and the strict path."""
    x, w = workloads.ptpc_square(1)
    gx, gxs, _ = hq.hq_quantize_fp8(dev_bf16(x), fp8.E4M3, Q.PER_TOKEN)
    pre, gws, _, _ = hq.hq_quantize_fp8_preshuffled(dev_bf16(w), fp8.E4M3)
    out = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, 4096))
    strict = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, 4096, strict=True))
    xq, xs, _ = Q.quantize_dynamic(x, Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    wq, ws, _ = Q.quantize_dynamic(w, Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    assert np.array_equal(host(gx), xq)
    assert np.array_equal(host(gws).view(np.uint32), ws.view(np.uint32))
    check_gemm(out, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, max_strict_frac=allowed_share("ptpc 4096^3", 4096 * 4096),
               label="ptpc 4096^3")
    check_gemm(strict, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, strict_only=True, label="ptpc 4096^3 strict")


@pytest.mark.parametrize("m", [1, 8, 32])
def test_decode_skinny_into_view(hq, m):
    """Output written into a dense [m, 2048] view at a 16-byte aligned, non-zero
    offset of a sentinel-filled flat buffer; the rest must stay untouched."""
    x, w = workloads.decode_skinny(m)
    n, k = 2048, 7168
    gx, gxs, _ = hq.hq_quantize_fp8(dev_bf16(x), fp8.E4M3, Q.PER_TOKEN)
    gw, gws, _ = hq.hq_quantize_fp8(dev_bf16(w), fp8.E4M3, Q.PER_TOKEN)
    pre = hq.hq_preshuffle_weight(gw)
    sentinel = 0x7FC1
    flat = torch.full((m * n + 1024,), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    off = 520  # bf16 elements: 1040 bytes, 16-byte aligned
    view = flat[off:off + m * n].view(m, n)
    hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, n, out=view)
    allb = host(flat)
    assert np.all(allb[:off] == sentinel) and np.all(allb[off + m * n:] == sentinel)
    xq, xs, _ = Q.quantize_dynamic(x, Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    wq, ws, _ = Q.quantize_dynamic(w, Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    check_gemm(allb[off:off + m * n].reshape(m, n), xq, fp8.E4M3, wq, fp8.E4M3, xs, ws,
               max_strict_frac=allowed_share(f"decode m={m}", m * n), label=f"decode m={m}")
    flat.view(torch.int16).fill_(sentinel)
    hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, n, out=view, strict=True)
    allb = host(flat)
    assert np.all(allb[:off] == sentinel) and np.all(allb[off + m * n:] == sentinel)
    check_gemm(allb[off:off + m * n].reshape(m, n), xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, strict_only=True,
               label=f"decode m={m} strict")


# shapes whose unsplit launch needs more than one chunk of loads per wavefront
# and has fewer than 256 column groups (the only ones the plan splits): K
# blocks > 64 for M <= 16 (two half-fragment groups per 16 columns), > 32 for
# M <= 32, > 16 for M <= 64
@pytest.mark.parametrize("shape", [(1, 1024, 14336), (16, 1024, 9216), (32, 2048, 7168), (33, 96, 2304),
                                   (64, 520, 4096), (8, 64, 8336)])
def test_skinny_split_matches_unsplit_and_oracle(hq, shape):
    """The decode shapes split their weight stream over several workgroups when
    given a workspace; the output must be bit-identical to the unsplit launch
    (same summation order), stay so over repeated calls on the same workspace
    (the last workgroup of each column group resets its counter), leave the
    counters zero, and match the oracle within the GEMM bound."""
    m, n, k = shape
    need = hq.hq_gemm_workspace_bytes(m, n, k)
    assert need > 0
    rng = np.random.default_rng(hash(shape) % 2**32)
    xq = _finite_codes(rng, (m, k), fp8.E4M3)
    wq = _finite_codes(rng, (n, k), fp8.E4M3)
    xs = rng.uniform(1e-4, 1e-2, m).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, n).astype(np.float32)
    gx, gw = dev_u8(xq), dev_u8(wq)
    pre = hq.hq_preshuffle_weight(gw)
    gxs, gws = dev_f32(xs), dev_f32(ws)
    plain = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, n, workspace=False))
    work = torch.zeros(need + 64, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        split = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, n, workspace=work))
        assert np.array_equal(split, plain)
    torch.cuda.synchronize()
    # the per-group counters (the workspace's first words) are back at zero
    frags = -(-n // 32) * 2
    groups = 2 * frags if m <= 16 else -(-frags // 2)
    assert int(work[:4 * groups].count_nonzero()) == 0
    key = f"split {shape}"
    check_gemm(plain, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, max_strict_frac=allowed_share(key, m * n), label=key)
    # the strict form splits the same way (M <= 32) or takes the tiles
    for _ in range(2):
        strict = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, n, workspace=work, strict=True))
        check_gemm(strict, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, strict_only=True, label=key + " strict")
    torch.cuda.synchronize()
    assert int(work[:4 * groups].count_nonzero()) == 0


def test_workspace_shared_across_decode_shapes(hq):
    """One workspace serves split launches of different shapes in turn: a
    shape with few column groups (its partial sums right after the counter
    region), then one with many (whose counters must not land on those
    partials), then the first again; each bit-identical to its unsplit launch."""
    shapes = [(1, 320, 14336), (1, 1536, 14336), (1, 320, 14336), (16, 1024, 9216)]
    need = max(hq.hq_gemm_workspace_bytes(*s) for s in shapes)
    work = torch.zeros(need, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(99)
    for m, n, k in shapes:
        assert hq.hq_gemm_workspace_bytes(m, n, k) > 0
        xq = _finite_codes(rng, (m, k), fp8.E4M3)
        wq = _finite_codes(rng, (n, k), fp8.E4M3)
        gx, pre = dev_u8(xq), hq.hq_preshuffle_weight(dev_u8(wq))
        xs, ws = dev_f32(rng.uniform(1e-3, 1e-2, m)), dev_f32(rng.uniform(1e-3, 1e-2, n))
        plain = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, xs, ws, n, workspace=False))
        split = host(hq.hq_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, xs, ws, n, workspace=work))
        assert np.array_equal(split, plain), (m, n, k)
    torch.cuda.synchronize()
    assert int(work[:1024].count_nonzero()) == 0


def test_empty_output_is_noop(hq):
    xq = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    wq = torch.zeros((64, 128), dtype=torch.uint8, device="cuda")
    pre = hq.hq_preshuffle_weight(wq)
    out = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    hq.hq_gemm_a8w8(xq, fp8.E4M3, pre, fp8.E4M3, torch.ones(1, device="cuda"), torch.ones(1, device="cuda"), 64,
                    out=out)
    torch.cuda.synchronize()


def test_invalid_gemm_leaves_out_untouched(hq):
    xq = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    wq = torch.zeros((16, 128), dtype=torch.uint8, device="cuda")
    pre = hq.hq_preshuffle_weight(wq)
    out = torch.full((8, 16), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        hq.hq_gemm_a8w8(xq, fp8.E4M3, pre, fp8.E4M3, torch.ones(3, device="cuda"), torch.ones(1, device="cuda"),
                        16, out=out)
    flat = torch.zeros(8 * 16 + 1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # odd bf16 offset: not 16-byte aligned
        hq.hq_gemm_a8w8(xq, fp8.E4M3, pre, fp8.E4M3, torch.ones(1, device="cuda"), torch.ones(1, device="cuda"),
                        16, out=flat[1:].view(8, 16))
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((flat == 0).all())


# ---- grouped -------------------------------------------------------------------

def _grouped(hq, xq, xf, wq_e, wf, xs, ws, offsets, out=None, strict=False):
    e, n, k = wq_e.shape
    pre = torch.cat([hq.hq_preshuffle_weight(dev_u8(wq_e[i])) for i in range(e)])
    off = torch.from_numpy(np.asarray(offsets, dtype=np.int32)).cuda()
    o = hq.hq_grouped_gemm_a8w8(dev_u8(xq), xf, pre, wf, dev_f32(np.atleast_1d(xs)), dev_f32(ws.reshape(-1)),
                                off, e, n, out=out, strict=strict)
    torch.cuda.synchronize()
    return o


def _check_grouped(out_bits, xq, xf, wq_e, wf, xs, ws, offsets, strict=False, key=None):
    t = xq.shape[0]
    e = wq_e.shape[0]
    xsv = np.full(t, np.float32(xs)) if np.ndim(xs) == 0 or np.size(xs) == 1 else np.asarray(xs, np.float32)
    for i in range(e):
        lo, hi = int(offsets[i]), int(offsets[i + 1])
        if hi <= lo:
            continue
        wse = ws[i] if ws.ndim == 2 else np.full(wq_e.shape[1], ws[i], np.float32)
        share = None if strict else allowed_share(f"{key} expert {i}", (hi - lo) * wq_e.shape[1])
        check_gemm(out_bits[lo:hi], xq[lo:hi], xf, wq_e[i], wf, xsv[lo:hi], wse, strict_only=strict,
                   max_strict_frac=share, label=None if key is None else f"{key} expert {i}")


@pytest.mark.parametrize("pair", PAIRS[:2])
def test_grouped_narrow_strict_with_empty_experts(hq, pair):
    xf, wf = pair
    rng = np.random.default_rng(3)
    counts = [5, 0, 130, 1, 0, 257, 64]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    t, n, k = int(offsets[-1]), 144, 400
    xq = narrow_codes(rng, (t, k), xf)
    wq = narrow_codes(rng, (len(counts), n, k), wf)
    xs = rng.uniform(0.01, 1, t).astype(np.float32)
    ws = rng.uniform(0.01, 1, (len(counts), n)).astype(np.float32)
    out = host(_grouped(hq, xq, xf, wq, wf, xs, ws, offsets))
    _check_grouped(out, xq, xf, wq, wf, xs, ws, offsets, strict=True)
    assert np.array_equal(host(_grouped(hq, xq, xf, wq, wf, xs, ws, offsets, strict=True)), out)


def test_grouped_per_expert_scalar_scale_and_uncovered_rows(hq):
    """w_scale with one entry per expert; rows past offsets[E] stay untouched."""
    rng = np.random.default_rng(4)
    offsets = np.array([0, 10, 10, 50], dtype=np.int32)
    t, n, k = 64, 32, 128
    xq = narrow_codes(rng, (t, k), fp8.E4M3)
    wq = narrow_codes(rng, (3, n, k), fp8.E4M3)
    xs = rng.uniform(0.1, 1, t).astype(np.float32)
    ws = np.array([0.5, 2.0, 0.25], np.float32)
    sentinel = 0x7FC1
    out = torch.full((t, n), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    _grouped(hq, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, offsets, out=out)
    ob = host(out)
    assert np.all(ob[50:] == sentinel)
    _check_grouped(ob, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, offsets, strict=True)


def test_grouped_call_sequence_no_contamination(hq):
    """Expert counts 1, 2, 1, 4 on 4x4-ish and 16x16-ish problems in sequence
    (the megablocks notes' state-contamination sequence)."""
    rng = np.random.default_rng(6)
    for z in (1, 2, 1, 4):
        for base in (4, 16):
            counts = rng.integers(0, 3 * base, size=z)
            offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
            t = max(int(offsets[-1]), 1)
            offsets[-1] = t
            n, k = 16 * base // 4 + 16, 128
            xq = narrow_codes(rng, (t, k), fp8.E4M3)
            wq = narrow_codes(rng, (z, n, k), fp8.E4M3)
            xs = rng.uniform(0.1, 1, t).astype(np.float32)
            ws = rng.uniform(0.1, 1, (z, n)).astype(np.float32)
            out = host(_grouped(hq, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, offsets))
            _check_grouped(out, xq, fp8.E4M3, wq, fp8.E4M3, xs, ws, offsets, strict=True)


def test_grouped_moe_full_size(hq):
    """8 experts, 8192 tokens, N=2048, K=1024 with two empty experts; GPU
    quantization feeds the grouped GEMM; every output element per expert, for
    the FP8 path and the strict path."""
    x, w, offsets = workloads.grouped_moe(3)
    e, n, k = w.shape
    gx, gxs, _ = hq.hq_quantize_fp8(dev_bf16(x), fp8.E4M3, Q.PER_TOKEN)
    gw, gws, _ = hq.hq_quantize_fp8(dev_bf16(w.reshape(-1, k)), fp8.E4M3, Q.PER_TOKEN)
    pre = torch.cat([hq.hq_preshuffle_weight(gw[i * n:(i + 1) * n]) for i in range(e)])
    off = torch.from_numpy(offsets).cuda()
    sentinel = 0x7FC1
    out = torch.full((x.shape[0], n), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    hq.hq_grouped_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, off, e, n, out=out)
    ob = host(out)
    xq, xs, _ = Q.quantize_dynamic(x, Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    wq, ws, _ = Q.quantize_dynamic(w.reshape(-1, k), Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    assert np.array_equal(host(gx), xq) and np.array_equal(host(gw), wq)
    assert not np.any(ob == sentinel)
    _check_grouped(ob, xq, fp8.E4M3, wq.reshape(e, n, k), fp8.E4M3, xs, ws.reshape(e, n), offsets, key="moe")
    out.view(torch.int16).fill_(sentinel)
    hq.hq_grouped_gemm_a8w8(gx, fp8.E4M3, pre, fp8.E4M3, gxs, gws, off, e, n, out=out, strict=True)
    ob = host(out)
    assert not np.any(ob == sentinel)
    _check_grouped(ob, xq, fp8.E4M3, wq.reshape(e, n, k), fp8.E4M3, xs, ws.reshape(e, n), offsets, strict=True,
                   key="moe strict")


def test_training_linear_gemm_shapes(hq):
    """One step of one layer of the training workload: E4M3 forward
    2048x4096x1024, E5M2 dgrad 2048x1024x4096 and wgrad 4096x1024x2048 with
    per-tensor scales from the rings' current scale (transposes made on torch)."""
    base, factors = workloads.training_linear(4, layers=1, steps=1)
    xb, wb, gb = workloads.training_step_inputs(base, factors, 0, 0)
    rng = np.random.default_rng(1)

    def qt(bits, fmt):
        return Q.quantize_dynamic(bits, Q.BF16, fmt, Q.PER_TENSOR)

    cases = []
    xq, xs, _ = qt(xb, fp8.E4M3)
    wq, ws, _ = qt(wb, fp8.E4M3)
    cases.append((xq, fp8.E4M3, wq, fp8.E4M3, xs, ws))                  # fwd: X W^T
    gq, gs, _ = qt(gb, fp8.E5M2)
    wq5, ws5, _ = qt(wb, fp8.E5M2)
    cases.append((gq, fp8.E5M2, np.ascontiguousarray(wq5.T), fp8.E5M2, gs, ws5))   # dgrad: G W
    xq5, xs5, _ = qt(xb, fp8.E5M2)
    cases.append((np.ascontiguousarray(gq.T), fp8.E5M2, np.ascontiguousarray(xq5.T), fp8.E5M2, gs, xs5))  # wgrad
    for name, (xq_, xf_, wq_, wf_, xs_, ws_) in zip(("fwd", "dgrad", "wgrad"), cases):
        out = _gemm(hq, xq_, xf_, wq_, wf_, xs_, ws_)
        n_el = xq_.shape[0] * wq_.shape[0]
        check_gemm(out, xq_, xf_, wq_, wf_, xs_, ws_, max_strict_frac=allowed_share(f"training {name}", n_el),
                   label=f"training {name}")
        strict = _gemm(hq, xq_, xf_, wq_, wf_, xs_, ws_, strict=True)
        check_gemm(strict, xq_, xf_, wq_, wf_, xs_, ws_, strict_only=True, label=f"training {name} strict")
