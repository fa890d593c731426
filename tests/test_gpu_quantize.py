"""GPU parity of hq_quantize_fp8 / hq_scale_ring_update with the oracle: codes,
scales, amax and ring state must match bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from oracle import fp8, quantize as Q
from tests.gpu_helpers import dev_bf16, dev_f32, host, require_gpu

pytestmark = pytest.mark.gpu

GRANS = [Q.PER_TENSOR, Q.PER_TOKEN, Q.PER_CHANNEL]
FMTS = [fp8.E4M3, fp8.E5M2]


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _gpu_quant(hq, x_np, dtype, fmt, gran):
    x = dev_bf16(x_np) if dtype == Q.BF16 else dev_f32(x_np)
    q, s, a = hq.hq_quantize_fp8(x, fmt, gran)
    torch.cuda.synchronize()
    return host(q), host(s), host(a)


def _assert_same(hq, x_np, dtype, fmt, gran, what=""):
    q, s, a = _gpu_quant(hq, x_np, dtype, fmt, gran)
    q_ref, s_ref, a_ref = Q.quantize_dynamic(x_np, dtype, fmt, gran)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), f"scale mismatch {what}"
    assert np.array_equal(a.view(np.uint32), a_ref.view(np.uint32)), f"amax mismatch {what}"
    if not np.array_equal(q, q_ref):
        bad = np.argwhere(q != q_ref)
        i, j = bad[0]
        raise AssertionError(f"{len(bad)} code mismatches {what}; first at ({i},{j}): gpu {q[i, j]:#04x} "
                             f"oracle {q_ref[i, j]:#04x}")


def test_tiny_per_tensor_workload(hq):
    x, w = workloads.tiny_per_tensor(0)
    for t in (x, w):
        for fmt in FMTS:
            _assert_same(hq, t, Q.F32, fmt, Q.PER_TENSOR, "tiny")


# shapes chosen to cover one vector, several blocks, ragged tails and every
# register-cache variant of the per-row kernel (incl. the streamed fallback)
SHAPES_BF16 = [(1, 16), (3, 48), (64, 512), (130, 4112), (257, 2064), (5, 16512), (300, 272)]
SHAPES_F32 = [(1, 16), (16, 128), (70, 1040), (9, 8208), (129, 4096)]


@pytest.mark.parametrize("shape", SHAPES_BF16)
@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("fmt", FMTS)
def test_bf16_random(hq, shape, gran, fmt):
    rng = np.random.default_rng(hash((shape, gran, fmt)) % 2**32)
    x = rng.standard_t(3, size=shape).astype(np.float32)
    x *= np.exp(rng.standard_normal((shape[0], 1)) * 2).astype(np.float32)
    _assert_same(hq, workloads.to_bf16_bits(x), Q.BF16, fmt, gran, f"{shape}")


@pytest.mark.parametrize("shape", SHAPES_F32)
@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("fmt", FMTS)
def test_f32_random(hq, shape, gran, fmt):
    rng = np.random.default_rng(hash((shape, gran, fmt, 1)) % 2**32)
    x = (rng.standard_normal(shape) * np.exp(rng.standard_normal((1, shape[1])) * 3)).astype(np.float32)
    _assert_same(hq, x, Q.F32, fmt, gran, f"{shape}")


@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("fmt", FMTS)
def test_special_values(hq, gran, fmt):
    rng = np.random.default_rng(99)
    x = rng.standard_normal((40, 64)).astype(np.float32)
    x[0, 3] = np.nan
    x[1, 5] = np.inf
    x[2, 7] = -np.inf
    x[3, :] = 0.0
    x[4, :] = -0.0
    x[5, 1] = -0.0
    x[6, :] = 1e-40            # float32 subnormals
    x[7, 2] = 3.0e38
    x[8, :] = 2.0 ** -130
    x[9, 9] = -np.nan
    x[:, 10] = 0.0
    x[:, 11] = np.nan
    _assert_same(hq, x, Q.F32, fmt, gran, "special f32")
    bits = workloads.to_bf16_bits(x)
    bits[20, 0] = 0x0001       # smallest bf16 subnormal
    bits[20, 1] = 0x8001
    bits[21, 0] = 0x7F80       # +Inf
    bits[22, 0] = 0xFFC1       # NaN with payload
    _assert_same(hq, bits, Q.BF16, fmt, gran, "special bf16")


def test_every_bf16_pattern(hq):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    for fmt in FMTS:
        for gran in GRANS:
            _assert_same(hq, bits, Q.BF16, fmt, gran, "all bf16 patterns")


# ---- the workloads at full size ------------------------------------------------

def test_ptpc_square_full(hq):
    x, w = workloads.ptpc_square(1)
    _assert_same(hq, x, Q.BF16, fp8.E4M3, Q.PER_TOKEN, "ptpc X per-token")
    _assert_same(hq, w, Q.BF16, fp8.E4M3, Q.PER_TOKEN, "ptpc W per-output-channel")
    _assert_same(hq, x, Q.BF16, fp8.E4M3, Q.PER_TENSOR, "ptpc X per-tensor")
    _assert_same(hq, x, Q.BF16, fp8.E4M3, Q.PER_CHANNEL, "ptpc X per-channel")


@pytest.mark.parametrize("m", [1, 8, 32])
def test_decode_skinny_full(hq, m):
    x, w = workloads.decode_skinny(m)
    _assert_same(hq, x, Q.BF16, fp8.E4M3, Q.PER_TOKEN, f"decode X m={m}")
    if m == 32:
        _assert_same(hq, w, Q.BF16, fp8.E4M3, Q.PER_TOKEN, "decode W")


def test_grouped_moe_full(hq):
    x, w, _ = workloads.grouped_moe(3)
    _assert_same(hq, x, Q.BF16, fp8.E4M3, Q.PER_TOKEN, "moe X")
    _assert_same(hq, w.reshape(-1, w.shape[-1]), Q.BF16, fp8.E4M3, Q.PER_TOKEN, "moe W")


def test_more_than_2_31_elements(hq):
    """A bf16 [65540, 32768] tensor: 2^31 + 131072 elements (4.3 GB), so every
    index past element 2^31 must be carried in 64 bits. Checked against the
    oracle on sampled rows on both sides of element 2^31 (per token: a row's
    codes, scale and amax depend on that row alone), on sampled columns (per
    channel, likewise), and per tensor with the maximum planted in the last
    element (every other value is clamped to |x| <= 8 except one planted in the
    next-to-last row), so the reduction has to reach it."""
    rows, cols = 65540, 32768
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20240531)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 8192):  # slabs: one fp32 draw of the whole tensor would take 8.6 GB
        r1 = min(rows, r0 + 8192)
        x[r0:r1] = torch.randn((r1 - r0, cols), generator=gen, device="cuda").clamp_(-8.0, 8.0)
    x[rows - 1, cols - 1] = 100.0
    x[rows - 2, 7] = -96.0
    rng = np.random.default_rng(5)
    srows = np.unique(np.concatenate([[0, 1, 65535, 65536, 65537, rows - 2, rows - 1], rng.integers(0, rows, 25)]))
    scols = np.unique(np.concatenate([[0, 7, cols - 1], rng.integers(0, cols, 13)]))
    ir, ic = torch.from_numpy(srows).cuda(), torch.from_numpy(scols).cuda()
    xr = host(x.index_select(0, ir).contiguous())
    xc = host(x.index_select(1, ic).contiguous())
    planted = (np.array([[100.0]], dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)

    def same_f32(gpu, ref):
        return np.array_equal(np.asarray(gpu, np.float32).view(np.uint32), np.asarray(ref, np.float32).view(np.uint32))

    for fmt in FMTS:
        q, s, a = hq.hq_quantize_fp8(x, fmt, Q.PER_TOKEN)
        q_ref, s_ref, a_ref = Q.quantize_dynamic(xr, Q.BF16, fmt, Q.PER_TOKEN)
        assert np.array_equal(host(q.index_select(0, ir)), q_ref), f"per-token codes, fmt {fmt}"
        assert same_f32(host(s)[srows], s_ref) and same_f32(host(a)[srows], a_ref), f"per-token scales, fmt {fmt}"
        del q, s, a

        q, s, a = hq.hq_quantize_fp8(x, fmt, Q.PER_CHANNEL)
        q_ref, s_ref, a_ref = Q.quantize_dynamic(xc, Q.BF16, fmt, Q.PER_CHANNEL)
        assert np.array_equal(host(q.index_select(1, ic).contiguous()), q_ref), f"per-channel codes, fmt {fmt}"
        assert same_f32(host(s)[scols], s_ref) and same_f32(host(a)[scols], a_ref), f"per-channel scales, fmt {fmt}"
        del q, s, a

        q, s, a = hq.hq_quantize_fp8(x, fmt, Q.PER_TENSOR)
        _, s_ref, a_ref = Q.quantize_dynamic(planted, Q.BF16, fmt, Q.PER_TENSOR)
        assert same_f32(host(a), a_ref) and same_f32(host(s), s_ref), f"per-tensor amax / scale, fmt {fmt}"
        q_ref, _, _ = Q.quantize_with_scale(xr, Q.BF16, fmt, s_ref)
        assert np.array_equal(host(q.index_select(0, ir)), q_ref), f"per-tensor codes, fmt {fmt}"
        del q, s, a
    del x
    torch.cuda.empty_cache()


def test_repeated_calls_with_shared_workspace(hq):
    """Per-tensor and per-channel reuse one workspace (zero-filled once) across
    calls of different sizes, single-pass and two-pass per-tensor grids
    included; each result must be independent of the previous call."""
    rng = np.random.default_rng(5)
    # float32 vectors: 131072 and 153600 (single pass, 4 per thread), 2^21
    # (single pass, 512 blocks of 16 per thread), 2^21 + 2^11 (two passes)
    shapes = [(512, 1024), (16, 64), (300, 2048), (1, 16), (2048, 4096), (1028, 8192)]
    ws = torch.zeros(max(hq.hq_quantize_workspace_bytes(g, *s) for s in shapes for g in GRANS),
                     dtype=torch.uint8, device="cuda")
    for it in range(2):
        for shape in shapes:
            for gran in (Q.PER_TENSOR, Q.PER_CHANNEL):
                x = (rng.standard_normal(shape) * (10.0 ** rng.integers(-3, 3))).astype(np.float32)
                q, s, a = hq.hq_quantize_fp8(dev_f32(x), fp8.E4M3, gran, workspace=ws)
                q_ref, s_ref, a_ref = Q.quantize_dynamic(x, Q.F32, fp8.E4M3, gran)
                assert np.array_equal(host(q), q_ref)
                assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))


def test_single_pass_barrier_state(hq):
    """Dynamic per-tensor calls of up to 2^24 bf16 elements run as one pass whose
    blocks agree on the amax through the workspace. After every call the arrival
    counters and the top counter are back at zero; the 64-bit barrier word holds
    the number of single-pass calls so far in its high half and the last such
    call's amax bits in its low half. A tensor one row too large for the single
    pass (two passes) and a delayed call in between leave the word alone. A
    single-pass per-channel call (bf16, at most 512 tiles of 128 rows x 256
    columns) advances the generation with an empty amax half; its column
    partials follow the per-tensor region."""
    rng = np.random.default_rng(23)
    ws = torch.zeros(hq.hq_quantize_workspace_bytes(Q.PER_CHANNEL, 4096, 4096), dtype=torch.uint8, device="cuda")
    arrivals = slice(4096, 8192)        # 1024 partial words, then 32 arrival lines
    word_lo, word_hi, top = 2048, 2049, 2048 + 32  # uint32 indices of the barrier lines
    gen, last_amax = 0, 0
    ring, st, flag = hq.Ring(4), Q.ring_new(4), 0
    steps = [(1, 16), (300, 1024), (4096, 4096), (4097, 4096), "delayed", (64, 2048), ("col", 4096, 4096),
             (4096, 4096), ("col", 300, 2048), (1, 16)]
    for t, sh in enumerate(steps):
        if sh[0] == "col":
            bits = workloads.random_bf16(rng, sh[1:], std=float(10.0 ** rng.integers(-2, 3)))
            q, s, a = hq.hq_quantize_fp8(dev_bf16(bits), fp8.E4M3, Q.PER_CHANNEL, workspace=ws)
            q_ref, s_ref, a_ref = Q.quantize_dynamic(bits, Q.BF16, fp8.E4M3, Q.PER_CHANNEL)
            assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32)), (t, sh)
            assert np.array_equal(host(a).view(np.uint32), a_ref.view(np.uint32)), (t, sh)
            gen, last_amax = gen + 1, 0
        elif sh == "delayed":
            bits = workloads.random_bf16(rng, (128, 256))
            q, _, _ = hq.hq_quantize_fp8(dev_bf16(bits), fp8.E4M3, Q.PER_TENSOR, ring=ring, ring_idx=0, workspace=ws)
            q_ref, _, _, st, flag = Q.quantize_delayed(bits, Q.BF16, fp8.E4M3, st, 0, 0, flag)
        else:
            bits = workloads.random_bf16(rng, sh, std=float(10.0 ** rng.integers(-2, 3)))
            q, s, a = hq.hq_quantize_fp8(dev_bf16(bits), fp8.E4M3, Q.PER_TENSOR, workspace=ws)
            q_ref, s_ref, a_ref = Q.quantize_dynamic(bits, Q.BF16, fp8.E4M3, Q.PER_TENSOR)
            assert host(s).view(np.uint32)[0] == s_ref.view(np.uint32)[0], (t, sh)
            assert host(a).view(np.uint32)[0] == a_ref.view(np.uint32)[0], (t, sh)
            if sh[0] * sh[1] <= 1 << 24:
                gen, last_amax = gen + 1, int(a_ref.view(np.uint32)[0])
        torch.cuda.synchronize()
        assert np.array_equal(host(q), q_ref), (t, sh)
        w = host(ws).view(np.uint32)
        assert not host(ws)[arrivals].any(), (t, sh)
        assert w[top] == 0, (t, sh)
        assert (int(w[word_hi]), int(w[word_lo])) == (gen, last_amax), (t, sh)


def test_single_pass_give_up_is_reported(hq):
    """A one-pass per-tensor or per-channel call whose blocks cannot all meet
    (forced from the host: the workspace filled with 0x40 bytes, so no arrival
    counter ever reaches its last member and no block releases the others)
    has every block give up its bounded wait (0.5 s) and exit: every scale it
    writes is NaN and the workspace's sticky status bit reports it. After a
    zero fill the same workspace serves a normal call again, status clear."""
    rng = np.random.default_rng(31)
    bits = workloads.random_bf16(rng, (1024, 2048))
    ws = torch.zeros(hq.hq_quantize_workspace_bytes(Q.PER_CHANNEL, 1024, 2048), dtype=torch.uint8, device="cuda")
    assert not hq.hq_quantize_workspace_status(ws)
    for gran in (Q.PER_TENSOR, Q.PER_CHANNEL):
        ws.fill_(0x40)
        assert not hq.hq_quantize_workspace_status(ws)  # bit 0 of 0x40404040 is clear
        _, s, _ = hq.hq_quantize_fp8(dev_bf16(bits), fp8.E4M3, gran, workspace=ws)
        torch.cuda.synchronize()
        assert np.all(np.isnan(host(s))), gran
        assert hq.hq_quantize_workspace_status(ws), gran
        ws.zero_()
        q, s, a = hq.hq_quantize_fp8(dev_bf16(bits), fp8.E4M3, gran, workspace=ws)
        q_ref, s_ref, a_ref = Q.quantize_dynamic(bits, Q.BF16, fp8.E4M3, gran)
        assert np.array_equal(host(q), q_ref)
        assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
        assert not hq.hq_quantize_workspace_status(ws)


# ---- delayed scaling ---------------------------------------------------------------

def test_delayed_shared_workspace_varying_grids(hq):
    """Delayed calls whose grids have 1, a few, hundreds and the maximum number
    of blocks share one zero-filled workspace: each call's codes and ring match
    the oracle, and the arrival counters are back at zero after every call."""
    rng = np.random.default_rng(11)
    shapes = [(1, 16), (8, 2048), (300, 1024), (2048, 4096), (64, 64)]
    ws = torch.zeros(hq.hq_quantize_workspace_bytes(Q.PER_TENSOR, 1, 16), dtype=torch.uint8, device="cuda")
    rings = {sh: (hq.Ring(4), Q.ring_new(4)) for sh in shapes}
    flags = {sh: 0 for sh in shapes}
    for t in range(3):
        for sh in shapes:
            ring, st = rings[sh]
            bits = workloads.random_bf16(rng, sh, std=float(10.0 ** rng.integers(-2, 2)))
            q, s, a = hq.hq_quantize_fp8(dev_bf16(bits), fp8.E4M3, Q.PER_TENSOR, ring=ring, ring_idx=t % 4,
                                         workspace=ws)
            q_ref, s_ref, a_ref, st, flags[sh] = Q.quantize_delayed(bits, Q.BF16, fp8.E4M3, st, t % 4, 0, flags[sh])
            rings[sh] = (ring, st)
            torch.cuda.synchronize()
            assert np.array_equal(host(q), q_ref), (t, sh)
            assert np.array_equal(host(ring.state).view(np.uint32), st.view(np.uint32)), (t, sh)
            counters = host(ws)[4096:].view(np.uint32)
            assert not counters.any(), (t, sh, np.nonzero(counters))


def _ring_host(r):
    return host(r.state).copy(), int(host(r.flag)[0])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", [Q.BF16, Q.F32])
def test_delayed_ring_sequence(hq, fmt, dtype):
    """20 steps (wraps a 16-entry ring) with a moving amax, a NaN step and an
    all-zero step; codes, used scale, amax and the whole ring state must match
    the oracle after every step."""
    rng = np.random.default_rng(17 + fmt + 2 * dtype)
    ring = hq.Ring(16, margin=1 if fmt == fp8.E4M3 else 0)
    st = Q.ring_new(16)
    flag = 0
    shape = (96, 320)
    for t in range(20):
        x = (rng.standard_normal(shape) * np.exp(rng.standard_normal() * 2)).astype(np.float32)
        if t == 7:
            x[5, 5] = np.nan
        if t == 9:
            x[:] = 0.0
        xin = workloads.to_bf16_bits(x) if dtype == Q.BF16 else x
        xd = dev_bf16(xin) if dtype == Q.BF16 else dev_f32(xin)
        q, s, a = hq.hq_quantize_fp8(xd, fmt, Q.PER_TENSOR, ring=ring, ring_idx=t % 16)
        q_ref, s_ref, a_ref, st, flag = Q.quantize_delayed(xin, dtype, fmt, st, t % 16, ring.margin, flag)
        torch.cuda.synchronize()
        assert np.array_equal(host(q), q_ref), f"codes differ at step {t}"
        assert host(s).view(np.uint32)[0] == s_ref.view(np.uint32)[0], f"scale differs at step {t}"
        assert host(a).view(np.uint32)[0] == a_ref.view(np.uint32)[0], f"amax differs at step {t}"
        gst, gflag = _ring_host(ring)
        assert np.array_equal(gst.view(np.uint32), st.view(np.uint32)), f"ring differs at step {t}"
        assert gflag == flag


def test_delayed_large_tensor_many_blocks(hq):
    """A tensor large enough for the maximum number of partial blocks; the
    last-block election must see every block's amax."""
    x, w = workloads.ptpc_square(1, m=2048, n=64, k=4096)
    ring = hq.Ring(16)
    st = Q.ring_new(16)
    flag = 0
    for t in range(3):
        q, s, a = hq.hq_quantize_fp8(dev_bf16(x), fp8.E4M3, Q.PER_TENSOR, ring=ring, ring_idx=t)
        q_ref, s_ref, a_ref, st, flag = Q.quantize_delayed(x, Q.BF16, fp8.E4M3, st, t, 0, flag)
        torch.cuda.synchronize()
        assert np.array_equal(host(q), q_ref)
        assert np.array_equal(host(ring.state).view(np.uint32), st.view(np.uint32))


def test_ring_update_entry_point(hq):
    ring = hq.Ring(4, margin=-1)
    st = Q.ring_new(4)
    flag = 0
    samples = [3.0, 0.5, np.inf, 7.0, 0.0, 1e-30, np.nan, 2.5, 9.0]
    for t, smp in enumerate(samples):
        amax = torch.tensor([smp], dtype=torch.float32, device="cuda")
        hq.hq_scale_ring_update(ring, amax, fp8.E5M2, ring_idx=t % 4)
        st, flag = Q.ring_update(st, t % 4, -1, np.float32(smp), False, fp8.E5M2, flag)
        torch.cuda.synchronize()
        assert np.array_equal(host(ring.state).view(np.uint32), st.view(np.uint32)), t
        assert int(host(ring.flag)[0]) == flag


def test_training_linear_rings(hq):
    """Two layers of the training workload for 20 steps: forward E4M3 X and W
    rings, backward E5M2 G ring (16 entries, margin 0)."""
    base, factors = workloads.training_linear(4, layers=2, steps=20)
    for layer in range(2):
        rings = [hq.Ring(16) for _ in range(3)]
        sts = [Q.ring_new(16) for _ in range(3)]
        flags = [0, 0, 0]
        fmts = [fp8.E4M3, fp8.E4M3, fp8.E5M2]
        for t in range(20):
            tensors = workloads.training_step_inputs(base, factors, t, layer)
            for i, (bits, fmt) in enumerate(zip(tensors, fmts)):
                q, s, a = hq.hq_quantize_fp8(dev_bf16(bits), fmt, Q.PER_TENSOR, ring=rings[i], ring_idx=t % 16)
                q_ref, s_ref, a_ref, sts[i], flags[i] = Q.quantize_delayed(bits, Q.BF16, fmt, sts[i], t % 16, 0,
                                                                          flags[i])
                torch.cuda.synchronize()
                assert np.array_equal(host(q), q_ref), (layer, t, i)
                assert np.array_equal(host(rings[i].state).view(np.uint32), sts[i].view(np.uint32)), (layer, t, i)


def test_invalid_arguments_leave_outputs_untouched(hq):
    x = torch.randn(8, 48, device="cuda")
    q = torch.full((8, 48), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((8,), -1.0, device="cuda")
    with pytest.raises(ValueError):
        hq.hq_quantize_fp8(x, 7, Q.PER_TOKEN, q=q, scale_out=s)
    with pytest.raises(ValueError):
        hq.hq_quantize_fp8(x[:, :40], fp8.E4M3, Q.PER_TOKEN, q=q[:, :40], scale_out=s)
    torch.cuda.synchronize()
    assert bool((q == 0xAB).all()) and bool((s == -1.0).all())


# ---- scaled values one float32 ulp above fmax ------------------------------------

def _ulp_above_fmax_amaxes(fmt, dtype):
    """Every positive normal amax a of the input type whose scaled value
    fl32(a * fl32(1 / max(fl32(a / fmax), 2^-126))) lies above fmax (one float32
    ulp above, at most). Found by enumerating the type's values (bf16: all of
    them; float32: one in 2^7 of the mantissas, all exponents)."""
    if dtype == Q.BF16:
        bits = (np.arange(0x0080, 0x7F80, dtype=np.uint32) << np.uint32(16))
    else:
        bits = np.arange(0x00800000, 0x7F800000, 128, dtype=np.uint32)
    a = bits.view(np.float32)
    fmax = np.float32(fp8.fmax(fmt))
    s = np.maximum((a / fmax).astype(np.float32), np.float32(2.0 ** -126))
    r = (np.float32(1.0) / s).astype(np.float32)
    v = (a * r).astype(np.float32)
    assert np.all(v <= np.nextafter(fmax, np.float32(np.inf)))
    return a[v > fmax]


def _rows_with_amax(rng, amax, cols):
    """One row per amax: +-amax planted at a random column (and its negation in
    another), the other entries amax times factors in (-1, 1) rounded towards
    zero to bf16, so the row's amax is the planted value."""
    n = len(amax)
    x = (amax[:, None] * rng.uniform(-1.0, 1.0, (n, cols))).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    c = rng.integers(0, cols, n)
    x[np.arange(n), c] = amax * np.where(rng.random(n) < 0.5, 1, -1).astype(np.float32)
    x[np.arange(n), (c + 1 + rng.integers(0, cols - 1, n)) % cols] = -x[np.arange(n), c]
    return x


@pytest.mark.parametrize("dtype", [Q.BF16, Q.F32])
@pytest.mark.parametrize("fmt", FMTS)
def test_scaled_value_one_ulp_above_fmax(hq, fmt, dtype):
    """With dynamic scales every finite element has |x| <= amax, and the kernels
    cast such vectors without the clamp to +-fmax: the largest scaled value,
    fl32(amax * r), can sit one float32 ulp above fmax, and the conversion's own
    nearest-even rounding must give the fmax code there. Every group here has
    such an amax (all of them for bf16, a sample for float32): per token, per
    channel (the transpose), per tensor, per row into the pre-shuffled layout
    and block-wise, each checked byte for byte against the oracle."""
    from oracle import blockwise as B
    from oracle import preshuffle as P
    rng = np.random.default_rng(17 + fmt + 2 * dtype)
    amax = _ulp_above_fmax_amaxes(fmt, dtype)
    assert len(amax) > 1000
    if len(amax) > 8192:
        amax = rng.choice(amax, 8192, replace=False)
    x = _rows_with_amax(rng, amax, 64)
    x_in = workloads.to_bf16_bits(x) if dtype == Q.BF16 else x
    if dtype == Q.BF16:
        assert np.array_equal(workloads.to_bf16_bits(x), (x.view(np.uint32) >> 16).astype(np.uint16))
    _assert_same(hq, x_in, dtype, fmt, Q.PER_TOKEN, "per token, amax*r above fmax")
    _assert_same(hq, np.ascontiguousarray(x_in[:1024].T), dtype, fmt, Q.PER_CHANNEL, "per channel")
    for i in rng.choice(len(amax), 8, replace=False):
        t = _rows_with_amax(rng, np.full(32, amax[i], np.float32), 64)
        _assert_same(hq, workloads.to_bf16_bits(t) if dtype == Q.BF16 else t, dtype, fmt, Q.PER_TENSOR,
                     "per tensor")
    xd = dev_bf16(x_in) if dtype == Q.BF16 else dev_f32(x_in)
    q_pre, s, _, q = hq.hq_quantize_fp8_preshuffled(xd, fmt, row_major=True)
    got = hq.hq_quantize_fp8_blockwise(xd, fmt, 64)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = Q.quantize_dynamic(x_in, dtype, fmt, Q.PER_TOKEN)
    assert np.array_equal(host(q), q_ref) and np.array_equal(host(q_pre), P.preshuffle(q_ref))
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    bq, bs, _ = B.quantize_blockwise(x_in, dtype, fmt, 64)
    assert np.array_equal(host(got[0]), bq) and np.array_equal(host(got[1]).view(np.uint32), bs.view(np.uint32))
