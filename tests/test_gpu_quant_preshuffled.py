"""GPU parity of hq_quantize_fp8_preshuffled: per-row dynamic quantization of a
weight [n, k] written straight into the GEMM's pre-shuffled layout. q_pre must
equal, byte for byte, the oracle's pre-shuffle index map applied to the
oracle's per-row codes (zero padding included); scales and amax must equal the
oracle's per-row ones bit for bit, and the optional row-major codes the
oracle's codes."""
import numpy as np
import pytest
import torch

import workloads
from oracle import fp8, preshuffle as P, quantize as Q
from tests.gpu_helpers import dev_bf16, dev_f32, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _input(rng, shape, dtype, specials):
    """Random rows of varied magnitude; with `specials`, a row with NaN / Inf,
    an all-zero row and a row whose only finite values are tiny."""
    rows, cols = shape
    x = rng.standard_normal(shape).astype(np.float32) * (10.0 ** rng.integers(-3, 4, (rows, 1))).astype(np.float32)
    if specials and rows >= 4:
        x[0, rng.integers(0, cols, 3)] = [np.nan, np.inf, -np.inf]
        x[1] = 0.0
        x[2] = np.float32(1e-30)
        x[2, 0] = np.inf
        x[3, cols - 1] = 1e4  # an outlier in the last column
    if dtype == Q.BF16:
        bits = workloads.to_bf16_bits(x)
        return bits, dev_bf16(bits)
    return x, dev_f32(x)


# (rows, cols): single row; N not a multiple of 32 and K not of 128 (padding in
# both); one-vector-per-lane rows; ragged K; rows longer than the register path
# (bf16 K > 4096, fp32 K > 2048: read twice); 16-row groups over several CUs
SHAPES = [(1, 16), (33, 144), (64, 512), (100, 272), (40, 4112), (70, 2064), (520, 1024)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
@pytest.mark.parametrize("dtype", [Q.BF16, Q.F32])
def test_preshuffled_per_row_equals_oracle(hq, shape, fmt, dtype):
    rng = np.random.default_rng(shape[0] * 131 + shape[1] + 7 * fmt + dtype)
    x, xd = _input(rng, shape, dtype, specials=True)
    q_pre, s, a, q = hq.hq_quantize_fp8_preshuffled(xd, fmt, row_major=True)
    torch.cuda.synchronize()
    q_ref, s_ref, a_ref = Q.quantize_dynamic(x, dtype, fmt, Q.PER_TOKEN)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)
    pre = host(q_pre)
    assert pre.size == P.preshuffled_bytes(*shape)
    assert np.array_equal(pre, P.preshuffle(q_ref))


def test_padding_overwritten_and_row_major_optional(hq):
    """Without row-major output only q_pre, scales and amax are written, and
    the padding bytes are written as zeros over whatever the buffer held."""
    rng = np.random.default_rng(11)
    shape = (45, 208)
    x, xd = _input(rng, shape, Q.BF16, specials=False)
    q_pre = torch.full((P.preshuffled_bytes(*shape),), 0xA5, dtype=torch.uint8, device="cuda")
    _, s, a, q = hq.hq_quantize_fp8_preshuffled(xd, fp8.E4M3, q_pre=q_pre)
    torch.cuda.synchronize()
    assert q is None
    q_ref, s_ref, _ = Q.quantize_dynamic(x, Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    assert np.array_equal(host(q_pre), P.preshuffle(q_ref))
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))


def test_weight_4096_equals_oracle(hq):
    """The PTPC weight, bf16 [4096, 4096] N(0, 0.02^2), in the launch
    configuration the step uses (256 workgroups of 16 rows)."""
    _, w_bits = workloads.ptpc_square(1)
    q_pre, s, a, _ = hq.hq_quantize_fp8_preshuffled(dev_bf16(w_bits), fp8.E4M3)
    torch.cuda.synchronize()
    q_ref, s_ref, a_ref = Q.quantize_dynamic(w_bits, Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(a).view(np.uint32), a_ref.view(np.uint32))
    assert np.array_equal(host(q_pre), P.preshuffle(q_ref))


def test_same_bytes_as_per_token_then_preshuffle(hq):
    """The fused entry point and the two-launch path (hq_quantize_fp8 per token,
    then hq_preshuffle_weight) give the same bytes."""
    rng = np.random.default_rng(12)
    x, xd = _input(rng, (300, 1040), Q.BF16, specials=True)
    q_pre, s, _, _ = hq.hq_quantize_fp8_preshuffled(xd, fp8.E5M2)
    q2, s2, _ = hq.hq_quantize_fp8(xd, fp8.E5M2, Q.PER_TOKEN)
    pre2 = hq.hq_preshuffle_weight(q2)
    torch.cuda.synchronize()
    assert torch.equal(q_pre, pre2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
