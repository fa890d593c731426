"""hq_gemm_a8w8_noalloc (the GEMM for callers that cannot allocate) against
hq_gemm_a8w8 with a caller workspace: the same output bits on two calls in a
row, the second with a smaller input, in the split decode plan that uses the
library's scratch, and on a shape that needs none."""
import numpy as np
import pytest
import torch

from oracle import fp8
from tests.gpu_helpers import dev_f32, dev_u8, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _operands(hq, rng, m, n, k):
    t = fp8.decode_table(fp8.E4M3)
    finite = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    xq = dev_u8(rng.choice(finite, size=(m, k)))
    pre = hq.hq_preshuffle_weight(dev_u8(rng.choice(finite, size=(n, k))))
    xs = dev_f32(rng.uniform(1e-3, 1e-2, m))
    ws = dev_f32(rng.uniform(1e-3, 1e-2, n))
    return xq, pre, xs, ws


def _compare(hq, rng, m, n, k):
    xq, pre, xs, ws = _operands(hq, rng, m, n, k)
    need = hq.hq_gemm_workspace_bytes(m, n, k)
    work = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    want = host(hq.hq_gemm_a8w8(xq, fp8.E4M3, pre, fp8.E4M3, xs, ws, n, workspace=work))
    sentinel = 0x7FC1
    out = torch.full((m, n), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    hq.hq_gemm_a8w8_noalloc(xq, fp8.E4M3, pre, fp8.E4M3, xs, ws, n, out)
    got = host(out)
    assert np.array_equal(got, want), (m, n, k)
    return need


def test_noalloc_matches_workspace_gemm_two_calls(hq):
    rng = np.random.default_rng(7)
    # a split decode plan (m <= 16, 128 half-fragment groups, 9216 > 64 blocks
    # of 128): the library scratch is used
    assert _compare(hq, rng, 16, 1024, 9216) > 0
    # a smaller input, split too, with fewer column groups: its partial sums sit
    # where the first call's did
    assert _compare(hq, rng, 1, 512, 8448) > 0


def test_noalloc_without_split_and_tiled(hq):
    rng = np.random.default_rng(8)
    assert _compare(hq, rng, 8, 1024, 2048) == 0    # decode shape, no split
    assert _compare(hq, rng, 200, 384, 640) == 0    # tiled shape
    assert _compare(hq, rng, 32, 2048, 7168) > 0    # two row blocks, split again after the others
