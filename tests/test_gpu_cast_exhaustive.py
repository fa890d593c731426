"""The device FP8 cast against the oracle's encoder on every float32 pattern of
the binades that decide it (hip-quant README, "FP8 Formats (both APIs)":
saturating round-to-nearest-even to OCP E4M3 / E5M2).

The kernels cast fl32(x * r) with a v_med3 clamp to +-fmax, the hardware
v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 and a NaN patch; with a given scale of 1
(hq_quantize_fp8_layouts, r = fl32(1/1) = 1) the value cast is x itself, so a
float32 input tensor holding chosen bit patterns puts each pattern through the
cast exactly. Covered, both signs, every mantissa:
  * biased exponents 107 .. 144 (2^-20 up to 2^18): every value either format
    can round to a non-zero code, every tie, every value near the saturation
    thresholds (448 + 16 for E4M3, 57344 + 4096 for E5M2) and above them;
  * biased exponent 0 (zero and the float32 subnormals) and 255 (Inf and every
    NaN pattern).
Every other binade lies wholly below 2^-20 (rounds to a signed zero in both
formats) or wholly above 2^18 (saturates); those are checked on 2^16 sampled
mantissas each.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

from oracle import fp8
from tests.gpu_helpers import host, require_gpu

pytestmark = pytest.mark.gpu

FULL = [0] + list(range(127 - 20, 127 + 18)) + [255]
SAMPLED = [e for e in range(256) if e not in FULL]
COLS = 4096
PER_CLASS = 1 << 24  # 2^23 mantissas, both signs


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _patterns_host(e, mant):
    pos = (np.uint32(e) << np.uint32(23)) | mant.astype(np.uint32)
    return np.concatenate([pos, pos | np.uint32(0x80000000)])


def _oracle(e, fmt):
    return fp8.encode(_patterns_host(e, np.arange(1 << 23, dtype=np.uint32)).view(np.float32), fmt)


def _device_codes(hq, bits_dev, fmt):
    x = bits_dev.view(torch.float32).view(-1, COLS)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    out = hq.hq_quantize_fp8_layouts(x, fmt, scale_in=one, q=True)
    return out["q"].view(-1)


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_cast_every_pattern_of_the_deciding_binades(hq, fmt):
    mant = torch.arange(1 << 23, dtype=torch.int32, device="cuda")
    classes = []
    for e in FULL:
        pos = mant | (e << 23)
        classes += [pos, pos | torch.tensor(-2 ** 31, dtype=torch.int32, device="cuda")]
    bits = torch.cat(classes)
    del classes
    codes = host(_device_codes(hq, bits, fmt)).reshape(len(FULL), PER_CLASS)
    del bits
    torch.cuda.synchronize()
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        futures = {e: ex.submit(_oracle, e, fmt) for e in FULL}
        for i, e in enumerate(FULL):
            want = futures[e].result()
            bad = np.nonzero(codes[i] != want)[0]
            if bad.size:
                b = int(bad[0])
                pattern = (e << 23) | (b % (1 << 23)) | ((b >> 23) << 31)
                raise AssertionError(f"exponent {e}: {bad.size} patterns differ; first {pattern:#010x}: "
                                     f"got {codes[i][b]:#04x} want {want[b]:#04x}")


@pytest.mark.parametrize("fmt", [fp8.E4M3, fp8.E5M2])
def test_cast_sampled_outer_binades(hq, fmt):
    rng = np.random.default_rng(1234 + fmt)
    host_bits = np.concatenate([_patterns_host(e, rng.integers(0, 1 << 23, 1 << 15)) for e in SAMPLED])
    want = fp8.encode(host_bits.view(np.float32), fmt)
    pad = (-len(host_bits)) % COLS
    dev = torch.from_numpy(np.concatenate([host_bits, np.zeros(pad, np.uint32)]).view(np.int32)).cuda()
    got = host(_device_codes(hq, dev, fmt))[:len(host_bits)]
    # below 2^-20 every value is a signed zero, above 2^18 every value saturates
    assert np.array_equal(got, want)
    small = (host_bits >> 23 & 0xFF) < 107
    assert np.all((got[small] & 0x7F) == 0)
    assert np.all((got[~small] & 0x7F) == fp8.max_code(fmt))
