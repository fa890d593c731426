"""GPU check of hq_stream_rows_probe, the row-streaming measurement aid that
bench.py times beside the per-token quantize: every output byte is the high
byte of its 16-bit input element, for full, ragged and single-vector rows and
for grids smaller and larger than the row count."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


@pytest.mark.parametrize("rows,cols,waves", [
    (4096, 4096, 3072),    # the per-token quantize's workload and grid
    (4096, 4096, 1024),
    (1000, 4000, 3072),    # ragged row: 500 vectors, not a multiple of 64
    (37, 8, 5),            # one vector per row, more rows than wavefronts
    (3, 4096, 3072),       # fewer rows than wavefronts
    (9, 520, 2),           # ragged, two wavefronts walking 9 rows
])
def test_probe_writes_the_high_byte_of_every_element(hq, rows, cols, waves):
    rng = np.random.default_rng(rows * 7919 + cols)
    bits = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).cuda()
    out = torch.full((rows, cols), 0x5A, dtype=torch.uint8, device="cuda")
    hq.hq_stream_rows_probe(x, waves, out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), (bits >> 8).astype(np.uint8))
