"""CPU oracle for dynamic FP8 quantization and the scaled FP8 (a8w8) GEMM.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link or
execute anything in this package: only the tests, the smoke check and the CPU
baseline leg of the benchmark use it. The GPU library shares no code, header,
table or helper with it; the two meet only in the seeded input generators of
the ``workloads`` package, which hold none of the method's arithmetic.

The oracle is deliberately plain and slow: numpy in float64 where the method
leaves the precision open, and float32 exactly where the method fixes a float32
step (the scale division, the reciprocal, the pre-cast product), so that a
quantised code is decided in the same precision on both sides.

Modules
  fp8         OCP E4M3 / E5M2 decode tables and the saturating RNE encoder
  quantize    amax, scale and codes at per-tensor / per-token / per-channel
              granularity; delayed scaling with the amax-history ring
  gemm        the scaled a8w8 GEMM and its grouped (per-expert) variant in
              float64, plus the comparison tolerance
  preshuffle  the byte map of the pre-shuffled weight layout
  stochastic  Philox-4x32-10 and the stochastic E5M2 rounding rule
  blockwise   block-wise scaling and the block-scaled GEMM, with its tolerance

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (closed forms, library cross-checks, brute force and
invariants); the block-scaled GEMM tolerance by ``tests/test_mfma_model.py``
(the fold's float32 rounding accepted, a dropped term rejected). The pre-shuffled byte map is a layout of this library's own design
(the pages leave the layout open); it is pinned by its bijectivity, by
hand-derived byte positions written out in ``tests/test_oracle_preshuffle.py``
and, end to end, by the GEMM on pre-shuffled weights matching the plain oracle
GEMM.
"""

from . import fp8, quantize, gemm, preshuffle  # noqa: F401
