// Row-streaming probe: the memory traffic of the per-token quantize without its
// arithmetic. Each wavefront reads whole 16-bit rows with 16-byte loads and
// writes one byte per element (the high byte of each 16-bit word, so the
// output depends on every load), walking rows w, w + W, ... with the next
// row's loads issued before the current row's stores, at a grid the caller
// chooses. Timed at the quantize's own grid it is the HBM ceiling for a pass
// of that size and shape: the same bytes, the same access order, no amax
// reduction, no scale and no conversion.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

namespace {

constexpr int kProbeWavesPerBlock = 4;

template <int NV>
__global__ __launch_bounds__(64 * kProbeWavesPerBlock) void stream_rows_probe_kernel(
    const uint4* __restrict__ x, uint8_t* __restrict__ q, int64_t rows, int vpr) {
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * kProbeWavesPerBlock;
  int64_t row = (int64_t)blockIdx.x * kProbeWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint4 cur[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) cur[j] = x[(size_t)row * vpr + min(lane + 64 * j, vpr - 1)];
  for (; row < rows; row += W) {
    const int64_t nrow = row + W;
    uint4 nxt[NV];
    if (nrow < rows) {
#pragma unroll
      for (int j = 0; j < NV; ++j) nxt[j] = x[(size_t)nrow * vpr + min(lane + 64 * j, vpr - 1)];
    }
    uint8_t* qr = q + (size_t)row * vpr * 8;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = lane + 64 * j;
      if (i < vpr) {
        // bytes 1 and 3 of each 32-bit word: the high byte of each 16-bit element
        const uint32_t w[2] = {__builtin_amdgcn_perm(cur[j].y, cur[j].x, 0x07050301u),
                               __builtin_amdgcn_perm(cur[j].w, cur[j].z, 0x07050301u)};
        store_codes<8>(qr + (size_t)i * 8, w);
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) cur[j] = nxt[j];
  }
}

}  // namespace

hipError_t launch_stream_rows_probe(const void* x, int64_t rows, int row_vecs, int waves, uint8_t* q,
                                    hipStream_t st) {
  const uint4* xv = static_cast<const uint4*>(x);
  const int blocks = (int)std::min<int64_t>((rows + kProbeWavesPerBlock - 1) / kProbeWavesPerBlock,
                                            (waves + kProbeWavesPerBlock - 1) / kProbeWavesPerBlock);
  const dim3 grid(blocks), block(64 * kProbeWavesPerBlock);
  if (row_vecs <= 64) {
    hipLaunchKernelGGL(stream_rows_probe_kernel<1>, grid, block, 0, st, xv, q, rows, row_vecs);
  } else if (row_vecs <= 128) {
    hipLaunchKernelGGL(stream_rows_probe_kernel<2>, grid, block, 0, st, xv, q, rows, row_vecs);
  } else if (row_vecs <= 256) {
    hipLaunchKernelGGL(stream_rows_probe_kernel<4>, grid, block, 0, st, xv, q, rows, row_vecs);
  } else {
    hipLaunchKernelGGL(stream_rows_probe_kernel<8>, grid, block, 0, st, xv, q, rows, row_vecs);
  }
  return hipGetLastError();
}

}  // namespace hq
