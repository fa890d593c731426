// Dynamic and delayed FP8 quantization kernels for gfx950.
//
// What is computed (the method statement; hip-quant README "Scale / amax
// tracking" and "Training-path numerical guards"; fuel-ir quant_scale.rs for the
// granularities): per group, amax = max |x| over finite x, s = max(amax/fmax,
// 2^-126), r = 1/s, q = saturating RNE cast of fl32(x*r).
//
// Kernels (all read the input once from HBM with 16-byte vector loads):
//   quant_rows_wave  one wavefront per row ("per token", rows up to 512
//                    vectors): the row is held in registers between the amax
//                    reduction (wavefront shuffles) and the cast
//   quant_rows       one workgroup per row for longer rows, same scheme
//   amax_partials +  per tensor: block partial maxima, then every block folds
//   quant_tensor     the partials and casts its share (two launches)
//   colmax_partials  per column ("per channel"): 256-column x 128-row tiles write
//   + quant_cols     column partial maxima, then the cast pass folds them
//   quant_delayed    per tensor with the scale taken from an amax-history ring;
//                    a last-block epilogue folds the amax into the ring and
//                    publishes the next scale (AstrAI ops.cu, commit "finalize fp8
//                    scale rings inside quantize kernels": threadfence + counter
//                    election, no extra launch)
//   ring_update      the same ring fold as a one-thread launch
//
// Partial maxima are stored as float32 magnitude bits in bits 0..30 with bit 31
// set when the block saw a non-finite element.
#include <atomic>

#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;  // vectors in flight per thread in the grid-stride kernels
constexpr int kPartialUnroll = 8;  // in the per-tensor partial-max pass
constexpr uint32_t kNonfiniteBit = 0x80000000u;

// ---------------------------------------------------------------------------
// per row
// ---------------------------------------------------------------------------

// NV > 0: each thread keeps up to NV vectors of the row in registers.
// NV == 0: the row is streamed twice (first pass for amax, second for the cast).
template <int XT, int FMT, int NV, int BLOCK, bool SR>
__global__ __launch_bounds__(BLOCK) void quant_rows_kernel(
    const uint4* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ scale,
    float* __restrict__ amax_out, int vpr, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  __shared__ uint32_t red[BLOCK / 64];
  const size_t row = blockIdx.x;
  const uint4* xr = x + row * (size_t)vpr;
  uint8_t* qr = q + row * (size_t)vpr * E;

  uint4 v[NV > 0 ? NV : 1];
  uint32_t raw[NV > 0 ? NV : 1];
  uint32_t mx = 0;
  if (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = threadIdx.x + j * BLOCK;
      raw[j] = 0;
      if (i < vpr) {
        v[j] = xr[i];
        raw[j] = vec_absmax_raw<XT>(v[j]);
      }
      mx = max(mx, raw[j]);
    }
  } else {
    for (int i = threadIdx.x; i < vpr; i += BLOCK) mx = max(mx, vec_absmax_raw<XT>(xr[i]));
  }
  mx = block_max_u32<BLOCK>(mx, red);
  if (mx >= kInfBits) {  // the row holds an Inf/NaN: recompute over finite elements
    uint32_t f = 0;
    if (NV > 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j)
        if (threadIdx.x + j * BLOCK < vpr) f = max(f, vec_absmax_finite<XT>(v[j]));
    } else {
      for (int i = threadIdx.x; i < vpr; i += BLOCK) f = max(f, vec_absmax_finite<XT>(xr[i]));
    }
    mx = block_max_u32<BLOCK>(f, red);
  }
  const float amax = __uint_as_float(mx);
  const float s = scale_from_amax<FMT>(amax);
  const float r = 1.0f / s;
  if (threadIdx.x == 0) {
    scale[row] = s;
    if (amax_out) amax_out[row] = amax;
  }
  if (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = threadIdx.x + j * BLOCK;
      if (i < vpr) {
        uint32_t w[E / 4];
        cast_vec<XT, FMT, SR, true>(v[j], r, raw[j], w, sd, (row * vpr + i) * E);
        store_codes<E>(qr + (size_t)i * E, w);
      }
    }
  } else {
    for (int i = threadIdx.x; i < vpr; i += BLOCK) {
      const uint4 vv = xr[i];
      uint32_t w[E / 4];
      cast_vec<XT, FMT, SR, true>(vv, r, vec_absmax_raw<XT>(vv), w, sd, (row * vpr + i) * E);
      store_codes<E>(qr + (size_t)i * E, w);
    }
  }
}

// One wavefront per row, for rows of up to 64*NV vectors: the amax is a
// wavefront shuffle reduction (no LDS round trip, no barrier). Each wavefront
// walks rows w, w + W, w + 2W, ... (W = wavefronts in the grid) and issues the
// loads of its next row before it reduces, casts and stores the current one, so
// code stores of one row overlap the input reads of the next.
constexpr int kRowsPerBlock = 4;
// Measured on 4096 x 4096 bf16: 9.6 us at 12 wavefronts per CU, 10.0 at 8 (two
// rows each, no tail) or 16, 11.6 at 4; non-temporal loads 10.0.
constexpr int kRowWavesPerCU = 12;

template <int XT, int FMT, int NV, bool SR>
__global__ __launch_bounds__(64 * kRowsPerBlock) void quant_rows_wave_kernel(
    const uint4* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ scale,
    float* __restrict__ amax_out, int rows, int vpr, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  const int lane = threadIdx.x & 63;
  // row indices step in 64 bits: rows up to 2^31 - 1 would overflow row + W
  const int64_t W = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wavefronts only
  // lanes past the row end reload the row's last vector (a real element, so it
  // cannot change the max) and skip the store
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
    uint32_t raw[NV];
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      raw[j] = vec_absmax_raw<XT>(cur[j]);
      mx = max(mx, raw[j]);
    }
    mx = wave_max_u32(mx);
    // a full row (every lane holds NV whole vectors) without Inf or NaN, scaled
    // by its own amax: no bounds check, no NaN patch and no clamp per vector
    // (bf16 [4096, 4096]: 9.335 -> 9.135 us in interleaved rounds on one box)
    const bool full_finite = !SR && mx < kInfBits && vpr == 64 * NV;  // wavefront-uniform
    if (mx >= kInfBits) {  // the row holds an Inf/NaN: recompute over finite elements
      uint32_t f = 0;
#pragma unroll
      for (int j = 0; j < NV; ++j) f = max(f, vec_absmax_finite<XT>(cur[j]));
      mx = wave_max_u32(f);
    }
    const float amax = __uint_as_float(mx);
    const float s = scale_from_amax<FMT>(amax);
    const float r = 1.0f / s;
    if (lane == 0) {
      scale[row] = s;
      if (amax_out) amax_out[row] = amax;
    }
    uint8_t* qr = q + (size_t)row * vpr * E;
    if (full_finite) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        uint32_t w[E / 4];
        vec_cast<XT, FMT, false>(cur[j], r, false, w);
        store_codes<E>(qr + (size_t)(lane + 64 * j) * E, w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int i = lane + 64 * j;
        if (i < vpr) {
          uint32_t w[E / 4];
          cast_vec<XT, FMT, SR, true>(cur[j], r, raw[j], w, sd, ((size_t)row * vpr + i) * E);
          store_codes<E>(qr + (size_t)i * E, w);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) cur[j] = nxt[j];
  }
}

template <int XT, int FMT, bool SR>
static hipError_t launch_rows_t(const void* x, int rows, int vpr, uint8_t* q, float* scale,
                                float* amax, SrSeed sd, hipStream_t st) {
  const uint4* xv = static_cast<const uint4*>(x);
  const dim3 grid(rows);
  const int wblocks = (int)std::min<int64_t>(((int64_t)rows + kRowsPerBlock - 1) / kRowsPerBlock,
                                             kNumCUs * kRowWavesPerCU / kRowsPerBlock);
  const dim3 wgrid(wblocks), wblock(64 * kRowsPerBlock);
  if (vpr <= 64) {
    hipLaunchKernelGGL((quant_rows_wave_kernel<XT, FMT, 1, SR>), wgrid, wblock, 0, st, xv, q, scale, amax, rows, vpr, sd);
  } else if (vpr <= 128) {
    hipLaunchKernelGGL((quant_rows_wave_kernel<XT, FMT, 2, SR>), wgrid, wblock, 0, st, xv, q, scale, amax, rows, vpr, sd);
  } else if (vpr <= 256) {
    hipLaunchKernelGGL((quant_rows_wave_kernel<XT, FMT, 4, SR>), wgrid, wblock, 0, st, xv, q, scale, amax, rows, vpr, sd);
  } else if (vpr <= 512) {
    hipLaunchKernelGGL((quant_rows_wave_kernel<XT, FMT, 8, SR>), wgrid, wblock, 0, st, xv, q, scale, amax, rows, vpr, sd);
  } else if (vpr <= 1024) {
    hipLaunchKernelGGL((quant_rows_kernel<XT, FMT, 4, kBlock, SR>), grid, dim3(kBlock), 0, st, xv, q, scale, amax, vpr, sd);
  } else if (vpr <= 2048) {
    hipLaunchKernelGGL((quant_rows_kernel<XT, FMT, 8, kBlock, SR>), grid, dim3(kBlock), 0, st, xv, q, scale, amax, vpr, sd);
  } else {
    hipLaunchKernelGGL((quant_rows_kernel<XT, FMT, 0, kBlock, SR>), grid, dim3(kBlock), 0, st, xv, q, scale, amax, vpr, sd);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// per tensor (dynamic): partial maxima, then fold + cast
// ---------------------------------------------------------------------------

template <int XT>
__global__ __launch_bounds__(kBlock) void amax_partials_kernel(const uint4* __restrict__ x, size_t nvec,
                                                               uint32_t* __restrict__ partial) {
  constexpr int U = kPartialUnroll;
  __shared__ uint32_t red[kBlock / 64];
  uint32_t raw = 0, fin = 0;
  const size_t stride = (size_t)gridDim.x * kBlock * U;
  for (size_t base = blockIdx.x * (size_t)kBlock * U + threadIdx.x; base < nvec; base += stride) {
    uint4 v[U];
    uint32_t m[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + u * kBlock < nvec) v[u] = x[base + u * kBlock];
    uint32_t mm = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m[u] = base + u * kBlock < nvec ? vec_absmax_raw<XT>(v[u]) : 0u;
      mm = max(mm, m[u]);
    }
    raw = max(raw, mm);
    if (__any(mm >= kInfBits)) {  // rare: filter the non-finite elements out
#pragma unroll
      for (int u = 0; u < U; ++u)
        fin = max(fin, m[u] < kInfBits ? m[u] : vec_absmax_finite<XT>(v[u]));
    } else {
      fin = max(fin, mm);
    }
  }
  const uint32_t braw = block_max_u32<kBlock>(raw, red);
  const uint32_t bfin = block_max_u32<kBlock>(fin, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = bfin | (braw >= kInfBits ? kNonfiniteBit : 0u);
}

// Fold `n` partials (every thread gets the finite amax bits and the flag).
__device__ __forceinline__ uint32_t fold_partials(const uint32_t* __restrict__ partial, int n, uint32_t* red,
                                                  bool* nonfinite) {
  uint32_t m = 0, f = 0;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const uint32_t p = partial[i];
    m = max(m, p & ~kNonfiniteBit);
    f |= p & kNonfiniteBit;
  }
  m = block_max_u32<kBlock>(m, red);
  f = block_max_u32<kBlock>(f, red);
  *nonfinite = f != 0;
  return m;
}

template <int XT, int FMT, bool SR>
__global__ __launch_bounds__(kBlock) void quant_tensor_kernel(const uint4* __restrict__ x, size_t nvec,
                                                              const uint32_t* __restrict__ partial, int npart,
                                                              uint8_t* __restrict__ q, float* __restrict__ scale,
                                                              float* __restrict__ amax_out, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  __shared__ uint32_t red[kBlock / 64];
  bool nonfinite;
  const float amax = __uint_as_float(fold_partials(partial, npart, red, &nonfinite));
  const float s = scale_from_amax<FMT>(amax);
  const float r = 1.0f / s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    scale[0] = s;
    if (amax_out) amax_out[0] = amax;
  }
  const size_t stride = (size_t)gridDim.x * kBlock * kUnroll;
  for (size_t base = blockIdx.x * (size_t)kBlock * kUnroll + threadIdx.x; base < nvec; base += stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (base + u * kBlock < nvec) v[u] = x[base + u * kBlock];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + u * kBlock;
      if (i < nvec) {
        uint32_t w[E / 4];
        if constexpr (SR) cast_vec<XT, FMT, true>(v[u], r, 0u, w, sd, i * E);
        else if (nonfinite) vec_cast<XT, FMT>(v[u], r, true, w);
        else vec_cast<XT, FMT, false>(v[u], r, false, w);
        store_codes<E>(q + i * E, w);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// per tensor (dynamic), single pass
// ---------------------------------------------------------------------------
// Every thread keeps its V vectors (i = global thread + k * threads) in
// registers while the grid agrees on the tensor amax, so X is read once. Each
// block publishes its maximum as its own partial word (a device-scope atomic
// store; one word per block, since atomics on one shared word serialise), waits
// for the store to complete, and counts in through the two-level arrival tree
// of the delayed path. The last arrival reduces the partials and publishes the
// tensor amax together with the next generation in one 64-bit word (generation
// in the high half, read by every block at its start); the other blocks poll
// that word, so one load both releases them and hands them the amax. Then every
// block casts its registers. The launcher only uses this kernel when the whole
// grid fits on the device at once (occupancy query), so every block is
// resident and the wait ends; as a guard the poll gives up after
// kBarrierSpinTicks of the 100 MHz real-time clock (a co-scheduled kernel
// holding CUs could keep blocks off the device). A block that gives up sets the
// workspace's sticky status bit (hq_quantize_workspace_status reports it) and
// writes a NaN scale; the block that writes the valid scale re-reads the bit
// after its write and overwrites the scale with NaN when it is set. Scale
// writes are device-scope atomic stores, so of two writes the later one in the
// coherence order stays: either the writer of the valid scale sees the bit, or
// the NaN write comes after it. NaN wins either way.
constexpr uint64_t kBarrierSpinTicks = 50000000;  // 0.5 s
constexpr int kFusedBlocks = 512;  // two per CU (measured: 12.8 us for bf16 [4096, 4096], 13.7 at 1024)

template <int XT, int FMT, bool SR, int V>
__global__ __launch_bounds__(kBlock) void quant_tensor_fused_kernel(const uint4* __restrict__ x, size_t nvec,
                                                                    uint8_t* __restrict__ q, float* __restrict__ scale,
                                                                    float* __restrict__ amax_out, uint32_t* partial,
                                                                    uint32_t* arrivals, uint32_t* bar, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  __shared__ uint32_t red[kBlock / 64];
  __shared__ uint32_t sh[3];  // generation at the start; last arrival?; amax bits, or ~0u when the wait gave up
  uint64_t* word = reinterpret_cast<uint64_t*>(bar + kBarGen);
  if (threadIdx.x == 0)
    sh[0] = (uint32_t)(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32);
  const size_t stride = (size_t)gridDim.x * kBlock;
  const size_t base = (size_t)blockIdx.x * kBlock + threadIdx.x;
  uint4 v[V];
  uint32_t m[V];
  // indices past the end reload the last vector (a real element: it cannot
  // change the max, and its codes are not stored)
#pragma unroll
  for (int k = 0; k < V; ++k) v[k] = x[min(base + k * stride, nvec - 1)];
  uint32_t mm = 0;
#pragma unroll
  for (int k = 0; k < V; ++k) {
    m[k] = vec_absmax_raw<XT>(v[k]);
    mm = max(mm, m[k]);
  }
  uint32_t fin = mm;
  if (__any(mm >= kInfBits)) {  // rare: filter the non-finite elements out
    fin = 0;
#pragma unroll
    for (int k = 0; k < V; ++k) fin = max(fin, m[k] < kInfBits ? m[k] : vec_absmax_finite<XT>(v[k]));
  }
  const uint32_t bfin = block_max_u32<kBlock>(fin, red);
  if (threadIdx.x == 0) {
    __hip_atomic_store(partial + blockIdx.x, bfin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    const uint32_t groups = min(gridDim.x, (uint32_t)kArrivalGroups);
    const uint32_t g = blockIdx.x % groups;
    const uint32_t members = (gridDim.x - g + groups - 1) / groups;
    uint32_t* sub = arrivals + g * kArrivalStride;
    bool last = false;
    if (__hip_atomic_fetch_add(sub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
      __hip_atomic_store(sub, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = __hip_atomic_fetch_add(bar + kBarTop, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1;
    }
    sh[1] = last;
  }
  __syncthreads();
  const uint32_t g0 = sh[0];
  if (sh[1]) {
    // the last arrival: every partial is in place
    uint32_t pm = 0;
    for (int i = threadIdx.x; i < (int)gridDim.x; i += kBlock)
      pm = max(pm, __hip_atomic_load(partial + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    pm = block_max_u32<kBlock>(pm, red);
    if (threadIdx.x == 0) {
      __hip_atomic_store(bar + kBarTop, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(word, ((uint64_t)(g0 + 1u) << 32) | pm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh[2] = pm;
    }
  } else if (threadIdx.x == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint32_t got = ~0u;
    for (;;) {
      const uint64_t w = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)(w >> 32) != g0) {
        got = (uint32_t)w;
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > kBarrierSpinTicks) {
        __hip_atomic_fetch_or(bar + kBarStatus, kGaveUpBit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    sh[2] = got;
  }
  __syncthreads();
  const uint32_t pm = sh[2];
  const bool gave_up = pm == ~0u;
  const float amax = __uint_as_float(pm);
  const float s = gave_up ? __uint_as_float(0x7fc00000u) : scale_from_amax<FMT>(amax);
  const float r = 1.0f / s;
  if (threadIdx.x == 0 && (blockIdx.x == 0 || gave_up)) {
    __hip_atomic_store(scale, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (amax_out) __hip_atomic_store(amax_out, amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!gave_up) {
      __builtin_amdgcn_s_waitcnt(0);
      if (__hip_atomic_load(bar + kBarStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kGaveUpBit)
        __hip_atomic_store(scale, __uint_as_float(0x7fc00000u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // (the codes need no tensor-wide non-finite flag: the cast patches NaN per vector)
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const size_t i = base + k * stride;
    if (i < nvec) {
      uint32_t w[E / 4];
      cast_vec<XT, FMT, SR, true>(v[k], r, m[k], w, sd, i * E);
      store_codes<E>(q + i * E, w);
    }
  }
}

// ---------------------------------------------------------------------------
// per column (dynamic)
// ---------------------------------------------------------------------------
// Tile: 32 vectors across (256 bf16 / 128 fp32 columns) x kColRows rows.
// Thread t: vector column t % 32, row lane t / 32 (8 lanes, stride 8); each
// thread issues all kColRows/8 of its loads before it uses any of them.

constexpr int kColVecs = 32;
constexpr int kColRows = kColChunkRows;
constexpr int kColPer = kColRows / 8;  // vectors per thread

// The thread's kColPer vectors of its tile (rows r0 + ty + 8j of vector column
// vc). Rows past the end reload the chunk's first row (a real element of the
// same column, so it cannot change the column max; its codes are not stored).
template <int XT>
__device__ __forceinline__ void col_tile_load(const uint4* __restrict__ x, int rows, int vpr, int r0, int vc, int ty,
                                              uint4 (&v)[kColPer]) {
#pragma unroll
  for (int j = 0; j < kColPer; ++j) {
    const int r = r0 + ty + 8 * j;
    v[j] = x[(size_t)(r < rows ? r : r0) * vpr + vc];
  }
}

// Column maxima of the tile: the thread's kColPer rows go into
// tile[ty][tx * E + e] (finite max in bits 0..30, non-finite seen in bit 31).
// Raw maxima first (bf16: two 16-bit magnitudes per max); the finite-only pass
// runs only where a raw max is Inf/NaN. Ends with a block barrier.
template <int XT>
__device__ __forceinline__ void col_tile_maxima(const uint4 (&v)[kColPer], bool valid, int tx, int ty,
                                                uint32_t (*tile)[kColVecs * VecTraits<XT>::kElems]) {
  constexpr int E = VecTraits<XT>::kElems;
  uint32_t m[E];
  uint32_t nf = 0;  // bit e: column e of this vector saw an Inf/NaN
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = 0;
  if (valid) {
    uint32_t any_nf = 0;
    if constexpr (XT == kBF16) {
      typedef unsigned short us2 __attribute__((ext_vector_type(2)));
      us2 p[4] = {us2{0, 0}, us2{0, 0}, us2{0, 0}, us2{0, 0}};
#pragma unroll
      for (int j = 0; j < kColPer; ++j) {
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) p[d] = __builtin_elementwise_max(p[d], __builtin_bit_cast(us2, w[d] & 0x7fff7fffu));
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        m[2 * d] = (uint32_t)p[d][0] << 16;
        m[2 * d + 1] = (uint32_t)p[d][1] << 16;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kColPer; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) m[e] = max(m[e], __float_as_uint(vec_elem<XT>(v[j], e)) & 0x7fffffffu);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) any_nf |= m[e] >= kInfBits ? 1u : 0u;
    if (__any(any_nf)) {
#pragma unroll
      for (int e = 0; e < E; ++e) m[e] = 0;
#pragma unroll
      for (int j = 0; j < kColPer; ++j) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t a = __float_as_uint(vec_elem<XT>(v[j], e)) & 0x7fffffffu;
          m[e] = max(m[e], a < kInfBits ? a : 0u);
          nf |= (a >= kInfBits ? 1u : 0u) << e;
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) tile[ty][tx * E + e] = m[e] | (((nf >> e) & 1u) ? kNonfiniteBit : 0u);
  __syncthreads();
}

// Partial word of tile column c: the 8 row lanes folded.
template <int E>
__device__ __forceinline__ uint32_t col_tile_word(uint32_t (*tile)[kColVecs * E], int c) {
  uint32_t acc = 0, flag = 0;
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    acc = max(acc, tile[l][c] & ~kNonfiniteBit);
    flag |= tile[l][c] & kNonfiniteBit;
  }
  return acc | flag;
}

// Fold column `col`'s nchunk partial words (8 loads in flight per round). The
// two-pass form keeps each partial in the low half of a 64-bit word whose high
// half is zero, so a one-pass call that later uses the same workspace bytes
// for its generation-tagged column words (tags >= 1) always overwrites them.
__device__ __forceinline__ uint32_t col_fold_partials(const uint64_t* partial, int nchunk, int cols, int col) {
  auto ld = [&](int k) -> uint32_t { return (uint32_t)partial[(size_t)k * cols + col]; };
  uint32_t acc = 0, flag = 0;
  int k = 0;
  for (; k + 8 <= nchunk; k += 8) {
    uint32_t p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = ld(k + u);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc = max(acc, p[u] & ~kNonfiniteBit);
      flag |= p[u] & kNonfiniteBit;
    }
  }
  for (; k < nchunk; ++k) {
    const uint32_t p = ld(k);
    acc = max(acc, p & ~kNonfiniteBit);
    flag |= p & kNonfiniteBit;
  }
  return acc | flag;
}

// The tile's column scales from their folded words: rcp and flags in LDS, the
// scales and amax written by the blocks of row chunk 0. Ends with a block barrier.
template <int FMT, int E>
__device__ __forceinline__ void col_tile_scales(const uint64_t* partial, int nchunk, int cols, float* __restrict__ scale,
                                                float* __restrict__ amax_out, float* rcp, uint32_t* flags) {
  for (int c = threadIdx.x; c < kColVecs * E; c += kBlock) {
    const int col = blockIdx.x * kColVecs * E + c;
    uint32_t word = 0;
    if (col < cols) {
      word = col_fold_partials(partial, nchunk, cols, col);
      const float amax = __uint_as_float(word & ~kNonfiniteBit);
      const float s = scale_from_amax<FMT>(amax);
      rcp[c] = 1.0f / s;
      if (blockIdx.y == 0) {
        scale[col] = s;
        if (amax_out) amax_out[col] = amax;
      }
    } else {
      rcp[c] = 0.0f;
    }
    flags[c] = word & kNonfiniteBit;
  }
  __syncthreads();
}

// Cast the thread's kColPer vectors with their columns' reciprocals.
template <int XT, int FMT, bool SR>
__device__ __forceinline__ void col_tile_cast(const uint4 (&v)[kColPer], int rows, int vpr, int r0, int vc, int tx,
                                              int ty, const float* rcp, const uint32_t* flags, uint8_t* __restrict__ q,
                                              SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  bool patch = false;
  float r[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    r[e] = rcp[tx * E + e];
    patch |= flags[tx * E + e] != 0;
  }
#pragma unroll
  for (int j = 0; j < kColPer; ++j) {
    const int row = r0 + ty + 8 * j;
    if (row >= rows) break;
    uint32_t w[E / 4];
#pragma unroll
    for (int d = 0; d < E / 4; ++d) {
      const float a = vec_elem<XT>(v[j], 4 * d + 0) * r[4 * d + 0];
      const float b = vec_elem<XT>(v[j], 4 * d + 1) * r[4 * d + 1];
      const float c = vec_elem<XT>(v[j], 4 * d + 2) * r[4 * d + 2];
      const float e = vec_elem<XT>(v[j], 4 * d + 3) * r[4 * d + 3];
      if constexpr (SR) {
        w[d] = e5m2_sr4(a, b, c, e, sd, ((size_t)row * vpr + vc) * E + 4 * d);
      } else {
        // r comes from the column's own amax, so without a non-finite element in
        // these columns no value needs the clamp (vec_cast_checked, OWN)
        if (patch) w[d] = patch_nan4(cvt4<FMT>(a, b, c, e), a, b, c, e);
        else w[d] = cvt4<FMT, false>(a, b, c, e);
      }
    }
    store_codes<E>(q + ((size_t)row * vpr + vc) * E, w);
  }
}

template <int XT>
__global__ __launch_bounds__(kBlock) void colmax_partials_kernel(const uint4* __restrict__ x, int rows, int vpr,
                                                                 uint64_t* __restrict__ partial) {
  constexpr int E = VecTraits<XT>::kElems;
  __shared__ uint32_t tile[8][kColVecs * E];
  const int tx = threadIdx.x % kColVecs, ty = threadIdx.x / kColVecs;
  const int vc = blockIdx.x * kColVecs + tx;
  const int r0 = blockIdx.y * kColRows;
  uint4 v[kColPer];
  if (vc < vpr) col_tile_load<XT>(x, rows, vpr, r0, vc, ty, v);
  col_tile_maxima<XT>(v, vc < vpr, tx, ty, tile);
  for (int c = threadIdx.x; c < kColVecs * E; c += kBlock) {
    const int col = blockIdx.x * kColVecs * E + c;
    if (col < vpr * E) partial[(size_t)blockIdx.y * vpr * E + col] = (uint64_t)col_tile_word<E>(tile, c);
  }
}

template <int XT, int FMT, bool SR>
__global__ __launch_bounds__(kBlock) void quant_cols_kernel(const uint4* __restrict__ x, int rows, int vpr,
                                                            const uint64_t* __restrict__ partial, int nchunk,
                                                            uint8_t* __restrict__ q, float* __restrict__ scale,
                                                            float* __restrict__ amax_out, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  __shared__ float rcp[kColVecs * E];
  __shared__ uint32_t flags[kColVecs * E];
  const int tx = threadIdx.x % kColVecs, ty = threadIdx.x / kColVecs;
  const int vc = blockIdx.x * kColVecs + tx;
  const int r0 = blockIdx.y * kColRows;
  // the chunk's input loads go out first; the column scales are folded while
  // they are in flight
  uint4 v[kColPer];
  if (vc < vpr) col_tile_load<XT>(x, rows, vpr, r0, vc, ty, v);
  col_tile_scales<FMT, E>(partial, nchunk, vpr * E, scale, amax_out, rcp, flags);
  if (vc >= vpr) return;
  col_tile_cast<XT, FMT, SR>(v, rows, vpr, r0, vc, tx, ty, rcp, flags, q, sd);
}

// Per column in one pass: the same tiles, held in registers while the grid
// agrees on the column maxima. Each column has a 64-bit word whose high half
// is a launch tag (the barrier generation + 1) and whose low half is the
// finite amax bits; each block applies a device-scope 64-bit atomic max of
// (tag, its tile's column max) to every column it covers, so the first update
// of a launch replaces whatever an earlier call left in those bytes (an
// earlier one-pass word has a smaller tag, a two-pass partial a zero high
// half) and no reset is needed. A tile holding an Inf or NaN also raises one tensor-wide
// flag word the same way (the cast then patches NaN in every column, which is
// exact for finite values too). Then the block counts in through the arrival
// tree, the last arrival advances the generation half of the barrier word and
// the others poll it (as in quant_tensor_fused_kernel; same residency
// condition and bounded poll), and every block reads its columns' words, one
// load each, and casts. Folding one partial word per row chunk and column with
// device-scope loads after the barrier instead (32 KB per block on bf16
// [4096, 4096]) took 14.0 us against 12.8 us.
template <int XT, int FMT, bool SR>
__global__ __launch_bounds__(kBlock) void quant_cols_fused_kernel(const uint4* __restrict__ x, int rows, int vpr,
                                                                  uint64_t* colw, uint32_t* arrivals, uint32_t* bar,
                                                                  uint8_t* __restrict__ q, float* __restrict__ scale,
                                                                  float* __restrict__ amax_out, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  __shared__ uint32_t tile[8][kColVecs * E];
  __shared__ float rcp[kColVecs * E];
  __shared__ uint32_t flags[kColVecs * E];
  __shared__ uint32_t sh[2];  // generation at the start; 1 when the wait gave up
  uint64_t* word = reinterpret_cast<uint64_t*>(bar + kBarGen);
  const int tx = threadIdx.x % kColVecs, ty = threadIdx.x / kColVecs;
  const int vc = blockIdx.x * kColVecs + tx;
  const int r0 = blockIdx.y * kColRows;
  const int cols = vpr * E;
  if (threadIdx.x == 0)
    sh[0] = (uint32_t)(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32);
  uint4 v[kColPer];
  if (vc < vpr) col_tile_load<XT>(x, rows, vpr, r0, vc, ty, v);
  col_tile_maxima<XT>(v, vc < vpr, tx, ty, tile);  // ends with a block barrier: sh[0] is visible
  const uint64_t tag = (uint64_t)(sh[0] + 1u) << 32;  // >= 1: above any word a two-pass call leaves
  uint64_t* nf_word = reinterpret_cast<uint64_t*>(bar + kBarColFlag);
  for (int c = threadIdx.x; c < kColVecs * E; c += kBlock) {
    const int col = blockIdx.x * kColVecs * E + c;
    if (col < cols) {
      const uint32_t w = col_tile_word<E>(tile, c);
      __hip_atomic_fetch_max(colw + col, tag | (w & ~kNonfiniteBit), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (w & kNonfiniteBit) __hip_atomic_fetch_max(nf_word, tag | 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t g0 = sh[0];
    const uint32_t nblocks = gridDim.x * gridDim.y;
    const uint32_t b = blockIdx.y * gridDim.x + blockIdx.x;
    const uint32_t groups = min(nblocks, (uint32_t)kArrivalGroups);
    const uint32_t g = b % groups;
    const uint32_t members = (nblocks - g + groups - 1) / groups;
    uint32_t* sub = arrivals + g * kArrivalStride;
    bool last = false;
    if (__hip_atomic_fetch_add(sub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
      __hip_atomic_store(sub, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = __hip_atomic_fetch_add(bar + kBarTop, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1;
    }
    uint32_t gave_up = 0;
    if (last) {
      __hip_atomic_store(bar + kBarTop, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(word, (uint64_t)(g0 + 1u) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while ((uint32_t)(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) == g0) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kBarrierSpinTicks) {
          __hip_atomic_fetch_or(bar + kBarStatus, kGaveUpBit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_s_waitcnt(0);
          gave_up = 1u;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    sh[1] = gave_up;
  }
  __syncthreads();
  if (sh[1]) {
    // the wait gave up (status bit set above): NaN scales for this tile's
    // columns instead of codes
    for (int c = threadIdx.x; c < kColVecs * E; c += kBlock) {
      const int col = blockIdx.x * kColVecs * E + c;
      if (col < cols) __hip_atomic_store(scale + col, __uint_as_float(0x7fc00000u), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  {
    // this launch's words (every column of the grid has one update per row chunk)
    const bool nonfinite = __hip_atomic_load(nf_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (tag | 1u);
    for (int c = threadIdx.x; c < kColVecs * E; c += kBlock) {
      const int col = blockIdx.x * kColVecs * E + c;
      if (col < cols) {
        const float amax = __uint_as_float((uint32_t)__hip_atomic_load(colw + col, __ATOMIC_RELAXED,
                                                                       __HIP_MEMORY_SCOPE_AGENT));
        const float s = scale_from_amax<FMT>(amax);
        rcp[c] = 1.0f / s;
        if (blockIdx.y == 0) {
          __hip_atomic_store(scale + col, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (amax_out) __hip_atomic_store(amax_out + col, amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        rcp[c] = 0.0f;
      }
      flags[c] = nonfinite ? 1u : 0u;
    }
    __syncthreads();
  }
  if (blockIdx.y == 0) {
    // the writer of these columns' scales: once every thread's scale store has
    // completed, if any block gave up, NaN wins
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      sh[1] = __hip_atomic_load(bar + kBarStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kGaveUpBit;
    __syncthreads();
    if (sh[1]) {
      for (int c = threadIdx.x; c < kColVecs * E; c += kBlock) {
        const int col = blockIdx.x * kColVecs * E + c;
        if (col < cols) __hip_atomic_store(scale + col, __uint_as_float(0x7fc00000u), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (vc >= vpr) return;
  col_tile_cast<XT, FMT, SR>(v, rows, vpr, r0, vc, tx, ty, rcp, flags, q, sd);
}

// ---------------------------------------------------------------------------
// delayed scaling: the amax-history ring
// ---------------------------------------------------------------------------

// Fold one amax sample into the ring [hist[len] | scale | counter] and publish
// the next scale (readings: max-reduced window; next = max * 2^margin / fmax,
// floored at 2^-126; an all-zero window keeps the scale; a non-finite sample
// leaves the ring unchanged and sets the sticky flag). Resets the counter.
// Every thread of the block calls it: the window is read in parallel (one
// history entry per thread, the new sample standing in for entry idx) and
// reduced with the block max; thread 0 writes the ring.
template <int FMT, int BLOCK>
__device__ void ring_fold(float* state, int len, int idx, int margin, int32_t* flag, float amax,
                          bool nonfinite, uint32_t* red) {
  const bool ok = !nonfinite && amax <= 3.40282347e38f;  // false for NaN and Inf
  float w = 0.0f;
  if (ok)
    for (int i = threadIdx.x; i < len; i += BLOCK) w = fmaxf(w, i == idx ? amax : state[i]);
  // window entries are finite and >= 0, so their bit patterns order like the values
  w = __uint_as_float(block_max_u32<BLOCK>(__float_as_uint(w), red));
  if (threadIdx.x != 0) return;
  if (!ok) {
    if (flag) *flag = 1;
  } else {
    state[idx] = amax;
    if (w > 0.0f) {
      const float cand = ldexpf(w, margin) / Fp8Fmt<FMT>::kMax;
      if (cand <= 3.40282347e38f) state[len] = fmaxf(cand, kScaleFloor);
      else if (flag) *flag = 1;
    }
  }
  // the arrival counter goes back to zero at the coherence point, where the
  // next call's device-scope increments take place
  __hip_atomic_store(reinterpret_cast<uint32_t*>(state) + len + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT>
__global__ __launch_bounds__(64) void ring_update_kernel(float* state, int len, int idx, int margin, int32_t* flag,
                                                         const float* __restrict__ amax) {
  ring_fold<FMT, 64>(state, len, idx, margin, flag, *amax, false, nullptr);
}

// The tail every delayed-scaling kernel shares: publish this block's partial
// amax, count the block in, and let the last block fold the tensor amax into
// the ring (and report s_t and the amax). Every thread of the block calls it.
//
// The partial goes out as a device-scope atomic store, which writes through
// to the coherence point, and the count is issued only after that store has
// completed (s_waitcnt), so a block that sees the final count finds every
// partial there. No release fence: on this part an agent-scope fence writes
// back the XCD's whole L2, which cost more than the quantization itself. The
// last block reads the partials with device-scope atomic loads, which also go
// to the coherence point, so it needs no acquire fence either. Counting is a
// two-level tree: block b counts into arrival counter b % G; the last arrival
// of each group resets that counter and counts into the ring's counter, and
// the G-th arrival there is the last block overall.
template <int FMT>
__device__ void delayed_finish(uint32_t raw, uint32_t fin, float s_t, float* __restrict__ scale_out,
                               float* __restrict__ amax_out, float* state, int len, int idx, int margin,
                               int32_t* flag, uint32_t* partial, uint32_t* arrivals, uint32_t* red) {
  __shared__ bool is_last;
  const uint32_t braw = block_max_u32<kBlock>(raw, red);
  const uint32_t bfin = block_max_u32<kBlock>(fin, red);
  uint32_t* counter = reinterpret_cast<uint32_t*>(state) + len + 1;
  if (threadIdx.x == 0) {
    __hip_atomic_store(partial + blockIdx.x, bfin | (braw >= kInfBits ? kNonfiniteBit : 0u), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    const uint32_t groups = min(gridDim.x, (uint32_t)kArrivalGroups);
    const uint32_t g = blockIdx.x % groups;
    const uint32_t members = (gridDim.x - g + groups - 1) / groups;
    uint32_t* sub = arrivals + g * kArrivalStride;
    bool last = false;
    if (__hip_atomic_fetch_add(sub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
      __hip_atomic_store(sub, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == groups - 1;
    }
    is_last = last;
  }
  __syncthreads();
  if (!is_last) return;
  uint32_t m = 0, f = 0;
  for (int i = threadIdx.x; i < (int)gridDim.x; i += kBlock) {
    const uint32_t p = __hip_atomic_load(partial + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    m = max(m, p & ~kNonfiniteBit);
    f |= p & kNonfiniteBit;
  }
  m = block_max_u32<kBlock>(m, red);
  f = block_max_u32<kBlock>(f, red);
  const float amax = __uint_as_float(m);
  if (threadIdx.x == 0) {
    scale_out[0] = s_t;
    if (amax_out) amax_out[0] = amax;
  }
  ring_fold<FMT, kBlock>(state, len, idx, margin, flag, amax, f != 0, red);
}

template <int XT, int FMT, bool SR>
__global__ __launch_bounds__(kBlock) void quant_delayed_kernel(const uint4* __restrict__ x, size_t nvec,
                                                               uint8_t* __restrict__ q, float* __restrict__ scale_out,
                                                               float* __restrict__ amax_out, float* state, int len,
                                                               int idx, int margin, int32_t* flag,
                                                               uint32_t* partial, uint32_t* arrivals, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  __shared__ uint32_t red[kBlock / 64];
  const float s_t = state[len];
  const float r = 1.0f / s_t;
  uint32_t raw = 0, fin = 0;
  const size_t stride = (size_t)gridDim.x * kBlock * kUnroll;
  for (size_t base = blockIdx.x * (size_t)kBlock * kUnroll + threadIdx.x; base < nvec; base += stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (base + u * kBlock < nvec) v[u] = x[base + u * kBlock];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + u * kBlock;
      if (i < nvec) {
        const uint32_t m = vec_absmax_raw<XT>(v[u]);
        raw = max(raw, m);
        fin = max(fin, m < kInfBits ? m : vec_absmax_finite<XT>(v[u]));
        uint32_t w[E / 4];
        cast_vec<XT, FMT, SR>(v[u], r, m, w, sd, i * E);
        store_codes<E>(q + i * E, w);
      }
    }
  }
  delayed_finish<FMT>(raw, fin, s_t, scale_out, amax_out, state, len, idx, margin, flag, partial, arrivals, red);
}

// ---------------------------------------------------------------------------
// per tensor, into several layouts in one pass
// ---------------------------------------------------------------------------
// The codes of a per-tensor quantization do not depend on where they are
// stored, so one pass over X can write them row-major, transposed ([cols,
// rows] row-major) and in the GEMM's pre-shuffled weight layout of either (the
// fused quantize-plus-transpose of the hip-quant README, "Runtime codebooks and
// GPU execution features"; for the backward GEMMs it replaces the transposed
// copies and the separate pre-shuffle passes). A workgroup takes 128 x 128
// tiles; thread t owns the 8 x 8 block of rows 8*(t/16) .. +7 and columns
// 8*(t%16) .. +7, loads it once, casts it, and writes 8-byte pieces: rows of
// the block to the row-major outputs, and (after an in-register byte
// transpose) columns of the block to the transposed ones. Elements past the
// tensor read as zero, so the zero padding of the pre-shuffled layouts is
// written as zero codes.

// Byte offset of weight element (n, k) in the pre-shuffled layout with
// `kblocks` 128-deep K blocks: row n = 32G + 8g + 4p + r is slot 4g + r of
// fragment 2G + p; fragment (nb, kb) holds 2048 bytes at (nb * kblocks + kb) *
// 2048; column k_in of a slot sits at h*1024 + (q*16 + slot)*16 + b with
// q = k_in/32, h = (k_in%32)/16, b = k_in%16.
__device__ __forceinline__ size_t preshuffled_offset(int n, int k, int kblocks) {
  const int nb = 2 * (n >> 5) + ((n >> 2) & 1), slot = 4 * ((n >> 3) & 3) + (n & 3);
  const int kin = k & 127;
  return ((size_t)nb * kblocks + (k >> 7)) * 2048 + ((kin >> 4) & 1) * 1024 + ((kin >> 5) * 16 + slot) * 16 +
         (kin & 15);
}

enum { kScaleGiven = 0, kScaleRing = 1, kScaleDynamic = 2 };

template <int XT, int FMT, int MODE, bool SR, bool STAGE_T>
__global__ __launch_bounds__(kBlock) void quant_layouts_kernel(
    const uint4* __restrict__ x, int rows, int cols, LayoutOut o, const float* __restrict__ scale_in,
    const uint32_t* __restrict__ dyn_partial, int ndyn, float* __restrict__ scale_out,
    float* __restrict__ amax_out, float* state, int len, int idx, int margin, int32_t* flag, uint32_t* partial,
    uint32_t* arrivals, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  constexpr int VPC = 8 / E;  // 16-byte vectors per 8 columns
  // A whole tile's transposed codes go through LDS (128 rows of the
  // transposed tile, 136-byte pitch against bank conflicts) and out as whole
  // 128-byte lines: stored straight from the threads, each line of the
  // transposed output came in four 32-byte pieces from four wavefronts
  // (15.0 -> 13.9 us for a bf16 [2048, 4096] gradient, row-major and
  // transposed, with a ring). The transposed pre-shuffled output keeps the
  // per-thread stores: staged in the same way (each 128 x 128 tile is one K
  // block of 8 contiguous 2048-byte fragments) it was no faster on [4096,
  // 1024] and slower on [2048, 1024] (5.5 -> 5.9 us, 128 tiles: one workgroup
  // on half the CUs, whose extra barriers nothing overlaps).
  // (STAGE_T: launched when the transposed row-major output is asked for; the
  // other launches keep the registers of the plain form.)
  constexpr int kQtPitch = 136;
  __shared__ __align__(16) uint8_t qt_stage[STAGE_T ? 128 * kQtPitch : 16];
  __shared__ uint32_t red[kBlock / 64];
  float s;
  if (MODE == kScaleGiven) {
    s = scale_in[0];
  } else if (MODE == kScaleRing) {
    s = state[len];
  } else {
    bool nonfinite;
    const float amax = __uint_as_float(fold_partials(dyn_partial, ndyn, red, &nonfinite));
    s = scale_from_amax<FMT>(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0 && amax_out) amax_out[0] = amax;
  }
  const float r = 1.0f / s;
  if (MODE != kScaleRing && blockIdx.x == 0 && threadIdx.x == 0) scale_out[0] = s;
  const int rg = threadIdx.x >> 4, cv = threadIdx.x & 15;
  const int vpr = cols / E;
  const int tiles_c = (cols + 127) / 128;
  const int tiles = ((rows + 127) / 128) * tiles_c;
  uint32_t raw = 0, fin = 0;
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int r0 = (tile / tiles_c) * 128 + 8 * rg, c0 = (tile % tiles_c) * 128 + 8 * cv;
    const bool col_ok = c0 < cols;  // cols % 16 == 0: an 8-column piece is all in or all out
    uint4 v[8][VPC];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int u = 0; u < VPC; ++u)
        v[j][u] = (col_ok && r0 + j < rows) ? x[(size_t)(r0 + j) * vpr + c0 / E + u] : make_uint4(0u, 0u, 0u, 0u);
    uint2 c[8];  // codes: row j of the block, columns 0..3 in .x, 4..7 in .y
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t w[2];
#pragma unroll
      for (int u = 0; u < VPC; ++u) {
        const uint32_t m = vec_absmax_raw<XT>(v[j][u]);
        raw = max(raw, m);
        fin = max(fin, m < kInfBits ? m : vec_absmax_finite<XT>(v[j][u]));
        // stochastic rounding keys on the element's row-major index in x, so
        // every layout of an element gets the same code
        cast_vec<XT, FMT, SR>(v[j][u], r, m, w + u * (E / 4), sd, (size_t)(r0 + j) * cols + c0 + u * E);
      }
      c[j] = make_uint2(w[0], w[1]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = r0 + j;
      if (o.q && col_ok && row < rows) *reinterpret_cast<uint2*>(o.q + (size_t)row * cols + c0) = c[j];
      if (o.qp && row < o.np_q) *reinterpret_cast<uint2*>(o.qp + preshuffled_offset(row, c0, o.kb_q)) = c[j];
    }
    if (o.qt || o.qtp) {
      // t[i]: column i of the block, rows 0..3 in .x, 4..7 in .y
      uint2 t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo |= (((i < 4 ? c[j].x : c[j].y) >> (8 * (i & 3))) & 0xffu) << (8 * j);
          hi |= (((i < 4 ? c[j + 4].x : c[j + 4].y) >> (8 * (i & 3))) & 0xffu) << (8 * j);
        }
        t[i] = make_uint2(lo, hi);
      }
      const int tr0 = (tile / tiles_c) * 128, tc0 = (tile % tiles_c) * 128;
      (void)tr0;
      (void)tc0;
      const bool stage_t = STAGE_T && o.qt && tr0 + 128 <= rows && tc0 + 128 <= cols;  // workgroup-uniform
      if (stage_t) {
        __syncthreads();  // the previous tile's read-back is done
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint2*>(qt_stage + (8 * cv + i) * kQtPitch + 8 * rg) = t[i];
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 128 * 8 / kBlock; ++p) {
          const int idx = p * kBlock + threadIdx.x;  // 16-byte piece c16 of transposed row R
          const int R = idx >> 3, c16 = idx & 7;
          const uint2 lo = *reinterpret_cast<const uint2*>(qt_stage + R * kQtPitch + 16 * c16);
          const uint2 hi = *reinterpret_cast<const uint2*>(qt_stage + R * kQtPitch + 16 * c16 + 8);
          __builtin_nontemporal_store(hq_u4v{lo.x, lo.y, hi.x, hi.y},
                                      reinterpret_cast<hq_u4v*>(o.qt + (size_t)(tc0 + R) * rows + tr0 + 16 * c16));
        }
      }
      // rows % 16 == 0 when a transposed output is asked for: an 8-row piece is all in or all out
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int col = c0 + i;
        if (o.qt && !stage_t && col < cols && r0 < rows) *reinterpret_cast<uint2*>(o.qt + (size_t)col * rows + r0) = t[i];
        if (o.qtp && col < o.np_t) *reinterpret_cast<uint2*>(o.qtp + preshuffled_offset(col, r0, o.kb_t)) = t[i];
      }
    }
  }
  if (MODE == kScaleRing)
    delayed_finish<FMT>(raw, fin, s, scale_out, amax_out, state, len, idx, margin, flag, partial, arrivals, red);
}

// ---------------------------------------------------------------------------
// per row, straight into the pre-shuffled weight layout
// ---------------------------------------------------------------------------
// Row n of a weight [N, K] is the GEMM's output channel n, so per-row scaling
// is the per-output-channel weight scale, and the codes can go to the
// pre-shuffled layout at once instead of through a row-major copy.
//
// Per-row (per-output-channel) quantization of a weight straight into the
// pre-shuffled layout of the GEMM, for rows too long to keep in registers
// (more than 4096 bf16 or 2048 fp32 padded columns): one wavefront per row,
// the row read twice (amax pass, then cast pass), codes stored one vector at a
// time at their pre-shuffled offsets. Columns past K up to the 128-padded K,
// and rows past N up to the 32-padded N, are written as zero codes.
constexpr int kPreRows = 16;

template <int XT, int FMT>
__global__ __launch_bounds__(64 * kPreRows) void quant_rows_pre_long_kernel(
    const uint4* __restrict__ x, uint8_t* __restrict__ q, uint8_t* __restrict__ qp, float* __restrict__ scale,
    float* __restrict__ amax_out, int rows, int vpr, int kblocks) {
  constexpr int E = VecTraits<XT>::kElems;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kPreRows + (threadIdx.x >> 6);
  const bool valid = row < rows;
  const int vpp = kblocks * (128 / E);  // vectors per padded row
  const SrSeed sd{0u, 0u};
  const uint32_t zero[4] = {0u, 0u, 0u, 0u};
  const uint4* xr = x + (size_t)(valid ? row : 0) * vpr;
  uint32_t mx = 0;
  if (valid) {
    for (int i = lane; i < vpr; i += 64) mx = max(mx, vec_absmax_raw<XT>(xr[i]));
    mx = wave_max_u32(mx);
    if (mx >= kInfBits) {  // the row holds an Inf/NaN: recompute over finite elements
      uint32_t f = 0;
      for (int i = lane; i < vpr; i += 64) f = max(f, vec_absmax_finite<XT>(xr[i]));
      mx = wave_max_u32(f);
    }
  }
  const float amax = __uint_as_float(mx);
  const float s = scale_from_amax<FMT>(amax);
  const float r = 1.0f / s;
  if (valid && lane == 0) {
    scale[row] = s;
    if (amax_out) amax_out[row] = amax;
  }
  for (int i = lane; i < vpp; i += 64) {
    uint32_t w[E / 4];
    if (valid && i < vpr) {
      const uint4 v = xr[i];
      cast_vec<XT, FMT, false, true>(v, r, vec_absmax_raw<XT>(v), w, sd, 0);
      if (q) store_codes<E>(q + ((size_t)row * vpr + i) * E, w);
      store_codes_temporal<E>(qp + preshuffled_offset(row, i * E, kblocks), w);
    } else {
      store_codes_temporal<E>(qp + preshuffled_offset(row, i * E, kblocks), zero);
    }
  }
}

// Per-row quantization straight into the pre-shuffled layout, for rows whose
// padded length fits NV vectors per lane. Row 32G + 8g + 4p + r is slot 4g + r
// of fragment 2G + p, and a 128-byte line of the layout holds slots 0-7 or
// 8-15 of one (fragment, K block, half, 32-column group), so the 8 rows of a
// line group gi (16-row block gi / 2, fragment parity gi % 2: rows 16(gi/2) +
// 4(gi%2) + {0..3, 8..11}) fill whole lines. One workgroup of 8 wavefronts
// (one row each, held in registers between the amax and the cast) per line
// group; the codes are staged in LDS in output order (slot s8 of staged line L
// at position (s8 + L) % 8, which spreads a wavefront's writes over the banks)
// and written as whole lines, 8 lanes per line. Rows from N up to the next
// multiple of 32 are zero codes. Measured on bf16 [4096, 4096]: 10.1 us,
// against 11.4 us for 16-row workgroups (both fragment parities, 64 KB of
// LDS; 4096 rows give one workgroup per CU, so no workgroup's stores
// overlapped another's reads) and 12.1 us for one workgroup per CU walking
// several line groups, loading the next one's rows first.
constexpr int kPreWaves = 8;
constexpr int kPreStageMin = 54 << 10;
template <int XT, int FMT, int NV>
__global__ __launch_bounds__(64 * kPreWaves) void quant_rows_pre_group_kernel(
    const uint4* __restrict__ x, uint8_t* __restrict__ q, uint8_t* __restrict__ qp, float* __restrict__ scale,
    float* __restrict__ amax_out, int rows, int vpr, int kblocks) {
  constexpr int E = VecTraits<XT>::kElems;
  static_assert(NV > 0, "rows held in registers");
  // at least 54 KB, so at most two workgroups share a CU (160 KB of LDS):
  // measured on bf16 [4096, 4096], 10.1 us at two against 10.8 us at four
  constexpr int kStage = kPreWaves * 64 * NV * E > kPreStageMin ? kPreWaves * 64 * NV * E : kPreStageMin;
  __shared__ __align__(16) uint8_t stage[kStage];
  const int lane = threadIdx.x & 63;
  const int s8 = threadIdx.x >> 6;  // this wavefront's slot within each line
  const int g = blockIdx.x;
  const int row = (g >> 1) * 16 + 4 * (g & 1) + (s8 & 3) + 8 * (s8 >> 2);
  const bool valid = row < rows;
  const int vpp = kblocks * (128 / E);
  const SrSeed sd{0u, 0u};
  // lanes past the row end reload its last vector (a real element, so it
  // cannot change the max); rows past N read row 0 and store zero codes
  const uint4* xr = x + (size_t)(valid ? row : 0) * vpr;
  uint4 cur[NV];
  uint32_t raw[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) cur[j] = xr[min(lane + 64 * j, vpr - 1)];
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    raw[j] = vec_absmax_raw<XT>(cur[j]);
    mx = max(mx, raw[j]);
  }
  mx = wave_max_u32(mx);
  // a valid, full row (NV whole vectors per lane, K a multiple of 128) without
  // Inf or NaN: no bounds checks, no NaN patch and no clamp per vector
  const bool full_finite = valid && mx < kInfBits && vpr == 64 * NV && vpp == vpr;  // wavefront-uniform
  if (mx >= kInfBits) {  // the row holds an Inf/NaN: recompute over finite elements
    uint32_t f = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) f = max(f, vec_absmax_finite<XT>(cur[j]));
    mx = wave_max_u32(f);
  }
  const float amax = __uint_as_float(mx);
  const float s = scale_from_amax<FMT>(amax);
  const float r = 1.0f / s;
  if (valid && lane == 0) {
    scale[row] = s;
    if (amax_out) amax_out[row] = amax;
  }
  auto stage_codes = [&](int i, const uint32_t* w) {
    const int c0 = i * E, kin = c0 & 127;
    const int L = ((c0 >> 7) * 2 + ((kin >> 4) & 1)) * 4 + (kin >> 5);
    store_codes_temporal<E>(stage + L * 128 + (((s8 + L) & 7) << 4) + (kin & 15), w);
  };
  if (full_finite) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = lane + 64 * j;
      uint32_t w[E / 4];
      vec_cast<XT, FMT, false>(cur[j], r, false, w);
      if (q) store_codes<E>(q + ((size_t)row * vpr + i) * E, w);
      stage_codes(i, w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int i = lane + 64 * j;
      if (i < vpp) {
        uint32_t w[E / 4];
        if (valid && i < vpr) {
          cast_vec<XT, FMT, false, true>(cur[j], r, raw[j], w, sd, 0);
          if (q) store_codes<E>(q + ((size_t)row * vpr + i) * E, w);
        } else {
#pragma unroll
          for (int d = 0; d < E / 4; ++d) w[d] = 0u;
        }
        stage_codes(i, w);
      }
    }
  }
  __syncthreads();
  const int g16 = g >> 1, pf = g & 1, G = g16 >> 1, half = g16 & 1;
  const int pieces = 64 * kblocks;  // 8 lines per K block, 8 pieces of 16 bytes each
  for (int t = threadIdx.x; t < pieces; t += 64 * kPreWaves) {
    const int L = t >> 3, pos = t & 7;
    const hq_u4v v = *reinterpret_cast<const hq_u4v*>(stage + t * 16);
    const int slot = 8 * half + ((pos - L) & 7);
    const size_t off = ((size_t)(2 * G + pf) * kblocks + (L >> 3)) * 2048 + ((L >> 2) & 1) * 1024 +
                       ((L & 3) * 16 + slot) * 16;
    __builtin_nontemporal_store(v, reinterpret_cast<hq_u4v*>(qp + off));
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Blocks of the amax-partials pass and of the delayed kernel (= partials written).
int tensor_partial_blocks(size_t nvec) {
  size_t b = (nvec + kBlock * kUnroll - 1) / (kBlock * kUnroll);
  if (b < 1) b = 1;
  if (b > kMaxTensorPartials) b = kMaxTensorPartials;
  return (int)b;
}

int col_chunks(int rows) { return (rows + kColRows - 1) / kColRows; }

#define HQ_DISPATCH_XT_FMT(XT, FMT, CALL)                 \
  do {                                                    \
    if ((XT) == kBF16 && (FMT) == kE4M3) { CALL(kBF16, kE4M3, false); } \
    else if ((XT) == kBF16) { CALL(kBF16, kE5M2, false); }       \
    else if ((FMT) == kE4M3) { CALL(kF32, kE4M3, false); }       \
    else { CALL(kF32, kE5M2, false); }                           \
  } while (0)

// As above, plus the stochastic-rounding (E5M2 only) instances when `sr`.
#define HQ_DISPATCH_XT_FMT_SR(XT, FMT, SRF, CALL)                     \
  do {                                                                \
    if (SRF) {                                                        \
      if ((XT) == kBF16) { CALL(kBF16, kE5M2, true); }                \
      else { CALL(kF32, kE5M2, true); }                               \
    } else {                                                          \
      HQ_DISPATCH_XT_FMT(XT, FMT, CALL);                              \
    }                                                                 \
  } while (0)

static SrSeed sr_seed(uint64_t seed) { return SrSeed{(uint32_t)seed, (uint32_t)(seed >> 32)}; }

hipError_t launch_quant_rows(const void* x, int xt, int rows, int cols, int fmt, uint8_t* q, float* scale,
                             float* amax, bool sr, uint64_t seed, hipStream_t st) {
  const int vpr = xt == kBF16 ? cols / 8 : cols / 4;
  const SrSeed sd = sr_seed(seed);
#define CALL(A, B, S) return launch_rows_t<A, B, S>(x, rows, vpr, q, scale, amax, sd, st)
  HQ_DISPATCH_XT_FMT_SR(xt, fmt, sr, CALL);
#undef CALL
}

template <int XT, int FMT>
static hipError_t launch_rows_pre_t(const void* x, int rows, int cols, uint8_t* q, uint8_t* qp, float* scale,
                                    float* amax, hipStream_t st) {
  constexpr int E = VecTraits<XT>::kElems;
  const uint4* xv = static_cast<const uint4*>(x);
  const int vpr = cols / E;
  const int kblocks = (cols + 127) / 128;
  const int vpp = kblocks * (128 / E);
  const dim3 grid((rows + 31) / 32 * 32 / kPreRows), block(64 * kPreRows);
  // one workgroup per line group of 8 rows
  const dim3 wgrid((rows + 31) / 32 * 32 / kPreWaves), wblock(64 * kPreWaves);
  if (vpp <= 64) {
    hipLaunchKernelGGL((quant_rows_pre_group_kernel<XT, FMT, 1>), wgrid, wblock, 0, st, xv, q, qp, scale, amax, rows,
                       vpr, kblocks);
  } else if (vpp <= 128) {
    hipLaunchKernelGGL((quant_rows_pre_group_kernel<XT, FMT, 2>), wgrid, wblock, 0, st, xv, q, qp, scale, amax, rows,
                       vpr, kblocks);
  } else if (vpp <= 256) {
    hipLaunchKernelGGL((quant_rows_pre_group_kernel<XT, FMT, 4>), wgrid, wblock, 0, st, xv, q, qp, scale, amax, rows,
                       vpr, kblocks);
  } else if (vpp <= 512) {
    hipLaunchKernelGGL((quant_rows_pre_group_kernel<XT, FMT, 8>), wgrid, wblock, 0, st, xv, q, qp, scale, amax, rows,
                       vpr, kblocks);
  } else {
    hipLaunchKernelGGL((quant_rows_pre_long_kernel<XT, FMT>), grid, block, 0, st, xv, q, qp, scale, amax, rows, vpr,
                       kblocks);
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows_pre(const void* x, int xt, int rows, int cols, int fmt, uint8_t* q, uint8_t* qp,
                                 float* scale, float* amax, hipStream_t st) {
  if (xt == kBF16) {
    return fmt == kE4M3 ? launch_rows_pre_t<kBF16, kE4M3>(x, rows, cols, q, qp, scale, amax, st)
                        : launch_rows_pre_t<kBF16, kE5M2>(x, rows, cols, q, qp, scale, amax, st);
  }
  return fmt == kE4M3 ? launch_rows_pre_t<kF32, kE4M3>(x, rows, cols, q, qp, scale, amax, st)
                      : launch_rows_pre_t<kF32, kE5M2>(x, rows, cols, q, qp, scale, amax, st);
}

// Blocks of the single-pass kernel that one device holds at once, for this
// instantiation (its register use sets the occupancy; cached per process).
template <int XT, int FMT, bool SR, int V>
static int fused_capacity() {
  // cached per instantiation; concurrent first calls compute the same value
  static std::atomic<int> cached{-1};
  int per_cu = cached.load(std::memory_order_relaxed);
  if (per_cu < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, quant_tensor_fused_kernel<XT, FMT, SR, V>, kBlock, 0) !=
        hipSuccess) {
      (void)hipGetLastError();
      n = 0;
    }
    per_cu = n;
    cached.store(n, std::memory_order_relaxed);
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return per_cu * cus;
}

// Single pass when the tensor fits in the registers of at most kFusedBlocks
// blocks, and the device can hold the whole grid at once; the two-pass path
// otherwise.
template <int XT, int FMT, bool SR, int V>
static bool try_fused(const uint4* xv, size_t nvec, uint8_t* q, float* scale, float* amax, uint32_t* ws, SrSeed sd,
                      hipStream_t st, hipError_t* err) {
  constexpr size_t kPerBlock = (size_t)kBlock * V;
  const size_t grid = (nvec + kPerBlock - 1) / kPerBlock;
  if (grid > (size_t)kFusedBlocks || (int)grid > fused_capacity<XT, FMT, SR, V>()) return false;
  hipLaunchKernelGGL((quant_tensor_fused_kernel<XT, FMT, SR, V>), dim3((unsigned)grid), dim3(kBlock), 0, st, xv, nvec,
                     q, scale, amax, ws, ws + kArrivalOffsetWords, ws + kBarrierOffsetWords, sd);
  *err = hipGetLastError();
  return true;
}

template <int XT, int FMT, bool SR>
static bool launch_fused(const uint4* xv, size_t nvec, uint8_t* q, float* scale, float* amax, uint32_t* ws, SrSeed sd,
                         hipStream_t st, hipError_t* err) {
  constexpr size_t kB = (size_t)kFusedBlocks * kBlock;
  if (nvec <= kB * 4) return try_fused<XT, FMT, SR, 4>(xv, nvec, q, scale, amax, ws, sd, st, err);
  if (nvec <= kB * 8) return try_fused<XT, FMT, SR, 8>(xv, nvec, q, scale, amax, ws, sd, st, err);
  // (the stochastic cast at 16 vectors per thread would spill its registers)
  if (!SR && nvec <= kB * 16) return try_fused<XT, FMT, SR, SR ? 8 : 16>(xv, nvec, q, scale, amax, ws, sd, st, err);
  return false;
}

hipError_t launch_quant_tensor(const void* x, int xt, size_t numel, int fmt, uint8_t* q, float* scale,
                               float* amax, void* ws, bool sr, uint64_t seed, hipStream_t st) {
  const size_t nvec = xt == kBF16 ? numel / 8 : numel / 4;
  const int nb = tensor_partial_blocks(nvec);
  uint32_t* partial = static_cast<uint32_t*>(ws);
  const uint4* xv = static_cast<const uint4*>(x);
  const SrSeed sd = sr_seed(seed);
  size_t qb = (nvec + kBlock * kUnroll - 1) / (kBlock * kUnroll);
  if (qb > 2048) qb = 2048;
  if (qb < 1) qb = 1;
  hipError_t err = hipSuccess;
#define CALL(A, B, S)                                                                                    \
  if (launch_fused<A, B, S>(xv, nvec, q, scale, amax, partial, sd, st, &err)) return err;               \
  hipLaunchKernelGGL((amax_partials_kernel<A>), dim3(nb), dim3(kBlock), 0, st, xv, nvec, partial);        \
  hipLaunchKernelGGL((quant_tensor_kernel<A, B, S>), dim3((unsigned)qb), dim3(kBlock), 0, st, xv, nvec, \
                     (const uint32_t*)partial, nb, q, scale, amax, sd);                                  \
  return hipGetLastError()
  HQ_DISPATCH_XT_FMT_SR(xt, fmt, sr, CALL);
#undef CALL
}

// Blocks of the single-pass per-column kernel one device holds at once.
template <int XT, int FMT, bool SR>
static int cols_fused_capacity() {
  static std::atomic<int> cached{-1};
  int per_cu = cached.load(std::memory_order_relaxed);
  if (per_cu < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, quant_cols_fused_kernel<XT, FMT, SR>, kBlock, 0) !=
        hipSuccess) {
      (void)hipGetLastError();
      n = 0;
    }
    per_cu = n;
    cached.store(n, std::memory_order_relaxed);
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return per_cu * cus;
}

hipError_t launch_quant_cols(const void* x, int xt, int rows, int cols, int fmt, uint8_t* q, float* scale,
                             float* amax, void* ws, bool sr, uint64_t seed, hipStream_t st) {
  const int vpr = xt == kBF16 ? cols / 8 : cols / 4;
  const dim3 grid((vpr + kColVecs - 1) / kColVecs, col_chunks(rows));
  // the column partials of the two-pass form follow the per-tensor region, so
  // one workspace can serve every granularity without disturbing the
  // per-tensor counters; the one-pass form's column words follow them
  uint64_t* partial = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + kTensorWorkspaceBytes);
  uint64_t* colw = partial + (size_t)grid.y * cols;
  const uint4* xv = static_cast<const uint4*>(x);
  const SrSeed sd = sr_seed(seed);
  uint32_t* region = static_cast<uint32_t*>(ws);
  const bool one_pass = (size_t)grid.x * grid.y <= (size_t)kFusedBlocks;
#define CALL(A, B, S)                                                                                       \
  if (one_pass && (int)(grid.x * grid.y) <= cols_fused_capacity<A, B, S>()) {                               \
    hipLaunchKernelGGL((quant_cols_fused_kernel<A, B, S>), grid, dim3(kBlock), 0, st, xv, rows, vpr, colw,    \
                       region + kArrivalOffsetWords, region + kBarrierOffsetWords, q, scale, amax, sd);      \
    return hipGetLastError();                                                                               \
  }                                                                                                         \
  hipLaunchKernelGGL((colmax_partials_kernel<A>), grid, dim3(kBlock), 0, st, xv, rows, vpr, partial);        \
  hipLaunchKernelGGL((quant_cols_kernel<A, B, S>), grid, dim3(kBlock), 0, st, xv, rows, vpr,               \
                     (const uint64_t*)partial, (int)grid.y, q, scale, amax, sd);                           \
  return hipGetLastError()
  HQ_DISPATCH_XT_FMT_SR(xt, fmt, sr, CALL);
#undef CALL
}

hipError_t launch_quant_delayed(const void* x, int xt, size_t numel, int fmt, uint8_t* q, float* scale,
                                float* amax, float* state, int len, int idx, int margin, int32_t* flag, void* ws,
                                bool sr, uint64_t seed, hipStream_t st) {
  const size_t nvec = xt == kBF16 ? numel / 8 : numel / 4;
  const int nb = tensor_partial_blocks(nvec);
  uint32_t* partial = static_cast<uint32_t*>(ws);
  const uint4* xv = static_cast<const uint4*>(x);
  const SrSeed sd = sr_seed(seed);
#define CALL(A, B, S)                                                                                  \
  hipLaunchKernelGGL((quant_delayed_kernel<A, B, S>), dim3(nb), dim3(kBlock), 0, st, xv, nvec, q, scale, \
                     amax, state, len, idx, margin, flag, partial, partial + kArrivalOffsetWords, sd);   \
  return hipGetLastError()
  HQ_DISPATCH_XT_FMT_SR(xt, fmt, sr, CALL);
#undef CALL
}

hipError_t launch_quant_layouts(const void* x, int xt, int rows, int cols, int fmt, const LayoutOut& o,
                                const float* scale_in, float* scale_out, float* amax, float* state, int len, int idx,
                                int margin, int32_t* flag, void* ws, bool sr, uint64_t seed, hipStream_t st) {
  const int tiles = ((rows + 127) / 128) * ((cols + 127) / 128);
  const dim3 grid(min(tiles, kMaxTensorPartials)), block(kBlock);
  const uint4* xv = static_cast<const uint4*>(x);
  uint32_t* partial = static_cast<uint32_t*>(ws);
  uint32_t* arrivals = partial ? partial + kArrivalOffsetWords : nullptr;
  const int mode = scale_in ? kScaleGiven : (state ? kScaleRing : kScaleDynamic);
  const SrSeed sd = sr_seed(seed);
  int ndyn = 0;
  if (mode == kScaleDynamic) {
    const size_t nvec = (size_t)rows * cols / (xt == kBF16 ? 8 : 4);
    ndyn = tensor_partial_blocks(nvec);
    if (xt == kBF16)
      hipLaunchKernelGGL((amax_partials_kernel<kBF16>), dim3(ndyn), dim3(kBlock), 0, st, xv, nvec, partial);
    else
      hipLaunchKernelGGL((amax_partials_kernel<kF32>), dim3(ndyn), dim3(kBlock), 0, st, xv, nvec, partial);
  }
#define LAUNCH_MODE(A, B, S, T)                                                                            \
  do {                                                                                                     \
    if (mode == kScaleGiven)                                                                               \
      hipLaunchKernelGGL((quant_layouts_kernel<A, B, kScaleGiven, S, T>), grid, block, 0, st, xv, rows, cols, o, \
                         scale_in, nullptr, 0, scale_out, amax, state, len, idx, margin, flag, partial, arrivals, sd); \
    else if (mode == kScaleRing)                                                                           \
      hipLaunchKernelGGL((quant_layouts_kernel<A, B, kScaleRing, S, T>), grid, block, 0, st, xv, rows, cols, o, \
                         scale_in, nullptr, 0, scale_out, amax, state, len, idx, margin, flag, partial, arrivals, sd); \
    else                                                                                                   \
      hipLaunchKernelGGL((quant_layouts_kernel<A, B, kScaleDynamic, S, T>), grid, block, 0, st, xv, rows, cols, \
                         o, scale_in, partial, ndyn, scale_out, amax, state, len, idx, margin, flag, partial,   \
                         arrivals, sd);                                                                    \
  } while (0)
#define CALL(A, B, S)                        \
  do {                                       \
    if (o.qt) LAUNCH_MODE(A, B, S, true);    \
    else LAUNCH_MODE(A, B, S, false);        \
    return hipGetLastError();                \
  } while (0)
  HQ_DISPATCH_XT_FMT_SR(xt, fmt, sr, CALL);
#undef CALL
#undef LAUNCH_MODE
}

hipError_t launch_ring_update(float* state, int len, int idx, int margin, int32_t* flag, const float* amax,
                              int fmt, hipStream_t st) {
  if (fmt == kE4M3)
    hipLaunchKernelGGL((ring_update_kernel<kE4M3>), dim3(1), dim3(64), 0, st, state, len, idx, margin, flag, amax);
  else
    hipLaunchKernelGGL((ring_update_kernel<kE5M2>), dim3(1), dim3(64), 0, st, state, len, idx, margin, flag, amax);
  return hipGetLastError();
}

}  // namespace hq
