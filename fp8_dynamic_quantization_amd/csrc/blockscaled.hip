// Block-wise FP8 scaling and the block-scaled a8w8 GEMM, gfx950.
//
// What is computed (hip-quant README, "Block-wise FP8 Scaling" and "Block-scaled
// Linear and Adafactor Kernel Helpers"): FP8 codes plus one float32 dequant
// scale per block of BS consecutive elements along the last dimension (scales
// [rows, ceil(cols / BS)]); each block follows the rule of the other
// granularities (amax over its finite elements, s = max(amax / fmax, 2^-126),
// r = 1 / s, saturating RNE cast of x * r, or the stochastic E5M2 cast). The
// block-scaled GEMM consumes codes and block scales of both operands:
//   out[m, n] = bf16( sum_b xs[m, b] * ws[n, b] * sum_{k in block b} dec(XQ[m,k]) * dec(WQ[n,k]) )
//
// GEMM design. Per-block float32 scales cannot ride on the MFMA's hardware
// block scales (those are powers of two), so every block's partial sum is
// formed on its own from a zero accumulator, and one FMA per output element
// folds the partial into the running sum with the scale product xs * ws. The
// rescale costs two VALU operations per output element per block, which for
// BS = 32 is more issue time than the MFMAs themselves: that GEMM is bound by
// this arithmetic, not by HBM or the matrix cores.
#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

typedef float bv4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// block-wise quantization
// ---------------------------------------------------------------------------
// Max over aligned groups of G lanes (G a power of two up to 64); every lane
// of a group gets the group's max. Within a row of 16 lanes the partners come
// from DPP lane moves (quad permutations swapping neighbours and pairs, then
// the half-row and row mirrors, which pair each quad with the one it is
// mirrored onto); wider groups finish with cross-row shuffles.
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
  if constexpr (G >= 2) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadSwap1, 0xF, 0xF, false));
  if constexpr (G >= 4) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadSwap2, 0xF, 0xF, false));
  if constexpr (G >= 8) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowHalfMirror, 0xF, 0xF, false));
  if constexpr (G >= 16) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowMirror, 0xF, 0xF, false));
  if constexpr (G >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  if constexpr (G >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
  return v;
}

// One wavefront per row (rows w, w + W, ...); lane l holds vectors l + 64j.
// A row is taken in chunks of U vectors per lane, and the next chunk (of this
// row or of the wavefront's next row) is loaded before the current one is
// processed, so every lane keeps up to 2U loads in flight.
// A block of BS elements is G = BS / E consecutive lanes (E elements per
// 16-byte vector), so its amax is a shuffle reduction over G lanes. Lanes past
// the row end reload the row's last vector, which lies in the row's last
// block: it cannot change that block's max, and groups wholly past the end
// store nothing.
template <int XT, int FMT, int BS, bool SR>
__global__ __launch_bounds__(256) void quant_blocks_kernel(const uint4* __restrict__ x, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale, float* __restrict__ amax_out,
                                                           int rows, int vpr, int nb, SrSeed sd) {
  constexpr int E = VecTraits<XT>::kElems;
  constexpr int G = BS / E;  // lanes per block
  constexpr int U = 8;       // vectors per lane per chunk
  constexpr int CB = 64 * U * E / BS;  // blocks per chunk
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "block of whole vectors, power-of-two lanes");
  // a chunk's scales and maxima, gathered per wavefront for coalesced stores
  __shared__ float sb[4][2][CB];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // row indices step in 64 bits: rows up to 2^31 - 1 would overflow row + W
  const int64_t W = (int64_t)gridDim.x * 4;
  const int cpr = (vpr + 64 * U - 1) / (64 * U);  // chunks per row
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int c = 0;
  if (row >= rows) return;
  auto load = [&](uint4 (&v)[U], int64_t r, int ch) {
    const uint4* xr = x + (size_t)r * vpr;
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = xr[min(lane + 64 * (ch * U + u), vpr - 1)];
  };
  uint4 cur[U];
  load(cur, row, 0);
  while (row < rows) {
    int64_t nrow = row;
    int nc = c + 1;
    if (nc == cpr) {
      nc = 0;
      nrow += W;
    }
    uint4 nxt[U];
    if (nrow < rows) load(nxt, nrow, nc);  // wavefront-uniform
    uint8_t* qr = q + (size_t)row * vpr * E;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = c * U + u;
      if (j * 64 >= vpr) break;  // wavefront-uniform
      const int i = lane + 64 * j;
      const uint32_t own = vec_absmax_raw<XT>(cur[u]);
      uint32_t fin = own;
      if (__any(own >= kInfBits)) {  // rare: some vector holds an Inf or NaN
        if (own >= kInfBits) fin = vec_absmax_finite<XT>(cur[u]);
      }
      fin = group_max_u32<G>(fin);
      const float am = __uint_as_float(fin);
      const float s = scale_from_amax<FMT>(am);
      const float r = 1.0f / s;
      if (i < vpr) {
        if (lane % G == 0) {
          const int t = (lane + 64 * u) * E / BS;  // block within the chunk
          sb[wv][0][t] = s;
          sb[wv][1][t] = am;
        }
        uint32_t w[E / 4];
        cast_vec<XT, FMT, SR, true>(cur[u], r, own, w, sd, ((size_t)row * vpr + i) * E);
        store_codes<E>(qr + (size_t)i * E, w);
      }
    }
    // LDS operations of one wavefront complete in order: the chunk's entries
    // are in place for the reads below, and those reads finish before the
    // next chunk overwrites them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int b0 = c * CB;
#pragma unroll
    for (int t = lane; t < CB; t += 64) {
      if (b0 + t < nb) {
        const size_t si = (size_t)row * nb + b0 + t;
        __builtin_nontemporal_store(sb[wv][0][t], scale + si);
        if (amax_out) __builtin_nontemporal_store(sb[wv][1][t], amax_out + si);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    row = nrow;
    c = nc;
  }
}

hipError_t launch_quant_blocks(const void* x, int xt, int rows, int cols, int fmt, int bs, bool sr, uint64_t seed,
                               uint8_t* q, float* scale, float* amax, hipStream_t st) {
  const int vpr = xt == kBF16 ? cols / 8 : cols / 4;
  const int nb = (cols + bs - 1) / bs;
  const SrSeed sd{(uint32_t)seed, (uint32_t)(seed >> 32)};
  // 16 wavefronts per CU (measured best for [4096, 4096]: one row each)
  const dim3 grid((int)std::min<int64_t>(((int64_t)rows + 3) / 4, kNumCUs * 4)), block(256);
  const uint4* xv = static_cast<const uint4*>(x);
#define HQ_BLK(XT_, FMT_, BS_, SR_)                                                                            \
  hipLaunchKernelGGL((quant_blocks_kernel<XT_, FMT_, BS_, SR_>), grid, block, 0, st, xv, q, scale, amax, rows, vpr, \
                     nb, sd)
#define HQ_BLK_BS(XT_, FMT_, SR_)            \
  do {                                       \
    if (bs == 16) HQ_BLK(XT_, FMT_, 16, SR_);  \
    else if (bs == 32) HQ_BLK(XT_, FMT_, 32, SR_); \
    else if (bs == 64) HQ_BLK(XT_, FMT_, 64, SR_); \
    else HQ_BLK(XT_, FMT_, 128, SR_);        \
  } while (0)
  if (sr) {
    if (xt == kBF16) HQ_BLK_BS(kBF16, kE5M2, true);
    else HQ_BLK_BS(kF32, kE5M2, true);
  } else if (xt == kBF16) {
    if (fmt == kE4M3) HQ_BLK_BS(kBF16, kE4M3, false);
    else HQ_BLK_BS(kBF16, kE5M2, false);
  } else {
    if (fmt == kE4M3) HQ_BLK_BS(kF32, kE4M3, false);
    else HQ_BLK_BS(kF32, kE5M2, false);
  }
#undef HQ_BLK_BS
#undef HQ_BLK
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// block-scaled GEMM
// ---------------------------------------------------------------------------
// A 128 x 128 output tile per workgroup, two workgroups per CU (2 x 76 KB of
// LDS), so one wavefront's rescaling arithmetic runs while another's MFMAs
// issue. Each wavefront owns 64 rows x 16*NJ columns as 4 x NJ MFMA tiles of
// 16 x 16: NJ = 2 (8 wavefronts, at most 128 registers each) for blocks of 32,
// whose folds dominate, and NJ = 4 (4 wavefronts, at most 256 registers) for
// blocks of 64 and 128, where the larger tile halves the LDS reads per MFMA
// (measured: 235 vs 258 us at BS = 32, 197 vs 220 and 140 vs 162 us at BS = 64
// and 128, 4096^3, full-range codes). K moves in steps of 128 through
// double-buffered LDS (one barrier per step): the codes and block scales of
// step kb + 1 are loaded into registers while step kb computes.
//
// The weight is the MFMA's A operand and the activation its B operand, so an
// output lane holds one row m and four consecutive columns n (8-byte stores).
// Blocks of 128 take one 16x16x128 MFMA per tile (hardware block scales left
// at 1); blocks of 32 and 64 take one or two 16x16x32 MFMAs.
namespace bsg {
constexpr int kBM = 128, kBN = 128, kBK = 128;
template <int NJ>
constexpr int threads() { return 64 * 2 * (8 / NJ); }
}  // namespace bsg

// 16x16x32 FP8 MFMA, weight (format WF) as A and activation (XF) as B: lane l
// gives A row l%16 and B column l%16, each with the 8 k values 8*(l/16) .. +7;
// the result lane l holds B column l%16 (output row m) and A rows
// 4*(l/16) .. +3 (output columns n).
template <int XF, int WF>
__device__ __forceinline__ bv4f mfma32(long w, long x, bv4f c) {
  if constexpr (WF == kE4M3 && XF == kE4M3) return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(w, x, c, 0, 0, 0);
  else if constexpr (WF == kE4M3) return __builtin_amdgcn_mfma_f32_16x16x32_fp8_bf8(w, x, c, 0, 0, 0);
  else if constexpr (XF == kE4M3) return __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(w, x, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf8_bf8(w, x, c, 0, 0, 0);
}

// Tile order as the plain GEMM: workgroup b on XCD b % 8 takes a contiguous
// run of tiles, numbered in groups of 4 tile rows (column-major in a group).
__device__ __forceinline__ void bs_tile_coords(int b, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int total = tiles_m * tiles_n;
  const int t = total % 8 == 0 ? (b % 8) * (total / 8) + b / 8 : b;
  const int per_group = 4 * tiles_n;
  const int g = t / per_group;
  const int first_m = g * 4;
  const int gm = min(4, tiles_m - first_m);
  const int r = t % per_group;
  *tm = first_m + r % gm;
  *tn = r / gm;
}

template <int XF, int WF, int BS, int NJ>
__global__ __launch_bounds__(bsg::threads<NJ>()) __attribute__((amdgpu_waves_per_eu(NJ == 2 ? 4 : 2))) void gemm_blockscaled_kernel(BlockGemmArgs a, int tiles_m, int tiles_n) {
  using namespace bsg;
  constexpr int NBS = kBK / BS;                // scale blocks per K step
  constexpr int SUB = BS / 32;                 // 16x16x32 MFMAs per block (BS < 128)
  constexpr int kPitch = BS == 128 ? 144 : 136;  // LDS row pitch: 16-byte rows for the 128-wide reads
  constexpr int kStage = kBM * kPitch;
  constexpr int kThreads = threads<NJ>();
  constexpr int NP = kBM * kBK / 16 / kThreads;  // 16-byte pieces per thread per operand
  constexpr int NSC = (kBM * NBS + kThreads - 1) / kThreads;  // scale loads per thread per operand
  __shared__ __attribute__((aligned(16))) uint8_t sx[2][kStage];
  __shared__ __attribute__((aligned(16))) uint8_t sw[2][kStage];
  __shared__ __attribute__((aligned(16))) float sxs[2][NBS][kBM];
  __shared__ __attribute__((aligned(16))) float sws[2][NBS][kBN];
  int tm, tn;
  bs_tile_coords(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // 64-row half, 16*NJ-column slice
  const int K = a.k, nkb = (K + kBK - 1) / kBK;

  // staging: piece p = tid + kThreads * v of an operand stage is row p / 8, 16-byte
  // chunk p % 8. Rows past M or N only feed outputs that are never stored, so
  // their loads read a clamped row and are not zeroed; only the K tail of the
  // last step (K % 128 != 0) must read as zero codes, and scales past the last
  // block as zero. No load sits behind a branch.
  uint4 rx[NP], rw[NP];
  float rxs[NSC], rws[NSC];
  auto load = [&](int kb) {
    const bool tail = kb + 1 == nkb && (K & (kBK - 1)) != 0;
#pragma unroll
    for (int v = 0; v < NP; ++v) {
      const int p = tid + kThreads * v, row = p >> 3, kk = kb * kBK + (p & 7) * 16;
      const int kc = min(kk, K - 16);
      const int xr = min(m0 + row, a.m - 1), wr = min(n0 + row, a.n - 1);
      rx[v] = *reinterpret_cast<const uint4*>(a.xq + (size_t)xr * K + kc);
      rw[v] = *reinterpret_cast<const uint4*>(a.wq + (size_t)wr * K + kc);
      if (tail && kk >= K) {
        rx[v] = make_uint4(0u, 0u, 0u, 0u);
        rw[v] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int e = 0; e < NSC; ++e) {
      const int idx = tid + kThreads * e, row = idx / NBS, gb = kb * NBS + idx % NBS;
      if (kBM * NBS % kThreads == 0 || idx < kBM * NBS) {  // whole wavefronts
        const int gc = min(gb, a.nb - 1);
        const int xr = min(m0 + row, a.m - 1), wr = min(n0 + row, a.n - 1);
        rxs[e] = a.xs[(size_t)xr * a.nb + gc];
        rws[e] = a.ws[(size_t)wr * a.nb + gc];
        if (tail && gb >= a.nb) rxs[e] = rws[e] = 0.0f;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int v = 0; v < NP; ++v) {
      const int p = tid + kThreads * v, off = (p >> 3) * kPitch + (p & 7) * 16;
      *reinterpret_cast<uint4*>(&sx[buf][off]) = rx[v];
      *reinterpret_cast<uint4*>(&sw[buf][off]) = rw[v];
    }
#pragma unroll
    for (int e = 0; e < NSC; ++e) {
      const int idx = tid + kThreads * e;
      if (idx < kBM * NBS) {
        sxs[buf][idx % NBS][idx / NBS] = rxs[e];
        sws[buf][idx % NBS][idx / NBS] = rws[e];
      }
    }
  };

  bv4f acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = bv4f{0.f, 0.f, 0.f, 0.f};

  const int xrow = wm * 64 + (lane & 15);           // + 16 i
  const int wrow = wn * 16 * NJ + (lane & 15);      // + 16 j
  const int wcol = wn * 16 * NJ + 4 * (lane >> 4);  // + 16 j + r: the lane's output columns
  load(0);
  store(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load(kb + 1);
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      bv4f t[4][NJ];
      if constexpr (BS == 128) {
        const int kofs = 32 * (lane >> 4);
        v8i fw[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const uint8_t* pw = &sw[buf][(wrow + 16 * j) * kPitch + kofs];
          const uint4 lo = *reinterpret_cast<const uint4*>(pw), hi = *reinterpret_cast<const uint4*>(pw + 16);
          fw[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint8_t* px = &sx[buf][(xrow + 16 * i) * kPitch + kofs];
          const uint4 lo = *reinterpret_cast<const uint4*>(px), hi = *reinterpret_cast<const uint4*>(px + 16);
          const v8i fx = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            t[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw[j], fx, bv4f{0.f, 0.f, 0.f, 0.f}, WF, XF,
                                                                       0, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          const int kofs = b * BS + s * 32 + 8 * (lane >> 4);
          long fw[NJ], fx[4];
#pragma unroll
          for (int j = 0; j < NJ; ++j) fw[j] = *reinterpret_cast<const long*>(&sw[buf][(wrow + 16 * j) * kPitch + kofs]);
#pragma unroll
          for (int i = 0; i < 4; ++i) fx[i] = *reinterpret_cast<const long*>(&sx[buf][(xrow + 16 * i) * kPitch + kofs]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              t[i][j] = mfma32<XF, WF>(fw[j], fx[i], s == 0 ? bv4f{0.f, 0.f, 0.f, 0.f} : t[i][j]);
        }
      }
      // fold the block's partials: acc += t * (xs[m] * ws[n])
      bv4f wsv[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) wsv[j] = *reinterpret_cast<const bv4f*>(&sws[buf][b][wcol + 16 * j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xsv = sxs[buf][b][xrow + 16 * i];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(t[i][j][r], xsv * wsv[j][r], acc[i][j][r]);
      }
      // one block's partials live at a time: the empty asm makes this block's
      // folds complete here (the other wavefronts on the SIMD overlap their
      // MFMAs with them)
      if constexpr (NBS > 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(acc[i][j]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (kb + 1 < nkb) store(buf ^ 1);
    __syncthreads();
  }

  // epilogue: the bias (output units) added in float32, then four consecutive
  // columns per lane as one 8-byte store where the row's columns allow it
  if (a.bias) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = min(n0 + wcol + 16 * j + r, a.n - 1);
        const float b = __uint_as_float((uint32_t)a.bias[col] << 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j][r] += b;
      }
  }
  const bool vec = (a.n % 4 == 0) && (reinterpret_cast<uintptr_t>(a.out) % 8 == 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + xrow + 16 * i;
    if (row >= a.m) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + wcol + 16 * j;
      uint16_t* o = a.out + (size_t)row * a.n + col;
      if (vec && col + 3 < a.n) {
        // non-temporal: the output is written once and never read here
        const hq_u2v pk = {f32_to_bf16_rne(acc[i][j][0]) | (f32_to_bf16_rne(acc[i][j][1]) << 16),
                           f32_to_bf16_rne(acc[i][j][2]) | (f32_to_bf16_rne(acc[i][j][3]) << 16)};
        __builtin_nontemporal_store(pk, reinterpret_cast<hq_u2v*>(o));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (col + r < a.n) o[r] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
      }
    }
  }
}

hipError_t launch_gemm_blockscaled(const BlockGemmArgs& a, int xf, int wf, int bs, hipStream_t st) {
  const int tiles_m = (a.m + bsg::kBM - 1) / bsg::kBM, tiles_n = (a.n + bsg::kBN - 1) / bsg::kBN;
  const dim3 grid(tiles_m * tiles_n);
#define HQ_BSG_ONE(X_, W_, BS_, NJ_)                                                                       \
  hipLaunchKernelGGL((gemm_blockscaled_kernel<X_, W_, BS_, NJ_>), grid, dim3(bsg::threads<NJ_>()), 0, st, a, \
                     tiles_m, tiles_n)
#define HQ_BSG(X_, W_)                             \
  do {                                             \
    if (bs == 32) HQ_BSG_ONE(X_, W_, 32, 2);       \
    else if (bs == 64) HQ_BSG_ONE(X_, W_, 64, 4);  \
    else HQ_BSG_ONE(X_, W_, 128, 4);               \
  } while (0)
  if (xf == kE4M3 && wf == kE4M3) HQ_BSG(kE4M3, kE4M3);
  else if (xf == kE4M3) HQ_BSG(kE4M3, kE5M2);
  else if (wf == kE4M3) HQ_BSG(kE5M2, kE4M3);
  else HQ_BSG(kE5M2, kE5M2);
#undef HQ_BSG
#undef HQ_BSG_ONE
  return hipGetLastError();
}

}  // namespace hq
