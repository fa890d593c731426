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
// formed on its own: 16x16x32 FP8 MFMAs (one per 32 elements of K) start from
// a zero accumulator, and one FMA per output element folds the partial into
// the running sum with the scale product xs * ws. The rescale costs two VALU
// operations per output element per block, which for BS = 32 is more issue
// time than the MFMAs themselves: this GEMM is bound by that arithmetic, not
// by HBM or the matrix cores.
#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

typedef float bv4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// block-wise quantization
// ---------------------------------------------------------------------------
// One wavefront per row (rows w, w + W, ...); lane l holds vectors l + 64j.
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
  constexpr int U = 4;       // vectors in flight per lane
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "block of whole vectors, power-of-two lanes");
  const int lane = threadIdx.x & 63;
  const int W = gridDim.x * 4;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += W) {
    const uint4* xr = x + (size_t)row * vpr;
    uint8_t* qr = q + (size_t)row * vpr * E;
    for (int j0 = 0; j0 * 64 < vpr; j0 += U) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = xr[min(lane + 64 * (j0 + u), vpr - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if ((j0 + u) * 64 >= vpr) break;  // wavefront-uniform
        const int i = lane + 64 * (j0 + u);
        const uint32_t own = vec_absmax_raw<XT>(v[u]);
        uint32_t raw = own;
        uint32_t fin = own < kInfBits ? own : vec_absmax_finite<XT>(v[u]);
#pragma unroll
        for (int off = 1; off < G; off <<= 1) {
          raw = max(raw, (uint32_t)__shfl_xor((int)raw, off, 64));
          fin = max(fin, (uint32_t)__shfl_xor((int)fin, off, 64));
        }
        const float am = __uint_as_float(fin);
        const float s = scale_from_amax<FMT>(am);
        const float r = 1.0f / s;
        if (i < vpr) {
          if (lane % G == 0) {
            const size_t si = (size_t)row * nb + (size_t)i * E / BS;
            scale[si] = s;
            if (amax_out) amax_out[si] = am;
          }
          uint32_t w[E / 4];
          cast_vec<XT, FMT, SR>(v[u], r, own, w, sd, ((size_t)row * vpr + i) * E);
          store_codes<E>(qr + (size_t)i * E, w);
        }
      }
    }
  }
}

hipError_t launch_quant_blocks(const void* x, int xt, int rows, int cols, int fmt, int bs, bool sr, uint64_t seed,
                               uint8_t* q, float* scale, float* amax, hipStream_t st) {
  const int vpr = xt == kBF16 ? cols / 8 : cols / 4;
  const int nb = (cols + bs - 1) / bs;
  const SrSeed sd{(uint32_t)seed, (uint32_t)(seed >> 32)};
  const dim3 grid(min((rows + 3) / 4, kNumCUs * 3)), block(256);
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
namespace bsg {
constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kPitch = 136;  // LDS row pitch in bytes: 8 bytes of padding spread 16 rows over all banks
constexpr int kStage = kBM * kPitch;
}  // namespace bsg

// 16x16x32 FP8 MFMA with the activation (format XF) as A and the weight (WF)
// as B: lane l gives A row l%16 and B column l%16, each with the 8 k values
// 8*(l/16) .. +7; the result lane l holds column l%16, rows 4*(l/16) .. +3.
template <int XF, int WF>
__device__ __forceinline__ bv4f mfma32(long a, long b, bv4f c) {
  if constexpr (XF == kE4M3 && WF == kE4M3) return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
  else if constexpr (XF == kE4M3) return __builtin_amdgcn_mfma_f32_16x16x32_fp8_bf8(a, b, c, 0, 0, 0);
  else if constexpr (WF == kE4M3) return __builtin_amdgcn_mfma_f32_16x16x32_bf8_fp8(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf8_bf8(a, b, c, 0, 0, 0);
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

template <int XF, int WF, int BS>
__global__ __launch_bounds__(256) void gemm_blockscaled_kernel(BlockGemmArgs a, int tiles_m, int tiles_n) {
  using namespace bsg;
  constexpr int NBS = kBK / BS;  // scale blocks per K step
  constexpr int SUB = BS / 32;   // 16x16x32 MFMAs per block
  constexpr int NSC = (kBM * NBS + 255) / 256;  // scale loads per thread per operand
  __shared__ __attribute__((aligned(16))) uint8_t sa[2][kStage];
  __shared__ __attribute__((aligned(16))) uint8_t sb[2][kStage];
  __shared__ float sxs[2][kBM * NBS];
  __shared__ float sws[2][kBN * NBS];
  int tm, tn;
  bs_tile_coords(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;  // 2 x 2 wavefronts of 64 x 64
  const int K = a.k, nkb = (K + kBK - 1) / kBK;

  // staging: piece p = tid + 256 v of an operand stage is row p / 8, 16-byte chunk p % 8
  uint4 ra[4], rb[4];
  float rxs[NSC], rws[NSC];
  auto load = [&](int kb) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = tid + 256 * v, row = p >> 3, kk = kb * kBK + (p & 7) * 16;
      ra[v] = (m0 + row < a.m && kk < K) ? *reinterpret_cast<const uint4*>(a.xq + (size_t)(m0 + row) * K + kk)
                                         : make_uint4(0u, 0u, 0u, 0u);
      rb[v] = (n0 + row < a.n && kk < K) ? *reinterpret_cast<const uint4*>(a.wq + (size_t)(n0 + row) * K + kk)
                                         : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int e = 0; e < NSC; ++e) {
      const int idx = tid + 256 * e, row = idx / NBS, gb = kb * NBS + idx % NBS;
      const bool in = idx < kBM * NBS && gb < a.nb;
      rxs[e] = in && m0 + row < a.m ? a.xs[(size_t)(m0 + row) * a.nb + gb] : 0.0f;
      rws[e] = in && n0 + row < a.n ? a.ws[(size_t)(n0 + row) * a.nb + gb] : 0.0f;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = tid + 256 * v, off = (p >> 3) * kPitch + (p & 7) * 16;
      *reinterpret_cast<uint4*>(&sa[buf][off]) = ra[v];
      *reinterpret_cast<uint4*>(&sb[buf][off]) = rb[v];
    }
#pragma unroll
    for (int e = 0; e < NSC; ++e) {
      const int idx = tid + 256 * e;
      if (idx < kBM * NBS) {
        sxs[buf][idx] = rxs[e];
        sws[buf][idx] = rws[e];
      }
    }
  };

  bv4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = bv4f{0.f, 0.f, 0.f, 0.f};

  const int arow = wr * 64 + (lane & 15), brow = wc * 64 + (lane & 15), kofs = 8 * (lane >> 4);
  load(0);
  store(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load(kb + 1);
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      float wsv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wsv[j] = sws[buf][(brow + j * 16) * NBS + b];
      // the wavefront's 4 x 4 tiles in two halves of two row tiles, so only 8
      // partial sums are live at a time
#pragma unroll
      for (int ih = 0; ih < 2; ++ih) {
        float xsv[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            xsv[i][r] = sxs[buf][(wr * 64 + (2 * ih + i) * 16 + 4 * (lane >> 4) + r) * NBS + b];
        bv4f t[2][4];
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          long fa[2], fb[4];
#pragma unroll
          for (int i = 0; i < 2; ++i)
            fa[i] = *reinterpret_cast<const long*>(
                &sa[buf][(arow + (2 * ih + i) * 16) * kPitch + b * BS + s * 32 + kofs]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            fb[j] = *reinterpret_cast<const long*>(&sb[buf][(brow + j * 16) * kPitch + b * BS + s * 32 + kofs]);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              t[i][j] = mfma32<XF, WF>(fa[i], fb[j], s == 0 ? bv4f{0.f, 0.f, 0.f, 0.f} : t[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[2 * ih + i][j][r] = fmaf(t[i][j][r], xsv[i][r] * wsv[j], acc[2 * ih + i][j][r]);
      }
    }
    if (kb + 1 < nkb) store(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wc * 64 + j * 16 + (lane & 15);
      if (col >= a.n) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wr * 64 + i * 16 + 4 * (lane >> 4) + r;
        if (row < a.m) a.out[(size_t)row * a.n + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
      }
    }
}

hipError_t launch_gemm_blockscaled(const BlockGemmArgs& a, int xf, int wf, int bs, hipStream_t st) {
  const int tiles_m = (a.m + bsg::kBM - 1) / bsg::kBM, tiles_n = (a.n + bsg::kBN - 1) / bsg::kBN;
  const dim3 grid(tiles_m * tiles_n), block(256);
#define HQ_BSG(X_, W_)                                                                                          \
  do {                                                                                                         \
    if (bs == 32) hipLaunchKernelGGL((gemm_blockscaled_kernel<X_, W_, 32>), grid, block, 0, st, a, tiles_m, tiles_n); \
    else if (bs == 64) hipLaunchKernelGGL((gemm_blockscaled_kernel<X_, W_, 64>), grid, block, 0, st, a, tiles_m, tiles_n); \
    else hipLaunchKernelGGL((gemm_blockscaled_kernel<X_, W_, 128>), grid, block, 0, st, a, tiles_m, tiles_n); \
  } while (0)
  if (xf == kE4M3 && wf == kE4M3) HQ_BSG(kE4M3, kE4M3);
  else if (xf == kE4M3) HQ_BSG(kE4M3, kE5M2);
  else if (wf == kE4M3) HQ_BSG(kE5M2, kE4M3);
  else HQ_BSG(kE5M2, kE5M2);
#undef HQ_BSG
  return hipGetLastError();
}

}  // namespace hq
