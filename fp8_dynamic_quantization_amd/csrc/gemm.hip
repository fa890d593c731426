// Scaled FP8 (a8w8) GEMM, its grouped form and the weight pre-shuffle, gfx950.
//
//   out[m, n] = bf16_rne( sum_k dec(XQ[m,k]) * dec(WQ[n,k]) * x_scale[m] * w_scale[n] )
//
// (the method statement; operand set of the aiter PR "gemm_a8w8_bpreshuffle_out";
// NT layout of AstrAI's linear_forward_fp8). The contraction runs on the gfx950
// V_MFMA_F32_16X16X128_F8F6F4 instruction (FP8/BF8 selected per operand), fp32
// accumulators, and a fused scale + bf16 epilogue.
//
// Operand register layout of one 16x16x128 MFMA (per 64-lane wavefront): lane l
// holds row (or column) l % 16 and the 32 consecutive k values
// 32*(l/16) .. 32*(l/16)+31 of both A and B; the 4 results of lane l are
// column l % 16, rows 4*(l/16) + 0..3.
//
// Tiling: a workgroup computes a BM x BN output tile with WAVES_M x WAVES_N
// wavefronts; K advances in steps of 128 through double-buffered LDS:
//   A (XQ, row-major) is staged with an XOR swizzle of its 16-byte chunks
//     (chunk c of row r at slot c ^ (r & 7)) so both the row-wise stores and the
//     MFMA-order reads are free of bank conflicts;
//   B (pre-shuffled WQ) is copied verbatim: a 2048-byte fragment is already in
//     MFMA lane order, so each wavefront reads it as 64 consecutive 16-byte pieces.
// Tails: rows past M are clamped on load and masked on store; weight fragments past
// the last 16-column block are clamped on load and masked on store; the K tail of
// A is zero-filled (the pre-shuffled B is zero-padded to a multiple of 128).
#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;          // K per pipeline stage = one MFMA
constexpr int kFragBytes = 2048;  // 16 rows x 128 k

// ---------------------------------------------------------------------------
// pre-shuffle
// ---------------------------------------------------------------------------
// One thread per 16-byte piece of the output: piece P of fragment (nb, kb) holds
// h = P / 64, lane = P % 64 -> row nb*16 + lane%16, columns kb*128 + 32*(lane/16)
// + 16*h .. +15.
__global__ __launch_bounds__(256) void preshuffle_kernel(const uint8_t* __restrict__ wq, int n, int k, int kblocks,
                                                         size_t npieces, uint8_t* __restrict__ out) {
  const size_t pc = blockIdx.x * (size_t)256 + threadIdx.x;
  if (pc >= npieces) return;
  const size_t frag = pc / 128;
  const int p = (int)(pc % 128);
  const int h = p / 64, lane = p % 64;
  const int nb = (int)(frag / kblocks), kb = (int)(frag % kblocks);
  const int row = nb * 16 + (lane & 15);
  const int col = kb * kBK + (lane >> 4) * 32 + h * 16;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < n && col < k) v = *reinterpret_cast<const uint4*>(wq + (size_t)row * k + col);
  *reinterpret_cast<uint4*>(out + pc * 16) = v;
}

hipError_t launch_preshuffle(const uint8_t* wq, int n, int k, uint8_t* out, hipStream_t st) {
  const int nblocks16 = (n + 15) / 16;
  const int kblocks = (k + kBK - 1) / kBK;
  const size_t npieces = (size_t)nblocks16 * kblocks * 128;
  const size_t grid = (npieces + 255) / 256;
  hipLaunchKernelGGL(preshuffle_kernel, dim3((unsigned)grid), dim3(256), 0, st, wq, n, k, kblocks, npieces, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct TileCfg {
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kTM = BM / WAVES_M, kTN = BN / WAVES_N;
  static constexpr int kIM = kTM / 16, kIN = kTN / 16;
  static constexpr int kAVec = BM * 8 / kThreads;  // 16-byte A pieces per thread per stage
  static constexpr int kBVec = BN * 8 / kThreads;  // 16-byte B pieces per thread per stage
  static constexpr int kABytes = BM * kBK, kBBytes = BN * kBK;
  static constexpr int kStage = kABytes + kBBytes;
  static_assert(BM % (16 * WAVES_M) == 0 && BN % (16 * WAVES_N) == 0, "tile");
  static_assert((BM * 8) % kThreads == 0 && (BN * 8) % kThreads == 0, "loads");
};

// One output tile. Rows [m0, row_end) are valid (row_end > m0); weight `wq`
// points at this operand's pre-shuffled matrix; `ws` at its scales.
template <int XF, int WF, int BM, int BN, int WAVES_M, int WAVES_N>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, uint8_t* lds, int m0, int row_end, int n0,
                                          const uint8_t* __restrict__ wq, const float* __restrict__ ws) {
  using C = TileCfg<BM, BN, WAVES_M, WAVES_N>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int K = a.k;
  const int nkb = (K + kBK - 1) / kBK;
  const int nblk16 = (a.n + 15) / 16;

  // global source offsets (constant across K steps)
  size_t a_src[C::kAVec];
  int a_col[C::kAVec], a_dst[C::kAVec];
#pragma unroll
  for (int v = 0; v < C::kAVec; ++v) {
    const int L = v * C::kThreads + tid;
    const int r = L >> 3, c = L & 7;
    const int grow = min(m0 + r, row_end - 1);
    a_src[v] = (size_t)grow * K + c * 16;
    a_col[v] = c * 16;
    a_dst[v] = r * kBK + ((c ^ (r & 7)) << 4);
  }
  size_t b_src[C::kBVec];
  int b_dst[C::kBVec];
#pragma unroll
  for (int v = 0; v < C::kBVec; ++v) {
    const int L = v * C::kThreads + tid;
    const int f = L >> 7, p = L & 127;
    const int nb = min(n0 / 16 + f, nblk16 - 1);
    b_src[v] = (size_t)nb * nkb * kFragBytes + p * 16;
    b_dst[v] = C::kABytes + f * kFragBytes + p * 16;
  }

  v4f acc[C::kIM][C::kIN];
#pragma unroll
  for (int i = 0; i < C::kIM; ++i)
#pragma unroll
    for (int j = 0; j < C::kIN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // MFMA-order read offsets inside a stage
  int a_rd0[C::kIM], a_rd1[C::kIM];
#pragma unroll
  for (int i = 0; i < C::kIM; ++i) {
    const int r = wm * C::kTM + i * 16 + (lane & 15);
    const int c0 = 2 * (lane >> 4), c1 = c0 + 1;
    a_rd0[i] = r * kBK + ((c0 ^ (r & 7)) << 4);
    a_rd1[i] = r * kBK + ((c1 ^ (r & 7)) << 4);
  }
  const int b_rd = C::kABytes + (wn * C::kIN) * kFragBytes + lane * 16;

  uint4 ra[C::kAVec], rb[C::kBVec];
#define HQ_LOAD_STAGE(KB)                                                                              \
  do {                                                                                                 \
    const int k0_ = (KB) * kBK;                                                                        \
    _Pragma("unroll") for (int v = 0; v < C::kAVec; ++v) {                                             \
      ra[v] = make_uint4(0u, 0u, 0u, 0u);                                                              \
      if (k0_ + a_col[v] < K) ra[v] = *reinterpret_cast<const uint4*>(a.xq + a_src[v] + k0_);          \
    }                                                                                                  \
    _Pragma("unroll") for (int v = 0; v < C::kBVec; ++v)                                               \
      rb[v] = *reinterpret_cast<const uint4*>(wq + b_src[v] + (size_t)(KB) * kFragBytes);              \
  } while (0)
#define HQ_STORE_STAGE(BUF)                                                                            \
  do {                                                                                                 \
    uint8_t* base_ = lds + (BUF) * C::kStage;                                                          \
    _Pragma("unroll") for (int v = 0; v < C::kAVec; ++v) *reinterpret_cast<uint4*>(base_ + a_dst[v]) = ra[v]; \
    _Pragma("unroll") for (int v = 0; v < C::kBVec; ++v) *reinterpret_cast<uint4*>(base_ + b_dst[v]) = rb[v]; \
  } while (0)

  HQ_LOAD_STAGE(0);
  HQ_STORE_STAGE(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) HQ_LOAD_STAGE(kb + 1);
    const uint8_t* base = lds + cur * C::kStage;
    v8i fa[C::kIM], fb[C::kIN];
#pragma unroll
    for (int i = 0; i < C::kIM; ++i) {
      const uint4 lo = *reinterpret_cast<const uint4*>(base + a_rd0[i]);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + a_rd1[i]);
      fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < C::kIN; ++j) {
      const uint4 lo = *reinterpret_cast<const uint4*>(base + b_rd + j * kFragBytes);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + b_rd + j * kFragBytes + 1024);
      fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < C::kIM; ++i)
#pragma unroll
      for (int j = 0; j < C::kIN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], XF, WF, 0, 0, 0, 0);
    if (kb + 1 < nkb) HQ_STORE_STAGE(cur ^ 1);
    __syncthreads();
  }
#undef HQ_LOAD_STAGE
#undef HQ_STORE_STAGE

  // epilogue: scale, round to bf16, store (rows past row_end and columns past n masked)
#pragma unroll
  for (int j = 0; j < C::kIN; ++j) {
    const int col = n0 + wn * C::kTN + j * 16 + (lane & 15);
    if (col >= a.n) continue;
    const float wsc = a.w_scale_per_col ? ws[col] : ws[0];
#pragma unroll
    for (int i = 0; i < C::kIM; ++i) {
      const int rb0 = m0 + wm * C::kTM + i * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb0 + r;
        if (row < row_end) {
          const float xsc = a.x_scale_per_row ? a.x_scale[row] : a.x_scale[0];
          a.out[(size_t)row * a.n + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r] * xsc * wsc);
        }
      }
    }
  }
}

template <int XF, int WF, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(GemmArgs a, int tiles_n) {
  using C = TileCfg<BM, BN, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::kStage];
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM;
  gemm_tile<XF, WF, BM, BN, WAVES_M, WAVES_N>(a, lds, m0, min(a.m, m0 + BM), tn * BN, a.wq_pre, a.w_scale);
}

// Grouped: a linear tile id enumerates, per expert in order, its row tiles x the
// column tiles. Offsets are clamped so any input stays in bounds.
template <int XF, int WF, int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void grouped_gemm_kernel(GemmArgs a, const int32_t* offsets,
                                                                              int experts, int tiles_n,
                                                                              size_t expert_bytes) {
  using C = TileCfg<BM, BN, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::kStage];
  __shared__ int s_sel[3];  // expert, first row, row end
  if (threadIdx.x == 0) {
    const int tm_target = blockIdx.x / tiles_n;
    int acc = 0, lo = 0;
    s_sel[0] = -1;
    for (int e = 0; e < experts; ++e) {
      // clamp to [previous end, m] so the ranges are disjoint and in bounds
      const int b = min(max(offsets[e], lo), a.m);
      const int t = min(max(offsets[e + 1], b), a.m);
      lo = t;
      const int cnt = (t - b + BM - 1) / BM;
      if (tm_target < acc + cnt) {
        s_sel[0] = e;
        s_sel[1] = b + (tm_target - acc) * BM;
        s_sel[2] = t;
        break;
      }
      acc += cnt;
    }
  }
  __syncthreads();
  const int e = s_sel[0];
  if (e < 0) return;
  const int m0 = s_sel[1];
  const int row_end = min(s_sel[2], m0 + BM);
  const int tn = blockIdx.x % tiles_n;
  const float* ws = a.w_scale + (size_t)e * (a.w_scale_per_col ? a.n : 1);
  gemm_tile<XF, WF, BM, BN, WAVES_M, WAVES_N>(a, lds, m0, row_end, tn * BN, a.wq_pre + e * expert_bytes, ws);
}

template <int XF, int WF>
static hipError_t launch_gemm_t(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  const int tiles_m = (a.m + BM - 1) / BM, tiles_n = (a.n + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<XF, WF, BM, BN, 2, 2>), dim3(tiles_m * tiles_n), dim3(256), 0, st, a, tiles_n);
  return hipGetLastError();
}

template <int XF, int WF>
static hipError_t launch_grouped_t(const GemmArgs& a, const int32_t* offsets, int experts, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  const int tiles_n = (a.n + BN - 1) / BN;
  const int tiles_m = (a.m + BM - 1) / BM + experts;  // bound for valid offsets
  const size_t expert_bytes = (size_t)((a.n + 15) / 16 * 16) * (size_t)((a.k + kBK - 1) / kBK * kBK);
  hipLaunchKernelGGL((grouped_gemm_kernel<XF, WF, BM, BN, 2, 2>), dim3(tiles_m * tiles_n), dim3(256), 0, st, a,
                     offsets, experts, tiles_n, expert_bytes);
  return hipGetLastError();
}

#define HQ_DISPATCH_FMT_PAIR(XF, WF, CALL)               \
  do {                                                   \
    if ((XF) == kE4M3 && (WF) == kE4M3) { CALL(kE4M3, kE4M3); } \
    else if ((XF) == kE4M3) { CALL(kE4M3, kE5M2); }       \
    else if ((WF) == kE4M3) { CALL(kE5M2, kE4M3); }       \
    else { CALL(kE5M2, kE5M2); }                          \
  } while (0)

hipError_t launch_gemm(const GemmArgs& a, int xf, int wf, hipStream_t st) {
#define CALL(X, W) return launch_gemm_t<X, W>(a, st)
  HQ_DISPATCH_FMT_PAIR(xf, wf, CALL);
#undef CALL
}

hipError_t launch_grouped_gemm(const GemmArgs& a, const int32_t* offsets, int experts, int xf, int wf,
                               hipStream_t st) {
#define CALL(X, W) return launch_grouped_t<X, W>(a, offsets, experts, st)
  HQ_DISPATCH_FMT_PAIR(xf, wf, CALL);
#undef CALL
}

}  // namespace hq
