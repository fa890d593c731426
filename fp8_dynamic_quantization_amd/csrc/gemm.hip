// Scaled FP8 (a8w8) GEMM, its grouped form and the weight pre-shuffle, gfx950.
//
//   out[m, n] = bf16_rne( sum_k dec(XQ[m,k]) * dec(WQ[n,k]) * x_scale[m] * w_scale[n] )
//
// (the method statement; operand set of the aiter PR "gemm_a8w8_bpreshuffle_out";
// NT layout of AstrAI's linear_forward_fp8). The contraction runs on the gfx950
// V_MFMA_F32_16X16X128_F8F6F4 instruction (FP8/BF8 selected per operand), fp32
// accumulators, and a fused scale + bf16 epilogue.
//
// MFMA register layout (per 64-lane wavefront, 16x16x128): lane l holds row l%16
// of the first operand and column l%16 of the second, each with the 32
// consecutive k values 32*(l/16) .. +31; result lane l holds column l%16, rows
// 4*(l/16) + 0..3. The kernels pass the weight fragment as the first operand and
// the activation fragment as the second, so a lane's four results are four
// weight "slots" of one activation row. The pre-shuffled weight puts output
// channels 8g..8g+3 of a 32-channel group in slots 4g..4g+3 of its first
// fragment and channels 8g+4..8g+7 in the same slots of its second fragment:
// after the two MFMAs of a fragment pair, lane l holds 8 consecutive output
// columns of one row, stored as one 16-byte write.
//
// Tiling: a workgroup of 4*WM wavefronts (WM rows x 4 columns) computes a
// BM x (4*TN) tile: 256 x 256 with eight wavefronts (two per SIMD, 128
// accumulators each), or 128 x 256, 128 x 128 and 64 x 128 with four. The BM
// rows of A (XQ, row-major) are staged through double-buffered LDS with an XOR
// swizzle of their 16-byte chunks (chunk c of row r at slot c ^ (r & 7)), which
// keeps the row-wise stores and the MFMA-order reads free of bank conflicts.
// Wavefront w owns TN columns and streams their pre-shuffled B fragments from
// global memory straight into registers (each fragment half is one coalesced
// 1 KB load), so B never touches LDS. Tails: A rows past the tile's last row and
// B fragments past the padded N fall outside their buffer resource's extent and
// read as zero, and their outputs are masked on store; the K tail of A is zeroed
// on its way to LDS (B is zero-padded).
#include "hq_device.h"
#include "hq_launch.h"

#include <mutex>

namespace hq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

// Strict (exact-product) form. The FP8 matrix-core instructions add the
// products of each run of 8 consecutive k in a window 13 bits below the run's
// largest exponent sum and truncate the rest (measured on the device; the
// float16 instructions keep every product bit). Every E4M3 and E5M2 value is
// a float16 value, so the strict form converts each lane's operand bytes to
// float16 (v_cvt_scalef32_pk_f16_fp8 / _bf8 with scale 1: exact, NaN and Inf
// kept) and runs V_MFMA_F32_16X16X32_F16 four times per 128-deep step: call s
// takes bytes 8s .. 8s+7 of every lane's 32, i.e. matrix k 32g + 8s .. +7 of
// lane group g, on both operands, so the four calls together pair every k once
// and leave the accumulator layout of the FP8 instruction unchanged.
template <int FMT>
__device__ __forceinline__ h8v f16x8(uint32_t d0, uint32_t d1) {
  h2v a, b, c, d;
  if constexpr (FMT == kE4M3) {
    a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
  } else {
    a = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(d0, 1.0f, false);
    b = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(d0, 1.0f, true);
    c = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(d1, 1.0f, false);
    d = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(d1, 1.0f, true);
  }
  return h8v{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One 16 x 16 x 128 product of two fragments held as 32 bytes per lane (lo =
// bytes 0-15, hi = bytes 16-31), accumulated into acc: the FP8 instruction, or
// in the strict form four float16 instructions on the converted bytes (the
// first operand's conversions are passed in, converted once per step).
template <int FMT>
__device__ __forceinline__ void f16_frag(const uint4& lo, const uint4& hi, h8v out[4]) {
  out[0] = f16x8<FMT>(lo.x, lo.y);
  out[1] = f16x8<FMT>(lo.z, lo.w);
  out[2] = f16x8<FMT>(hi.x, hi.y);
  out[3] = f16x8<FMT>(hi.z, hi.w);
}
__device__ __forceinline__ v4f mfma_f16x4(const h8v w[4], const h8v x[4], v4f acc) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(w[s], x[s], acc, 0, 0, 0);
  return acc;
}

constexpr int kBK = 128;          // K per pipeline stage = one MFMA
constexpr int kFragBytes = 2048;  // 16 slots x 128 k
// Third flags word of a raw (stride 0) buffer resource on gfx9-class parts:
// 32-bit data format, range-checked against the extent.
constexpr int kRsrcFlags = 0x00020000;
constexpr int kBadOffset = int(0x80000000u);  // past any extent: a buffer load there reads zero

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 as_uint4(v4u v) { return make_uint4(v[0], v[1], v[2], v[3]); }

// ---------------------------------------------------------------------------
// pre-shuffle
// ---------------------------------------------------------------------------
// One thread per 16-byte piece of the output. Piece P of fragment (nb, kb):
// h = P / 64, slot = P % 16, quarter q = (P % 64) / 16 -> weight row
// 32*(nb/2) + 8*(slot/4) + 4*(nb%2) + slot%4, columns kb*128 + 32*q + 16*h .. +15.
__global__ __launch_bounds__(256) void preshuffle_kernel(const uint8_t* __restrict__ wq, int n, int k, int kblocks,
                                                         size_t npieces, uint8_t* __restrict__ out) {
  const size_t pc = blockIdx.x * (size_t)256 + threadIdx.x;
  if (pc >= npieces) return;
  const size_t frag = pc / 128;
  const int p = (int)(pc % 128);
  const int h = p / 64, q = (p % 64) / 16, slot = p % 16;
  const int nb = (int)(frag / kblocks), kb = (int)(frag % kblocks);
  const int row = 32 * (nb >> 1) + 8 * (slot >> 2) + 4 * (nb & 1) + (slot & 3);
  const int col = kb * kBK + q * 32 + h * 16;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < n && col < k) v = *reinterpret_cast<const uint4*>(wq + (size_t)row * k + col);
  *reinterpret_cast<uint4*>(out + pc * 16) = v;
}

// Number of 16-slot fragments along N after padding N to a multiple of 32.
__host__ __device__ inline int frag_rows(int n) { return (n + 31) / 32 * 2; }

hipError_t launch_preshuffle(const uint8_t* wq, int n, int k, uint8_t* out, hipStream_t st) {
  const int kblocks = (k + kBK - 1) / kBK;
  const size_t npieces = (size_t)frag_rows(n) * kblocks * 128;
  const size_t grid = (npieces + 255) / 256;
  hipLaunchKernelGGL(preshuffle_kernel, dim3((unsigned)grid), dim3(256), 0, st, wq, n, k, kblocks, npieces, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// epilogue helpers (bias, FP8 output)
// ---------------------------------------------------------------------------
// The bias of output column `col` as float32: a bf16 value widened, or an FP8
// code decoded (v_cvt_f32_fp8 / v_cvt_f32_bf8, exact) times the bias scale.
__device__ __forceinline__ float bias_at(const GemmArgs& a, int col, float bscale) {
  if (a.bias_kind == kBiasBF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.bias)[col] << 16);
  const int code = static_cast<const uint8_t*>(a.bias)[col];
  const float d = a.bias_kind == kBiasE4M3 ? __builtin_amdgcn_cvt_f32_fp8(code, 0) : __builtin_amdgcn_cvt_f32_bf8(code, 0);
  return d * bscale;
}

// N (4 or 8) epilogue values to FP8 codes of fl32(v * r_out) (saturating RNE,
// NaN -> 0x7F), four to a word.
template <int N>
__device__ __forceinline__ void fp8_out_codes(const float* v, float r_out, int fmt, uint32_t* w) {
#pragma unroll
  for (int d = 0; d < N / 4; ++d) {
    const float x0 = v[4 * d] * r_out, x1 = v[4 * d + 1] * r_out, x2 = v[4 * d + 2] * r_out, x3 = v[4 * d + 3] * r_out;
    w[d] = fmt == kE4M3 ? cvt4<kE4M3>(x0, x1, x2, x3) : cvt4<kE5M2>(x0, x1, x2, x3);
    w[d] = patch_nan4(w[d], x0, x1, x2, x3);
  }
}

// The codes of fp8_out_codes stored as one N-byte write when `full`, else byte
// by byte up to `left` columns.
template <int N>
__device__ __forceinline__ void store_fp8_out(uint8_t* dst, const float* v, float r_out, int fmt, bool full,
                                              int left) {
  uint32_t w[N / 4];
  fp8_out_codes<N>(v, r_out, fmt, w);
  if (full) {
    if constexpr (N == 8) __builtin_nontemporal_store(hq_u2v{w[0], w[1]}, reinterpret_cast<hq_u2v*>(dst));
    else __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(dst));
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e)
      if (e < left) dst[e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
  }
}

// ---------------------------------------------------------------------------
// GEMM tile
// ---------------------------------------------------------------------------
// Per 128-deep K step a wavefront issues BM/16 x TN/16 MFMAs. A is double-
// buffered in LDS and B in registers; the K loop is unrolled by two so every
// register buffer has a compile-time index.
template <int BM, int TN, int WM>
struct BsCfg {
  static constexpr int kWaves = 4 * WM;            // WM wavefront rows x 4 wavefront columns
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBN = 4 * TN;
  static constexpr int kWR = BM / WM;              // rows per wavefront
  static constexpr int kIM = kWR / 16, kIN = TN / 16;
  static constexpr int kAVec = BM * 8 / kThreads;  // 16-byte A pieces per thread per stage
  static constexpr int kRowStep = kThreads / 8;    // rows between a thread's A pieces
  static constexpr int kABytes = BM * kBK;         // one LDS stage
  static constexpr int kLdsBytes = 2 * kABytes + (BM + 2 * kBN) * 4;  // two A stages + epilogue scales and bias
  static constexpr int kBsfBytes = 2 * (BM + kBN) * 4;                // block-scaled form: two stages of block scales
  static_assert(BM % 32 == 0 && TN % 32 == 0 && kWR % 16 == 0, "tile");
};

// KTAIL: K is not a multiple of 128, so the A chunks past K are zeroed on their
// way to LDS; without it the K loop has no masking at all.
// BSZ > 0: the block-scaled form with blocks of BSZ (32, 64 or 128) along K:
// x_scale is [m, nblk] and w_scale [n, nblk] row-major; each block's MFMA sums
// start from zero and are folded as acc = fma(t, fl32(xs[m, b] * ws[n, b]), acc)
// in block order, the step's scales staged in LDS one step ahead; the epilogue
// then applies no scale (only the bias). Blocks narrower than the 128-deep MFMA
// take one MFMA per block, whose per-lane E8M0 operand scales are 2^0 for the
// block's 32-element chunks and 2^-127 for the others: their products are then
// scaled by 2^-254 and vanish below float32's range.
// KS == 2: split K inside the workgroup. A second group of the tile's
// wavefronts takes the odd K steps (with A stages of its own in LDS), the
// first the even ones; at the end the second hands its sums to the first
// through LDS and the first runs the epilogue. For launches of one tile per CU
// this puts two wavefronts on each SIMD, so one's loads hide behind the
// other's MFMAs. Both groups pass the same barriers: K is a multiple of 256.
template <int XF, int WF, int BM, int TN, int WM, bool KTAIL, int BSZ, bool STRICT = false, int KS = 1>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, uint8_t* lds, int m0, int row_end, int n0,
                                          const uint8_t* __restrict__ wq, const float* __restrict__ ws) {
  using C = BsCfg<BM, TN, WM>;
  static_assert(KS == 1 || (KS == 2 && !KTAIL && BSZ == 0 && !STRICT && WM == 1 && TN == 32), "split-K form");
  constexpr bool BSF = BSZ > 0;
  constexpr int NB = BSF ? kBK / BSZ : 1;  // scale blocks per K step
  static_assert(!BSF || BSZ == 32 || BSZ == 64 || BSZ == 128, "block size");
  static_assert(C::kAVec <= C::kIM && C::kIN <= C::kIM, "slot schedule: at most one A piece and two B halves per slot");
  static_assert(!BSF || BM + C::kBN <= C::kThreads, "block scales: one row or column per thread per step");
  static_assert(!(BSF && STRICT), "the strict form has no block scales");
  const int tid_all = threadIdx.x;
  const int ks = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid_all / C::kThreads);  // K group
  const int tid = tid_all - ks * C::kThreads;                                        // thread in the group
  uint8_t* const lds_g = lds + ks * 2 * C::kABytes;                                 // the group's A stages
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // wavefront column
  const int wrow = __builtin_amdgcn_readfirstlane(tid >> 8);        // wavefront row
  const int K = a.k;
  const int nkb = (K + kBK - 1) / kBK;
  const int nfrag = frag_rows(a.n);

  // A staging: piece v of thread t is row v*kRowStep + t/8, 16-byte chunk t%8.
  // The swizzle (chunk ^ row%8) only depends on t, so every piece of a thread
  // shares one LDS offset plus a compile-time v*kRowStep*128.
  const int a_c = tid & 7, a_r = tid >> 3;
  const int a_dst = a_r * kBK + ((a_c ^ (a_r & 7)) << 4);

  // Global loads are buffer loads: a resource (base and extent in bytes) in
  // scalar registers, one 32-bit per-lane offset that stays fixed for the whole
  // K loop, and a wavefront-uniform offset that carries the piece and the K
  // step. A load reads zero for every dword at or past the extent (the per-lane
  // and uniform offsets both count), which covers all tails without clamping:
  // A rows past row_end and B fragments past the padded N read zero, and their
  // outputs are masked on store. The hardware takes extents and offsets as
  // unsigned 32-bit values; K < 2^24 keeps them below 2^32 for tiles of up to
  // 256 rows, so they are formed in uint32_t (a 256-row extent at K >= 2^23
  // passes 2^31) and handed over as the same bits.
  const uint32_t uK = (uint32_t)K;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.xq + (size_t)m0 * K), (short)0, (int)((uint32_t)(row_end - m0) * uK), kRsrcFlags);
  const int a_vo = (int)((uint32_t)a_r * uK + (uint32_t)(a_c * 16));
  const int nbw = __builtin_amdgcn_readfirstlane((n0 + wave * TN) / 16);
  const int nbw_c = min(nbw, nfrag);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wq + (size_t)nbw_c * nkb * kFragBytes), (short)0, min(C::kIN, nfrag - nbw_c) * nkb * kFragBytes,
      kRsrcFlags);
  // Blocks narrower than 128 (NB > 1) need each operand byte at the K
  // position the MFMA's block scales assume: within a lane's 32 bytes, lane
  // group g = l / 16 holds K 16g .. 16g+15 in bytes 0-15 and K 64+16g .. +15 in
  // bytes 16-31 (scale block b = K 32b .. 32b+31 takes its scale from lane group
  // b). So the weight halves come from pieces (g % 2, g / 2) and (g % 2, 2 + g / 2)
  // of the pre-shuffled fragment, and the activation from chunks g and g + 4 of
  // the row; otherwise (the plain order) half h and chunks 2g, 2g + 1.
  const int kg = lane >> 4, slot16 = (lane & 15) * 16;
  const int b_vo0 = NB > 1 ? (kg & 1) * 1024 + (kg >> 1) * 256 + slot16 : lane * 16;
  const int b_vo1 = NB > 1 ? (kg & 1) * 1024 + (2 + (kg >> 1)) * 256 + slot16 : lane * 16 + 1024;

  // The epilogue's scales go to LDS (after the two A stages) during the
  // prologue: x_scale of the tile's BM rows, w_scale of its 4*TN columns
  // (clamped at the edges; masked on store), one of each per thread at most.
  // Their loads are issued after the first operand loads and written to LDS
  // just before the prologue's barrier, so no operand load waits for them.
  static_assert(BM <= C::kThreads && C::kBN <= C::kThreads, "one epilogue scale of each kind per thread");
  float* s_xs = reinterpret_cast<float*>(lds + KS * 2 * C::kABytes);
  float* s_ws = s_xs + BM;
  float* s_bias = s_ws + C::kBN;

  // Block scales (BSZ > 0): thread t < BM holds the NB scales of tile row t,
  // thread BM + c those of tile column c, for one K step; a step's values sit in
  // LDS stage (step % 2), [row or column][NB], after the tile's epilogue data.
  // Blocks past the last one (the K tail) get scale 0: their codes are zero.
  typedef float bsv_t __attribute__((ext_vector_type(NB)));
  float* s_bsf = reinterpret_cast<float*>(lds + C::kLdsBytes);
  auto bsf_load = [&](int kbq) -> bsv_t {
    bsv_t v;
    const float* src = tid < BM ? a.x_scale + (size_t)min(m0 + tid, row_end - 1) * a.nblk
                                : ws + (size_t)min(n0 + tid - BM, a.n - 1) * a.nblk;
#pragma unroll
    for (int b = 0; b < NB; ++b) v[b] = (tid < BM + C::kBN && kbq * NB + b < a.nblk) ? src[kbq * NB + b] : 0.0f;
    return v;
  };
  auto bsf_store = [&](int stage, bsv_t v) {
    if (tid < BM + C::kBN) *reinterpret_cast<bsv_t*>(s_bsf + (stage * (BM + C::kBN) + tid) * NB) = v;
  };
  // the lane's rows (16 i + l % 16 of its wavefront row) and its 8 columns,
  // one base each so every read of a step is a constant offset from it
  const float* xs_lane = s_bsf + (wrow * C::kWR + (lane & 15)) * NB;
  const float* ws_lane = s_bsf + (BM + wave * TN + 8 * (lane >> 4)) * NB;
  // E8M0 operand scale of block b for this lane's 32-element K chunk (l / 16)
  auto blk_sel = [&](int b) -> int { return ((lane >> 4) / (4 / NB)) == b ? 127 : 0; };

  // MFMA-order reads: fragment i is rows i*16 .. i*16+15; lane l reads row
  // i*16 + l%16, chunks 2*(l/16) and 2*(l/16)+1; the swizzle again only depends
  // on the lane, fragment i adds i*2048.
  const int rl = lane & 15, cg0 = NB > 1 ? kg : 2 * kg, cg1 = NB > 1 ? kg + 4 : 2 * kg + 1;
  const int a_rd0 = wrow * C::kWR * kBK + rl * kBK + ((cg0 ^ (rl & 7)) << 4);
  const int a_rd1 = wrow * C::kWR * kBK + rl * kBK + ((cg1 ^ (rl & 7)) << 4);

  v4f acc[C::kIM][C::kIN];
#pragma unroll
  for (int i = 0; i < C::kIM; ++i)
#pragma unroll
    for (int j = 0; j < C::kIN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 ra[C::kAVec];                       // A pieces in flight (two K steps ahead)
  bool ra_valid = true;                     // K-tail mask of the pieces in ra
  uint4 fb0[2 * C::kIN], fb1[2 * C::kIN];  // B fragment halves: current step, next step
  // A fragments read ahead from LDS: two ahead with one wavefront per SIMD, one
  // ahead with two (the second wavefront hides the rest, and registers are halved).
  constexpr int kFaDepth = WM == 1 ? 3 : 2;

#define HQ_LOAD_A_PIECE(KB, V) \
  ra[V] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_vo, (int)((uint32_t)((V) * C::kRowStep) * uK + (uint32_t)((KB) * kBK)), 0))
#define HQ_STORE_A_PIECE(BUF, V)                                          \
  *reinterpret_cast<uint4*>(lds_g + (BUF) * C::kABytes + a_dst + (V) * C::kRowStep * kBK) = \
      (!KTAIL || ra_valid) ? ra[V] : make_uint4(0u, 0u, 0u, 0u)
#define HQ_STORE_A_PIECE_V(BUF, V, VALID)                                  \
  *reinterpret_cast<uint4*>(lds_g + (BUF) * C::kABytes + a_dst + (V) * C::kRowStep * kBK) = \
      (!KTAIL || (VALID)) ? ra[V] : make_uint4(0u, 0u, 0u, 0u)
#define HQ_LOAD_B_HALF(KB, FB, H)                                                                 \
  FB[H] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(b_rsrc, ((H) & 1) ? b_vo1 : b_vo0,             \
                                                         ((H) >> 1) * nkb * kFragBytes + (KB) * kFragBytes, 0))
#define HQ_READ_A(BASE, I, LO, HI)                                         \
  do {                                                                     \
    LO = *reinterpret_cast<const uint4*>((BASE) + a_rd0 + (I) * 2048);     \
    HI = *reinterpret_cast<const uint4*>((BASE) + a_rd1 + (I) * 2048);     \
  } while (0)
#define HQ_V8(LO, HI) v8i{(int)LO.x, (int)LO.y, (int)LO.z, (int)LO.w, (int)HI.x, (int)HI.y, (int)HI.z, (int)HI.w}

  // Block-scaled fold of slot I's zero-start sums (block by block, in K order):
  // acc = fma(t, fl32(xs * ws), acc). Issued in the next slot after that slot's
  // MFMAs when at most two blocks share a step; with four (blocks of 32) in the
  // slot itself, which halves the sums held live.
  constexpr bool kFoldLate = NB <= 2;
#define HQ_FOLD(I, XS)                                                                                 \
  _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                       \
    _Pragma("unroll") for (int j = 0; j < C::kIN; ++j)                                                 \
      _Pragma("unroll") for (int r = 0; r < 4; ++r)                                                    \
        acc[(I)][j][r] = fmaf(tp_[(I) & 1][b][j][r], (XS)[b] * wsl_[b][j][r], acc[(I)][j][r])

  // One K step, as kIM slots. Slot i: read an upcoming A fragment from LDS, then memory
  // operations, then the kIN MFMAs of A fragment i. Slots 0 .. kIN-1 load the B
  // halves of step KB+1 (two each), as early as possible, since step KB+1 needs
  // them in its first slot. The last kAVec slots each store one A piece of step
  // KB+1 (loaded one step earlier) into the other LDS buffer and reuse its
  // register for the same piece of step KB+2, so every A load has a whole step to
  // land. Loads are never behind a branch, so the wait counters the compiler
  // inserts stay exact; steps past the end reload the last one.
#define HQ_STEP(KB, BUF, FBC, FBN)                                                                     \
  do {                                                                                                 \
    const int nb1_ = min((KB) + KS, nkb - 1);                                                          \
    const int nb2_ = min((KB) + 2 * KS, nkb - 1);                                                      \
    const uint8_t* cur_ = lds_g + (BUF) * C::kABytes;                                                  \
    uint4 lo0_, hi0_, lo1_, hi1_, lo2_, hi2_;                                                          \
    bool st_valid_ = ra_valid;                                                                         \
    bsv_t bs_nx_{};                                                                                    \
    if constexpr (BSF) bs_nx_ = bsf_load(nb1_);                                                        \
    float wsl_[NB][BSF ? C::kIN : 1][4];                                                               \
    v4f tp_[2][NB][C::kIN];                                                                            \
    bsv_t xs_prev_{};                                                                                  \
    if constexpr (BSF) {                                                                               \
      _Pragma("unroll") for (int j = 0; j < C::kIN; ++j)                                               \
        _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                                \
          const bsv_t w_ = *reinterpret_cast<const bsv_t*>(                                            \
              ws_lane + ((BUF) * (BM + C::kBN) + 32 * (j >> 1) + 4 * (j & 1) + r) * NB);               \
          _Pragma("unroll") for (int b = 0; b < NB; ++b) wsl_[b][j][r] = w_[b];                        \
        }                                                                                              \
    }                                                                                                  \
    h8v fbh_[STRICT ? C::kIN : 1][4];                                                                  \
    if constexpr (STRICT) {                                                                            \
      _Pragma("unroll") for (int j = 0; j < C::kIN; ++j) f16_frag<WF>(FBC[2 * j], FBC[2 * j + 1], fbh_[j]); \
    }                                                                                                  \
    HQ_READ_A(cur_, 0, lo0_, hi0_);                                                                    \
    if (kFaDepth == 3) HQ_READ_A(cur_, 1, lo1_, hi1_);                                                 \
    _Pragma("unroll") for (int i = 0; i < C::kIM; ++i) {                                               \
      if (kFaDepth == 3 && i + 2 < C::kIM) {                                                           \
        if (i % 3 == 0) HQ_READ_A(cur_, i + 2, lo2_, hi2_);                                            \
        else if (i % 3 == 1) HQ_READ_A(cur_, i + 2, lo0_, hi0_);                                       \
        else HQ_READ_A(cur_, i + 2, lo1_, hi1_);                                                       \
      }                                                                                                \
      if (kFaDepth == 2 && i + 1 < C::kIM) {                                                           \
        if (i & 1) HQ_READ_A(cur_, i + 1, lo0_, hi0_);                                                 \
        else HQ_READ_A(cur_, i + 1, lo1_, hi1_);                                                       \
      }                                                                                                \
      if (i < C::kIN) {                                                                                \
        HQ_LOAD_B_HALF(nb1_, FBN, 2 * i);                                                              \
        HQ_LOAD_B_HALF(nb1_, FBN, 2 * i + 1);                                                          \
      }                                                                                                \
      if (i >= C::kIM - C::kAVec) {                                                                    \
        const int v_ = i - (C::kIM - C::kAVec);                                                        \
        HQ_STORE_A_PIECE_V((BUF) ^ 1, v_, st_valid_);                                                  \
        HQ_LOAD_A_PIECE(nb2_, v_);                                                                     \
        if (v_ == C::kAVec - 1 && KTAIL) ra_valid = nb2_ * kBK + a_c * 16 < K;                         \
      }                                                                                                \
      const v8i fa_ = kFaDepth == 2 ? ((i & 1) ? HQ_V8(lo1_, hi1_) : HQ_V8(lo0_, hi0_))                \
                    : (i % 3 == 0) ? HQ_V8(lo0_, hi0_) : (i % 3 == 1) ? HQ_V8(lo1_, hi1_) : HQ_V8(lo2_, hi2_); \
      if constexpr (BSF) {                                                                             \
        _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                 \
          _Pragma("unroll") for (int j = 0; j < C::kIN; ++j)                                           \
            tp_[i & 1][b][j] = NB == 1                                                                 \
                ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(HQ_V8(FBC[2 * j], FBC[2 * j + 1]), fa_, \
                                                                   v4f{0.f, 0.f, 0.f, 0.f}, WF, XF, 0, 0, 0, 0) \
                : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(HQ_V8(FBC[2 * j], FBC[2 * j + 1]), fa_, \
                                                                   v4f{0.f, 0.f, 0.f, 0.f}, WF, XF, 0, blk_sel(b), \
                                                                   0, blk_sel(b));                     \
        if (kFoldLate && i > 0) {                                                                      \
          HQ_FOLD(i - 1, xs_prev_);                                                                    \
          /* the empty asm keeps the folds in this slot, so two slots' sums are live at most */        \
          _Pragma("unroll") for (int j = 0; j < C::kIN; ++j) asm volatile("" : "+v"(acc[i - 1][j]));   \
        }                                                                                              \
        xs_prev_ = *reinterpret_cast<const bsv_t*>(xs_lane + ((BUF) * (BM + C::kBN) + 16 * i) * NB);   \
        if (!kFoldLate) {                                                                              \
          HQ_FOLD(i, xs_prev_);                                                                        \
          _Pragma("unroll") for (int j = 0; j < C::kIN; ++j) asm volatile("" : "+v"(acc[i][j]));       \
        }                                                                                              \
      } else if constexpr (STRICT) {                                                                   \
        const h8v fah_[4] = {f16x8<XF>(fa_[0], fa_[1]), f16x8<XF>(fa_[2], fa_[3]),                     \
                             f16x8<XF>(fa_[4], fa_[5]), f16x8<XF>(fa_[6], fa_[7])};                    \
        _Pragma("unroll") for (int j = 0; j < C::kIN; ++j) acc[i][j] = mfma_f16x4(fbh_[j], fah_, acc[i][j]); \
      } else {                                                                                         \
        _Pragma("unroll") for (int j = 0; j < C::kIN; ++j)                                             \
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(HQ_V8(FBC[2 * j], FBC[2 * j + 1]), fa_, \
                                                                       acc[i][j], WF, XF, 0, 0, 0, 0); \
      }                                                                                                \
      __builtin_amdgcn_sched_barrier(0);                                                               \
    }                                                                                                  \
    if constexpr (BSF) {                                                                               \
      if (kFoldLate) HQ_FOLD(C::kIM - 1, xs_prev_);                                                    \
      bsf_store((BUF) ^ 1, bs_nx_);                                                                    \
    }                                                                                                  \
    __syncthreads();                                                                                   \
  } while (0)

  // prologue: A(0) to LDS buffer 0, B(0) to registers, A(1) in flight
  if constexpr (BSF) bsf_store(0, bsf_load(0));
#pragma unroll
  for (int v = 0; v < C::kAVec; ++v) HQ_LOAD_A_PIECE(ks, v);
  ra_valid = a_c * 16 < K;
#pragma unroll
  for (int h = 0; h < 2 * C::kIN; ++h) HQ_LOAD_B_HALF(ks, fb0, h);
  float xs_v = 0.0f, ws_v = 0.0f;
  if constexpr (!BSF) {
    if (tid < BM) xs_v = a.x_scale[a.x_scale_per_row ? min(m0 + tid, row_end - 1) : 0];
    if (tid < C::kBN) ws_v = ws[a.w_scale_per_col ? min(n0 + tid, a.n - 1) : 0];
  }
#pragma unroll
  for (int v = 0; v < C::kAVec; ++v) HQ_STORE_A_PIECE(0, v);
  {
    const int nb1 = min(ks + KS, nkb - 1);
#pragma unroll
    for (int v = 0; v < C::kAVec; ++v) HQ_LOAD_A_PIECE(nb1, v);
    ra_valid = nb1 * kBK + a_c * 16 < K;
  }
  if constexpr (!BSF) {
    if (tid < BM) s_xs[tid] = xs_v;
    if (tid < C::kBN) s_ws[tid] = ws_v;
  }
  if (a.bias_kind != kBiasNone) {
    const float bsc = a.bias_kind == kBiasBF16 ? 0.0f : a.bias_scale[0];
    if (tid < C::kBN) s_bias[tid] = bias_at(a, min(n0 + tid, a.n - 1), bsc);
  }
  __syncthreads();
  // Two unconditional steps per iteration (LDS buffers and B register sets both
  // alternate); an odd last step follows the loop, so the loop body has no branch.
  // The group's steps are ks, ks + KS, ks + 2 KS, ...
  const int nsteps = nkb / KS;
  int j = 0;
  for (; j + 2 <= nsteps; j += 2) {
    HQ_STEP(ks + KS * j, 0, fb0, fb1);
    HQ_STEP(ks + KS * (j + 1), 1, fb1, fb0);
  }
  if (j < nsteps) HQ_STEP(ks + KS * j, 0, fb0, fb1);
  if constexpr (KS == 2) {
    // the last step ended on a barrier: the A stages are free for the sums
    static_assert(C::kIM * C::kIN * C::kThreads * 16 <= KS * 2 * C::kABytes, "split-K sums fit the A stages");
    v4f* part = reinterpret_cast<v4f*>(lds);
    if (ks == 1) {
#pragma unroll
      for (int i = 0; i < C::kIM; ++i)
#pragma unroll
        for (int jn = 0; jn < C::kIN; ++jn) part[(i * C::kIN + jn) * C::kThreads + tid] = acc[i][jn];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int i = 0; i < C::kIM; ++i)
#pragma unroll
        for (int jn = 0; jn < C::kIN; ++jn) acc[i][jn] += part[(i * C::kIN + jn) * C::kThreads + tid];
    }
    __syncthreads();
  }
#undef HQ_LOAD_A_PIECE
#undef HQ_STORE_A_PIECE
#undef HQ_STORE_A_PIECE_V
#undef HQ_LOAD_B_HALF
#undef HQ_READ_A
#undef HQ_V8
#undef HQ_STEP
#undef HQ_FOLD

  // Epilogue: fragment pair (2*jp, 2*jp+1) gives lane l the 8 consecutive output
  // columns n0 + wave*TN + 32*jp + 8*(l/16) .. +7 of row m0 + 16*i + l%16.
  // Scale in fp32 (plus the bias), then either round to bf16
  // (v_cvt_pk_bf16_f32, nearest-even) and store 16 bytes, or cast to FP8 codes
  // and store 8 bytes. Output stores are non-temporal: the output is written
  // once and never read by the kernel, and streaming it past the L2 keeps the
  // operand lines other tiles still read there and leaves no dirty output to
  // write back when the kernel ends (4096^3: 66 -> 58-60 us; MoE 33 -> 28 us).
  // In the 256 x 256 tile (64 columns per wavefront) a 16-row block's two
  // fragment pairs hold whole 128-byte output lines (bf16, N % 64 == 0), but
  // each store instruction would cover only half of 16 lines, and streamed
  // half lines reach HBM as extra write traffic (1.33x the output at 4096^3). Lanes l and l ^ 8 (DPP
  // row_ror:8 within each 16-lane row) swap one 16-byte piece first: lanes of
  // rows 0-7 keep pair 0 of their row and take pair 0 of row r + 8, lanes of
  // rows 8-15 keep pair 1 of their row and take pair 1 of row r - 8, so each
  // of the two stores writes 8 complete lines (no partial-line writes to HBM).
  constexpr int kRowRor8 = 0x128;
  const bool vec_ok = (a.n & 7) == 0;
  const bool lines_ok = C::kIN == 4 && WM == 2 && !BSF && (a.n & 63) == 0 && !a.out_scale && n0 + wave * TN + TN <= a.n;
  const float r_out = a.out_scale ? 1.0f / a.out_scale[0] : 0.0f;
  const int ccol = 8 * (lane >> 4);
  float wsc[C::kIN / 2][8];
#pragma unroll
  for (int jp = 0; jp < C::kIN / 2; ++jp)
#pragma unroll
    for (int e = 0; e < 8; ++e) wsc[jp][e] = BSF ? 1.0f : s_ws[wave * TN + 32 * jp + ccol + e];
  // FP8 output codes of the 256 x 256 tile: the 64 KB code tile fits the two
  // A stages (free once the K loop has ended on its barrier), so it is staged
  // there (8-byte pieces, 16-byte chunks at chunk ^ (row % 16)) and stored as
  // whole row segments, 16 bytes per lane: an 8-byte store per lane would
  // stream half lines to HBM. (In the smaller tiles the same code pushed the
  // register count past a workgroup-per-CU boundary.)
  if constexpr (!BSF && WM == 2) {
    constexpr int kChunksF = C::kBN / 16;
    static_assert(BM * C::kBN <= 2 * C::kABytes && (BM * kChunksF) % C::kThreads == 0, "FP8 staging layout");
    if (a.out_scale && (a.n & 15) == 0 && n0 + C::kBN <= a.n) {  // workgroup-uniform
#pragma unroll
      for (int i = 0; i < C::kIM; ++i) {
        const int tr = wrow * C::kWR + i * 16 + (lane & 15);
        const float xsc = s_xs[tr];
#pragma unroll
        for (int jp = 0; jp < C::kIN / 2; ++jp) {
          const v4f p0 = acc[i][2 * jp], p1 = acc[i][2 * jp + 1];
          float v[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] * xsc * wsc[jp][e];
          if (a.bias_kind != kBiasNone) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += s_bias[wave * TN + 32 * jp + ccol + e];
          }
          uint32_t w[2];
          fp8_out_codes<8>(v, r_out, a.out_fmt, w);
          const int cb = wave * TN + 32 * jp + ccol;  // byte column in the tile row
          const int pc = (cb >> 4) ^ (tr & (kChunksF - 1));
          *reinterpret_cast<uint2*>(lds + tr * C::kBN + pc * 16 + (cb & 8)) = make_uint2(w[0], w[1]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < BM * kChunksF / C::kThreads; ++q) {
        const int idx = q * C::kThreads + tid;
        const int tr = idx / kChunksF, c = idx % kChunksF;
        const uint4 val = *reinterpret_cast<const uint4*>(lds + tr * C::kBN + ((c ^ (tr & (kChunksF - 1))) << 4));
        if (m0 + tr < row_end) {
          uint8_t* dst = static_cast<uint8_t*>(a.out) + (size_t)(m0 + tr) * a.n + n0 + 16 * c;
          __builtin_nontemporal_store(hq_u4v{val.x, val.y, val.z, val.w}, reinterpret_cast<hq_u4v*>(dst));
        }
      }
      return;
    }
  }
  // With 32 columns per wavefront (kIN == 2) a line spans two wavefronts, so
  // the bf16 tile goes through LDS: the K loop ended on a barrier, and its two
  // A stages (2 x BM x 128 bytes) hold the BM x 256-byte output tile exactly.
  // Each row's 16-byte chunks are stored at chunk ^ (row % 16), so the
  // wavefronts' writes (16 rows, one chunk column) and the read-back (one row,
  // 16 chunks) are both free of bank conflicts; each group of 16 lanes then
  // stores one whole 256-byte row segment.
  if constexpr (C::kIN == 2 && !BSF) {
    static_assert(C::kThreads == 256 && BM * 256 <= 2 * C::kABytes, "staged epilogue layout");
    if (!a.out_scale && (a.n & 63) == 0 && n0 + C::kBN <= a.n) {  // workgroup-uniform
#pragma unroll
      for (int i = 0; i < C::kIM; ++i) {
        if (ks != 0) break;  // split K: the first group holds the sums
        const int tr = wrow * C::kWR + i * 16 + (lane & 15);
        const float xsc = s_xs[tr];
        const v4f p0 = acc[i][0], p1 = acc[i][1];
        float v[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * xsc * wsc[0][e];
        if (a.bias_kind != kBiasNone) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += s_bias[wave * TN + ccol + e];
        }
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f2v pr = {v[2 * e], v[2 * e + 1]};
          w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf2v));
        }
        const int chunk = 4 * wave + (lane >> 4);
        *reinterpret_cast<uint4*>(lds + tr * 256 + ((chunk ^ (tr & 15)) << 4)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
      __syncthreads();
      const int c = tid_all & 15;
#pragma unroll
      for (int p = 0; p < BM * 16 / (KS * C::kThreads); ++p) {
        const int tr = (p * KS * C::kThreads + tid_all) >> 4;
        const uint4 val = *reinterpret_cast<const uint4*>(lds + tr * 256 + ((c ^ (tr & 15)) << 4));
        if (m0 + tr < row_end) {
          uint16_t* dst = static_cast<uint16_t*>(a.out) + (size_t)(m0 + tr) * a.n + n0 + 8 * c;
          __builtin_nontemporal_store(hq_u4v{val.x, val.y, val.z, val.w}, reinterpret_cast<hq_u4v*>(dst));
        }
      }
      return;
    }
  }
  if (KS == 2 && ks != 0) return;  // split K: the first group stores
#pragma unroll
  for (int i = 0; i < C::kIM; ++i) {
    const int row = m0 + wrow * C::kWR + i * 16 + (lane & 15);
    const float xsc = BSF ? 1.0f : s_xs[wrow * C::kWR + i * 16 + (lane & 15)];
    if constexpr (C::kIN == 4 && WM == 2 && !BSF) {
      if (lines_ok && m0 + wrow * C::kWR + i * 16 + 16 <= row_end) {  // wavefront-uniform
        uint32_t w[2][4];
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          const v4f p0 = acc[i][2 * jp], p1 = acc[i][2 * jp + 1];
          float v[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] * xsc * wsc[jp][e];
          if (a.bias_kind != kBiasNone) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += s_bias[wave * TN + 32 * jp + ccol + e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f2v pr = {v[2 * e], v[2 * e + 1]};
            w[jp][e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf2v));
          }
        }
        const bool lo = (lane & 15) < 8;
        uint32_t got[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          got[e] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(lo ? w[1][e] : w[0][e]), kRowRor8, 0xF, 0xF, false);
        // store 0: rows 0-7 of the block; store 1: rows 8-15
        const int r0 = m0 + wrow * C::kWR + i * 16 + (lane & 7);
        const int col = n0 + wave * TN + (lo ? 0 : 32) + ccol;
        uint16_t* d0 = static_cast<uint16_t*>(a.out) + (size_t)r0 * a.n + col;
        uint16_t* d1 = d0 + (size_t)8 * a.n;
        const uint32_t* s0 = lo ? w[0] : got;
        const uint32_t* s1 = lo ? got : w[1];
        __builtin_nontemporal_store(hq_u4v{s0[0], s0[1], s0[2], s0[3]}, reinterpret_cast<hq_u4v*>(d0));
        __builtin_nontemporal_store(hq_u4v{s1[0], s1[1], s1[2], s1[3]}, reinterpret_cast<hq_u4v*>(d1));
        continue;
      }
    }
    if (row >= row_end) continue;
#pragma unroll
    for (int jp = 0; jp < C::kIN / 2; ++jp) {
      const int col0 = n0 + wave * TN + 32 * jp + ccol;
      if (col0 >= a.n) continue;
      const v4f p0 = acc[i][2 * jp], p1 = acc[i][2 * jp + 1];
      float v[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
      if constexpr (!BSF) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * xsc * wsc[jp][e];
      }
      if (a.bias_kind != kBiasNone) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += s_bias[wave * TN + 32 * jp + ccol + e];
      }
      const size_t off = (size_t)row * a.n + col0;
      const bool full = vec_ok && col0 + 8 <= a.n;
      if (a.out_scale) {
        store_fp8_out<8>(static_cast<uint8_t*>(a.out) + off, v, r_out, a.out_fmt, full, a.n - col0);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f2v pr = {v[2 * e], v[2 * e + 1]};
          w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf2v));
        }
        uint16_t* dst = static_cast<uint16_t*>(a.out) + off;
        if (full) {
          __builtin_nontemporal_store(hq_u4v{w[0], w[1], w[2], w[3]}, reinterpret_cast<hq_u4v*>(dst));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col0 + e < a.n) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// Tile order: with T tiles, a multiple of the 8 XCDs, workgroup b (placed on XCD
// b % 8 by the dispatcher) takes tile (b % 8) * T/8 + b / 8, so each XCD gets one
// contiguous run of tiles; tiles are numbered in groups of kGroupM tile rows,
// column-major inside a group, so a run covers a compact block of A rows and B
// columns that stays resident in that XCD's L2.
constexpr int kGroupM = 4;

__device__ __forceinline__ int xcd_remap(int b, int total) {
  return total % 8 == 0 ? (b % 8) * (total / 8) + b / 8 : b;
}

__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  const int r = t % per_group;
  *tm = first_m + r % gm;
  *tn = r / gm;
}

template <int XF, int WF, int BM, int TN, int WM, bool KTAIL, bool STRICT, int KS = 1>
__global__ __launch_bounds__(256 * WM * KS) void gemm_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  using C = BsCfg<BM, TN, WM>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLdsBytes + (KS - 1) * 2 * C::kABytes];
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM;
  gemm_tile<XF, WF, BM, TN, WM, KTAIL, 0, STRICT, KS>(a, lds, m0, min(a.m, m0 + BM), tn * C::kBN, a.wq_pre,
                                                      a.w_scale);
}

// Block-scaled form (blocks of 128 along K) on the same data path.
template <int XF, int WF, int BM, int TN, int WM, bool KTAIL, int BSZ>
__global__ __launch_bounds__(256 * WM) __attribute__((amdgpu_waves_per_eu(2))) void gemm_bsf_kernel(GemmArgs a, int tiles_m, int tiles_n) {
  using C = BsCfg<BM, TN, WM>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLdsBytes + C::kBsfBytes * (128 / BSZ)];
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM;
  gemm_tile<XF, WF, BM, TN, WM, KTAIL, BSZ>(a, lds, m0, min(a.m, m0 + BM), tn * C::kBN, a.wq_pre, a.w_scale);
}

// Grouped: a linear tile id enumerates, per expert in order, its row tiles x the
// column tiles. Offsets are clamped so any input stays in bounds.
template <int XF, int WF, int BM, int TN, int WM, bool KTAIL, bool STRICT>
__global__ __launch_bounds__(256 * WM) void grouped_gemm_kernel(GemmArgs a, const int32_t* offsets, int experts,
                                                                int tiles_n, size_t expert_bytes) {
  using C = BsCfg<BM, TN, WM>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLdsBytes];
  __shared__ int s_sel[3];  // expert, first row, row end
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  if (threadIdx.x == 0) {
    const int tm_target = t / tiles_n;
    int acc = 0, lo = 0;
    s_sel[0] = -1;
    for (int e = 0; e < experts; ++e) {
      // clamp to [previous end, m] so the ranges are disjoint and in bounds
      const int b = min(max(offsets[e], lo), a.m);
      const int end = min(max(offsets[e + 1], b), a.m);
      lo = end;
      const int cnt = (end - b + BM - 1) / BM;
      if (tm_target < acc + cnt) {
        s_sel[0] = e;
        s_sel[1] = b + (tm_target - acc) * BM;
        s_sel[2] = end;
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
  const int tn = t % tiles_n;
  const float* ws = a.w_scale + (size_t)e * (a.w_scale_per_col ? a.n : 1);
  // the epilogue's bias is per expert: [experts, n] values, and an FP8 bias has
  // one bias scale per expert; the output scale is shared
  GemmArgs ae = a;
  if (a.bias) {
    ae.bias = static_cast<const uint8_t*>(a.bias) + (size_t)e * a.n * (a.bias_kind == kBiasBF16 ? 2 : 1);
    if (a.bias_scale) ae.bias_scale = a.bias_scale + e;
  }
  gemm_tile<XF, WF, BM, TN, WM, KTAIL, 0, STRICT>(ae, lds, m0, row_end, tn * C::kBN, a.wq_pre + e * expert_bytes, ws);
}

// ---------------------------------------------------------------------------
// skinny M (decode): weight streaming
// ---------------------------------------------------------------------------
// For M <= 64 the GEMM is bound by reading WQ once, and a CU streams from HBM
// at a rate set by how many misses it can keep in flight, so the work is
// spread over every CU. A fragment group is F consecutive 16-slot weight
// fragments (16*F output columns); its K blocks are dealt to kSkWaves
// wavefronts (wavefront g takes blocks g, g + kSkWaves, ...), which sit in S
// workgroups of kSkWaves/S wavefronts. Each wavefront issues every load of a
// chunk of KPW K blocks (F weight fragments and MB 16-row activation fragments
// each) before its MFMAs, and reuses each activation fragment for F weight
// fragments. Partial sums are added in LDS in wavefront order; with S > 1 each
// workgroup writes its sums to the workspace and the last of the S to finish
// (device-scope counter, reset by that workgroup) adds the S partials in split
// order and runs the epilogue, so results do not depend on arrival order.
constexpr int kSkWaves = 16;
// The weight is read exactly once, so its loads are streaming (the `nt` cache
// policy): N = 2048, K = 7168, M = 1 / 8 / 32: 7.03 / 7.55 / 11.1 -> 6.62 /
// 7.13 / 10.7 us. (The tile kernels' operands are re-read by other CUs through
// the L2; there the same policy was slower.)
constexpr int kNtLoad = 2;
// Workspace of a split launch: the column groups' arrival counters in a fixed
// leading region (a launch splits only below 256 groups, so 1 KB holds them
// all), then the partial sums. The region does not depend on the shape, so a
// workspace shared by launches of different shapes never finds partial sums
// where another shape's counters are.
constexpr size_t kSkCounterBytes = 1024;

SkinnyPlan skinny_plan(int m, int n, int k) {
  SkinnyPlan p{};
  p.mb = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  p.f = p.mb == 1 ? 1 : 2;
  p.kpw = p.mb == 1 ? 4 : (p.mb == 2 ? 2 : 1);  // loads in flight within the 128-VGPR budget
  p.groups = (frag_rows(n) + p.f - 1) / p.f;
  p.halves = 1;
  // One 16-row activation block and fewer fragments than CUs: each fragment's
  // two slot halves go to two workgroups (the other half's lanes load zeros),
  // so every CU streams weight with no cross-workgroup sum.
  if (p.mb == 1 && p.groups < 256) {
    p.halves = 2;
    p.groups *= 2;
  }
  // Split only when one workgroup per group would take its wavefronts through
  // more than one chunk of loads: below that the cross-workgroup step costs
  // more latency than the extra workgroups save.
  p.splits = 1;
  const int nkb = (k + kBK - 1) / kBK;
  p.kb = nkb;
  if (nkb > kSkWaves * p.kpw && p.groups < (int)(kSkCounterBytes / 4)) {
    while (p.splits < 8 && p.groups * p.splits < 256) p.splits *= 2;
    while (p.splits > 1 && nkb < p.splits * 2) p.splits /= 2;  // at least 2 K blocks per workgroup
  }
  p.workspace_bytes = p.splits == 1 ? 0 : kSkCounterBytes + (size_t)p.groups * p.splits * p.f * p.mb * 1024;
  // Wavefronts per fragment group: 16 for split plans; unsplit, the next power
  // of two of ceil(nkb / 8), at least 2 (each wavefront then takes up to 8 K
  // blocks, two chunks of loads). Smaller workgroups cost less to start and
  // reduce: N = 7168, K = 768 / 2048, M = 1 (one weight copy): 7.9 / 8.2 us at
  // 16 wavefronts, 3.1 / 3.9 us at 2; N = 2048, K = 7168: 6.7 us at 16, 6.55 at 8.
  p.waves = kSkWaves;
  if (p.splits == 1) {
    int w = 2;
    while (w < kSkWaves && w * 8 < nkb) w *= 2;
    p.waves = w;
  }
  return p;
}

// TPB: the largest workgroup the kernel is launched with; a plan whose
// workgroups are smaller compiles with a smaller bound and gets the registers
// for more K blocks per chunk of loads (KPW).
template <int XF, int WF, int MB, int F, int KPW, bool STRICT, int TPB = 64 * kSkWaves>
__global__ __launch_bounds__(TPB) void gemm_skinny_kernel(GemmArgs a, int splits, int chunk, int halves,
                                                                  uint32_t* counters, float* partials) {
  __shared__ __attribute__((aligned(16))) float red[kSkWaves][64][4];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int waves = blockDim.x >> 6;  // wavefronts of the group in this workgroup
  const int wtot = waves * splits;     // wavefronts of the fragment group (K blocks are dealt over them)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fg = blockIdx.x / splits, split = blockIdx.x % splits;
  const int g = split * waves + wave;  // wavefront index within the fragment group
  // with halves == 2 (F == 1): this group is slot half `half` of fragment fg / 2;
  // lanes of the other half load zeros and store nothing
  const int half = fg % halves;
  const bool my_slots = halves == 1 || ((lane & 15) >> 3) == half;
  const bool my_rows = halves == 1 || ((lane >> 4) >> 1) == half;
  const int K = a.k, nkb = (K + kBK - 1) / kBK;
  const int nfrag = frag_rows(a.n);
  // B: the group's fragment rows (F * nkb * 2048 contiguous bytes); fragments
  // past the padded N and blocks past nkb read zero.
  const int nb0 = fg / halves * F;
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.wq_pre + (size_t)nb0 * nkb * kFragBytes), (short)0, min(F, nfrag - nb0) * nkb * kFragBytes,
      kRsrcFlags);
  // X: rows past M read zero through the extent; columns past K are sent past
  // it too (they would otherwise read the next row).
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, (short)0, a.m * K, kRsrcFlags);
  const int xr = lane & 15, xc = 32 * (lane >> 4);

  // Epilogue scales of every slice this lane may store (indices clamped;
  // masked on store). Slice (f, i): row 16*i + l%16, columns col0(f) .. +3 (see
  // the epilogue). They are loaded after the first chunk's operand loads are
  // issued, so no operand load waits for them; a bias is read in the epilogue.
  float xs_r[MB], ws_r[F][4];
  auto load_scales = [&]() {
#pragma unroll
    for (int i = 0; i < MB; ++i) xs_r[i] = a.x_scale[a.x_scale_per_row ? min(i * 16 + xr, a.m - 1) : 0];
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int nb = nb0 + f;
      const int col0 = 32 * (nb >> 1) + 8 * (lane >> 4) + 4 * (nb & 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) ws_r[f][e] = a.w_scale[a.w_scale_per_col ? min(col0 + e, a.n - 1) : 0];
    }
  };

  v4f acc[F][MB];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[f][i] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (nkb + wtot * KPW - 1) / (wtot * KPW);
  for (int c = 0; c < nchunks; ++c) {
    uint4 fb[KPW][F][2], fx[KPW][MB][2];
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int kb = (c * KPW + j) * wtot + g;
      // a block past nkb would land in the next fragment's row: send it past the extent
      const int bvo = kb < nkb && my_slots ? lane * 16 : kBadOffset;
#pragma unroll
      for (int f = 0; f < F; ++f)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          fb[j][f][h] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(
              b_rsrc, bvo + h * 1024, (f * nkb + min(kb, nkb - 1)) * kFragBytes, kNtLoad));
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = kb * kBK + xc + 16 * h;
          const int vo = col < K ? (i * 16 + xr) * K + col : kBadOffset;
          fx[j][i][h] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(x_rsrc, vo, 0, 0));
        }
    }
    if (!STRICT && c == 0) load_scales();
    // keep every load of the chunk ahead of its first MFMA
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      if constexpr (STRICT) {
        // activation fragments converted per use: this kernel is bound by the
        // weight stream, and holding all MB converted fragments spills
#pragma unroll
        for (int f = 0; f < F; ++f) {
          h8v wh[4];
          f16_frag<WF>(fb[j][f][0], fb[j][f][1], wh);
#pragma unroll
          for (int i = 0; i < MB; ++i) {
            h8v xh[4];
            f16_frag<XF>(fx[j][i][0], fx[j][i][1], xh);
            acc[f][i] = mfma_f16x4(wh, xh, acc[f][i]);
          }
        }
      } else {
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const v8i bw = v8i{(int)fb[j][f][0].x, (int)fb[j][f][0].y, (int)fb[j][f][0].z, (int)fb[j][f][0].w,
                             (int)fb[j][f][1].x, (int)fb[j][f][1].y, (int)fb[j][f][1].z, (int)fb[j][f][1].w};
#pragma unroll
          for (int i = 0; i < MB; ++i) {
            const v8i xa = v8i{(int)fx[j][i][0].x, (int)fx[j][i][0].y, (int)fx[j][i][0].z, (int)fx[j][i][0].w,
                               (int)fx[j][i][1].x, (int)fx[j][i][1].y, (int)fx[j][i][1].z, (int)fx[j][i][1].w};
            acc[f][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bw, xa, acc[f][i], WF, XF, 0, 0, 0, 0);
          }
        }
      }
    }
  }

  // (the strict form's float16 conversions leave no registers for the scales
  // during the loop)
  if (STRICT) load_scales();

  // Epilogue of slice (f, i): lane l holds activation row 16*i + l%16 and weight
  // slots 4*(l/16) .. +3 of fragment nb0 + f, i.e. 4 consecutive output columns.
  // Scale, round to bf16, one 8-byte store.
  auto epilogue = [&](int f, int i, v4f t) {
    const int nb = nb0 + f;
    const int row = i * 16 + xr;
    const int col0 = 32 * (nb >> 1) + 8 * (lane >> 4) + 4 * (nb & 1);
    if (row >= a.m || col0 >= a.n || !my_rows) return;
    const float xsc = xs_r[i];
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = t[e] * xsc * ws_r[f][e];
    if (a.bias_kind != kBiasNone) {
      const float bsc = a.bias_kind == kBiasBF16 ? 0.0f : a.bias_scale[0];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += bias_at(a, min(col0 + e, a.n - 1), bsc);
    }
    const size_t off = (size_t)row * a.n + col0;
    const bool full = (a.n & 3) == 0;
    if (a.out_scale) {
      const float r_out = 1.0f / a.out_scale[0];
      store_fp8_out<4>(static_cast<uint8_t*>(a.out) + off, v, r_out, a.out_fmt, full, a.n - col0);
      return;
    }
    uint32_t w2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f2v pr = {v[2 * e], v[2 * e + 1]};
      w2[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf2v));
    }
    uint16_t* dst = static_cast<uint16_t*>(a.out) + off;
    if (full) {
      __builtin_nontemporal_store(hq_u2v{w2[0], w2[1]}, reinterpret_cast<hq_u2v*>(dst));
    } else {
      for (int e = 0; e < 4; ++e)
        if (col0 + e < a.n) dst[e] = (uint16_t)(w2[e >> 1] >> (16 * (e & 1)));
    }
  };

  // Workgroup sum of slice (f, i); wavefront (f*MB + i) % waves owns it. The
  // association is fixed by `chunk` (the wavefronts per workgroup of the
  // planned split): each run of `chunk` wavefronts is added left to right, then
  // the runs left to right, exactly as the split form adds its workgroups'
  // sums, so a launch gives the same bits split or not.
  // With splits > 1 the sums go to partials[fg][split][f][i][lane][4].
  float* mine = partials + ((size_t)fg * splits + split) * (F * MB * 256);
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      *reinterpret_cast<v4f*>(&red[wave][lane][0]) = acc[f][i];
      __syncthreads();
      if (wave == (f * MB + i) % waves) {
        v4f t = v4f{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < waves; c0 += chunk) {
          v4f u = *reinterpret_cast<const v4f*>(&red[c0][lane][0]);
          for (int w = 1; w < chunk; ++w) {
            const v4f v = *reinterpret_cast<const v4f*>(&red[c0 + w][lane][0]);
            u = v4f{u[0] + v[0], u[1] + v[1], u[2] + v[2], u[3] + v[3]};
          }
          t = c0 == 0 ? u : v4f{t[0] + u[0], t[1] + u[1], t[2] + u[2], t[3] + u[3]};
        }
        if (splits == 1) {
          epilogue(f, i, t);
        } else {
          float* p = mine + ((f * MB + i) * 64 + lane) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) __hip_atomic_store(p + e, t[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
    }
  if (splits == 1) return;

  // Cross-workgroup step: publish, count, and let the last workgroup finish.
  // The partials were written with device-scope atomic stores, which write
  // through to the coherence point; waiting for their completion before the
  // barrier, and the barrier before thread 0's counter increment, publishes
  // them without a release fence (on this part a fence writes back the XCD's
  // whole L2). The last workgroup reads them with device-scope atomic loads,
  // which also go to the coherence point, so it needs no acquire fence (that
  // would invalidate the L2 under the other workgroups of the XCD).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(counters + fg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done == (uint32_t)(splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  const float* base = partials + (size_t)fg * splits * (F * MB * 256);
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (wave != (f * MB + i) % waves) continue;
      v4f t = v4f{0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < splits; ++sp) {
        const float* p = base + ((size_t)sp * (F * MB) + f * MB + i) * 256 + lane * 4;
        const v4f u = v4f{__hip_atomic_load(p + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                          __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                          __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                          __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
        t = sp == 0 ? u : v4f{t[0] + u[0], t[1] + u[1], t[2] + u[2], t[3] + u[3]};
      }
      epilogue(f, i, t);
    }
  if (tid == 0) __hip_atomic_store(counters + fg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// `workspace` may be null: the plan then runs with one workgroup per group.
template <int XF, int WF, bool STRICT>
static hipError_t launch_skinny(const GemmArgs& a, void* workspace, size_t workspace_bytes, hipStream_t st) {
  SkinnyPlan p = skinny_plan(a.m, a.n, a.k);
  const int chunk = p.waves / p.splits;  // the planned association, kept when run unsplit
  if (p.splits > 1 && (workspace == nullptr || workspace_bytes < p.workspace_bytes)) p.splits = 1;
  uint32_t* counters = static_cast<uint32_t*>(workspace);
  float* partials = p.splits > 1
                        ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSkCounterBytes)
                        : nullptr;
  const int wg_waves = p.waves / p.splits;
  const dim3 grid(p.groups * p.splits), block(64 * wg_waves);
  const int halves = p.halves;
  // K blocks each wavefront takes (dealt over the group's p.waves wavefronts).
  // Where the workgroup is small enough, the register budget it leaves holds
  // all of them in one chunk of loads, so each wavefront waits for memory once
  // (N = 2048, K = 7168: M = 1 and 8 take 7 blocks per wavefront in one chunk
  // instead of two of 4; M = 32 takes 4 in one chunk instead of two of 2). The
  // K order each wavefront adds its blocks in does not depend on the chunking,
  // so the outputs are the same bits.
  // (The strict form keeps the 1024-thread bound: its float16 conversions
  // need the registers.)
  const int bpw = (p.kb + p.waves - 1) / p.waves;
  const bool deep1 = wg_waves <= 8 && bpw > 4, deep2 = wg_waves <= 4 && bpw > 2;
  if (p.mb == 1) {
    if constexpr (!STRICT) {
      if (deep1) {
        hipLaunchKernelGGL((gemm_skinny_kernel<XF, WF, 1, 1, 8, STRICT, 512>), grid, block, 0, st, a, p.splits, chunk,
                           halves, counters, partials);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((gemm_skinny_kernel<XF, WF, 1, 1, 4, STRICT>), grid, block, 0, st, a, p.splits, chunk, halves,
                       counters, partials);
  } else if (p.mb == 2) {
    if constexpr (!STRICT) {
      if (deep2) {
        hipLaunchKernelGGL((gemm_skinny_kernel<XF, WF, 2, 2, 4, STRICT, 256>), grid, block, 0, st, a, p.splits, chunk,
                           halves, counters, partials);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((gemm_skinny_kernel<XF, WF, 2, 2, 2, STRICT>), grid, block, 0, st, a, p.splits, chunk, halves,
                       counters, partials);
  } else if constexpr (!STRICT) {
    if (wg_waves <= 4 && bpw > 1)
      hipLaunchKernelGGL((gemm_skinny_kernel<XF, WF, 4, 2, 4, STRICT, 256>), grid, block, 0, st, a, p.splits, chunk,
                         halves, counters, partials);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<XF, WF, 4, 2, 1, STRICT>), grid, block, 0, st, a, p.splits, chunk, halves,
                         counters, partials);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Tile choice. Candidates (rows x columns per workgroup) with their measured
// throughput per tile area relative to the 256 x 256 tile (4096^3 with random
// FP8 operands, each candidate alone):
// 128 x 256 0.89, 128 x 128 0.81, 64 x 128 0.67. A launch costs about
// ceil(tiles / CUs) rounds of one tile each, so the choice minimises
// ceil(tiles / 256) * area / efficiency. Grouped launches choose between the
// two smaller tiles only (measured on the MoE shape: 128 x 128 32.5 us,
// 256 x 256 38.9 us) and count the upper bound of their
// row tiles, ceil(rows / BM) + experts, since the per-expert counts stay on
// the device.
enum TileCfg { kTile256, kTile128x256, kTile128, kTile64x128 };

static TileCfg pick_tile(long rows, long n, int experts, bool strict) {
  struct Cand {
    TileCfg cfg;
    int bm, bn;
    double eff;
  };
  const Cand cands[] = {{kTile256, 256, 256, 1.0},
                        {kTile128x256, 128, 256, 0.89},
                        {kTile128, 128, 128, 0.81},
                        {kTile64x128, 64, 128, 0.67}};
  TileCfg best = experts || strict ? kTile128 : kTile256;
  double best_cost = 0.0;
  for (const Cand& c : cands) {
    // grouped launches and the strict form (float16 operands need twice the
    // registers per fragment) take the 128-column tiles only
    if ((experts || strict) && (c.cfg == kTile256 || c.cfg == kTile128x256)) continue;
    const long tiles = ((rows + c.bm - 1) / c.bm + experts) * ((n + c.bn - 1) / c.bn);
    const double cost = (double)((tiles + kNumCUs - 1) / kNumCUs) * c.bm * c.bn / c.eff;
    if (best_cost == 0.0 || cost < best_cost) {
      best = c.cfg;
      best_cost = cost;
    }
  }
  return best;
}

template <int XF, int WF, int BM, int TN, int WM, bool STRICT>
static hipError_t launch_plain(const GemmArgs& a, hipStream_t st) {
  using C = BsCfg<BM, TN, WM>;
  const int tiles_m = (a.m + BM - 1) / BM, tiles_n = (a.n + C::kBN - 1) / C::kBN;
  if constexpr (BM == 64 && TN == 32 && WM == 1 && !STRICT) {
    // one 64 x 128 tile per CU or fewer (8 MFMAs per wavefront per K step, too
    // few to cover a load's latency): split K inside the workgroup (K % 256 ==
    // 0). Measured on 2048 x 1024 x 4096: 14.2 -> 13.35 us; the 128 x 128 tile
    // (16 MFMAs per step) got slower with it (4096 x 1024 x 2048: 11.8 -> 12.7).
    if (a.k % (2 * kBK) == 0 && tiles_m * tiles_n <= kNumCUs) {
      hipLaunchKernelGGL((gemm_kernel<XF, WF, BM, TN, WM, false, false, 2>), dim3(tiles_m * tiles_n),
                         dim3(2 * C::kThreads), 0, st, a, tiles_m, tiles_n);
      return hipGetLastError();
    }
  }
  if (a.k % kBK == 0)
    hipLaunchKernelGGL((gemm_kernel<XF, WF, BM, TN, WM, false, STRICT>), dim3(tiles_m * tiles_n), dim3(C::kThreads), 0,
                       st, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_kernel<XF, WF, BM, TN, WM, true, STRICT>), dim3(tiles_m * tiles_n), dim3(C::kThreads), 0,
                       st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int XF, int WF, int BM, int TN, int WM, bool STRICT>
static hipError_t launch_grouped_cfg(const GemmArgs& a, const int32_t* offsets, int experts, hipStream_t st) {
  using C = BsCfg<BM, TN, WM>;
  const int tiles_n = (a.n + C::kBN - 1) / C::kBN;
  const int tiles_m = (a.m + BM - 1) / BM + experts;  // bound for any clamped offsets
  const size_t expert_bytes = (size_t)frag_rows(a.n) * 16 * (size_t)((a.k + kBK - 1) / kBK * kBK);
  if (a.k % kBK == 0)
    hipLaunchKernelGGL((grouped_gemm_kernel<XF, WF, BM, TN, WM, false, STRICT>), dim3(tiles_m * tiles_n),
                       dim3(C::kThreads), 0, st, a, offsets, experts, tiles_n, expert_bytes);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<XF, WF, BM, TN, WM, true, STRICT>), dim3(tiles_m * tiles_n),
                       dim3(C::kThreads), 0, st, a, offsets, experts, tiles_n, expert_bytes);
  return hipGetLastError();
}

// Block-scaled form: 256 x 128, 128 x 128 or 64 x 128 tiles (64 accumulators
// per wavefront, room for the fold's sums and scales), chosen by the cost rule
// of pick_tile with their measured relative throughputs (0.83, 0.81, 0.67 of the
// plain 256 x 256 tile).
template <int XF, int WF, int BM, int TN, int WM, int BSZ>
static hipError_t launch_bsf_cfg(const GemmArgs& a, hipStream_t st) {
  using C = BsCfg<BM, TN, WM>;
  const int tiles_m = (a.m + BM - 1) / BM, tiles_n = (a.n + C::kBN - 1) / C::kBN;
  if (a.k % kBK == 0)
    hipLaunchKernelGGL((gemm_bsf_kernel<XF, WF, BM, TN, WM, false, BSZ>), dim3(tiles_m * tiles_n), dim3(C::kThreads), 0,
                       st, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_bsf_kernel<XF, WF, BM, TN, WM, true, BSZ>), dim3(tiles_m * tiles_n), dim3(C::kThreads), 0,
                       st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int XF, int WF, int BSZ>
static hipError_t launch_bsf_t(const GemmArgs& a, hipStream_t st) {
  const struct {
    int bm;
    double eff;
  } cands[] = {{256, 0.83}, {128, 0.81}, {64, 0.67}};
  int best = 0;
  double best_cost = 0.0;
  for (int c = 0; c < 3; ++c) {
    const long tiles = (long)((a.m + cands[c].bm - 1) / cands[c].bm) * ((a.n + 127) / 128);
    const double cost = (double)((tiles + kNumCUs - 1) / kNumCUs) * cands[c].bm * 128 / cands[c].eff;
    if (c == 0 || cost < best_cost) {
      best = c;
      best_cost = cost;
    }
  }
  if (best == 0) return launch_bsf_cfg<XF, WF, 256, 32, 2, BSZ>(a, st);
  if (best == 1) return launch_bsf_cfg<XF, WF, 128, 32, 1, BSZ>(a, st);
  return launch_bsf_cfg<XF, WF, 64, 32, 1, BSZ>(a, st);
}

// Up to this many rows the weight-streaming kernel runs the GEMM (the strict
// form up to kSkinnyMaxStrictM).
constexpr int kSkinnyMaxM = 64;
constexpr int kSkinnyMaxStrictM = 32;

template <int XF, int WF>
static hipError_t launch_gemm_t(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t st) {
  if (a.strict) {
    // the strict weight-streaming kernel stops at two activation blocks (four
    // would spill their float16 conversions); larger M takes the tiles
    if (a.m <= kSkinnyMaxStrictM) return launch_skinny<XF, WF, true>(a, ws, ws_bytes, st);
    if (pick_tile(a.m, a.n, 0, true) == kTile128) return launch_plain<XF, WF, 128, 32, 1, true>(a, st);
    return launch_plain<XF, WF, 64, 32, 1, true>(a, st);
  }
  if (a.m <= kSkinnyMaxM) return launch_skinny<XF, WF, false>(a, ws, ws_bytes, st);
  switch (pick_tile(a.m, a.n, 0, false)) {
    case kTile256: return launch_plain<XF, WF, 256, 64, 2, false>(a, st);
    case kTile128x256: return launch_plain<XF, WF, 128, 64, 1, false>(a, st);
    case kTile128: return launch_plain<XF, WF, 128, 32, 1, false>(a, st);
    default: return launch_plain<XF, WF, 64, 32, 1, false>(a, st);
  }
}

template <int XF, int WF, bool STRICT>
static hipError_t launch_grouped_s(const GemmArgs& a, const int32_t* offsets, int experts, hipStream_t st) {
  if (pick_tile(a.m, a.n, experts, STRICT) == kTile128)
    return launch_grouped_cfg<XF, WF, 128, 32, 1, STRICT>(a, offsets, experts, st);
  return launch_grouped_cfg<XF, WF, 64, 32, 1, STRICT>(a, offsets, experts, st);
}

template <int XF, int WF>
static hipError_t launch_grouped_t(const GemmArgs& a, const int32_t* offsets, int experts, hipStream_t st) {
  return a.strict ? launch_grouped_s<XF, WF, true>(a, offsets, experts, st)
                  : launch_grouped_s<XF, WF, false>(a, offsets, experts, st);
}

#define HQ_DISPATCH_FMT_PAIR(XF, WF, CALL)                        \
  do {                                                            \
    if ((XF) == kE4M3 && (WF) == kE4M3) { CALL(kE4M3, kE4M3); }   \
    else if ((XF) == kE4M3) { CALL(kE4M3, kE5M2); }               \
    else if ((WF) == kE4M3) { CALL(kE5M2, kE4M3); }               \
    else { CALL(kE5M2, kE5M2); }                                  \
  } while (0)

// ---------------------------------------------------------------------------
// library-held scratch (hq_gemm_a8w8_noalloc)
// ---------------------------------------------------------------------------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops), split decode launches take their workspace
// from this file-scope device array instead of a caller buffer. Each GPU holds
// its own copy until the process ends; host code reaches it only through the
// per-device address from hipGetSymbolAddress (the array's name in host code is
// a host-side stand-in, not a device address). The counter region is zeroed
// once per device at set-up, by a small kernel on the caller's stream, and every
// launch leaves it at zero; the partial sums need no reset. Every call on a GPU
// shares that GPU's array, so calls that overlap on one GPU race on it.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t noalloc_scratch(hipStream_t st, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    constexpr int words = (int)(kSkCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st, static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t gemm_workspace_bytes(int m, int n, int k) {
  return m >= 1 && m <= kSkinnyMaxM ? skinny_plan(m, n, k).workspace_bytes : 0;
}

hipError_t launch_gemm(const GemmArgs& a, int xf, int wf, void* workspace, size_t workspace_bytes, hipStream_t st) {
#define CALL(X, W) return launch_gemm_t<X, W>(a, workspace, workspace_bytes, st)
  HQ_DISPATCH_FMT_PAIR(xf, wf, CALL);
#undef CALL
}

hipError_t launch_gemm_bsf(const GemmArgs& a, int xf, int wf, int bs, hipStream_t st) {
#define CALL(X, W)                                            \
  return bs == 32 ? launch_bsf_t<X, W, 32>(a, st)             \
         : bs == 64 ? launch_bsf_t<X, W, 64>(a, st) : launch_bsf_t<X, W, 128>(a, st)
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
