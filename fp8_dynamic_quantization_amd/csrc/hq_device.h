// Device-side helpers shared by the quantize and GEMM kernels of libhq (gfx950).
//
// FP8 formats (hip-quant README, "FP8 Formats (both APIs)"): E4M3 bias 7, max
// 448, NaN only; E5M2 bias 15, max 57344, +-Inf/NaN. The cast used everywhere is
// saturating round-to-nearest-even: the scaled value is clamped to +-fmax with
// v_med3_f32 and converted with the gfx950 OCP conversion instructions
// (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32, round-to-nearest-even). Clamp + convert
// equals the saturating RNE encoder on every float32 input the encoder decides
// (every pattern from 2^-20 up to 2^18, zero, subnormals, Inf and NaN, compared on
// the device with the CPU encoder; below and above those binades every value is a
// signed zero or saturates); NaN inputs, which the clamp would turn into +-fmax,
// are patched to the canonical code 0x7F. Casts whose scale comes from the amax
// of the elements' own group, on vectors without Inf or NaN, leave the clamp
// out: their scaled values are never more than one float32 ulp above fmax, which
// the conversion rounds to fmax (vec_cast_checked, OWN).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

constexpr uint32_t kInfBits = 0x7f800000u;   // float32 +Inf; magnitudes >= this are non-finite
constexpr float kScaleFloor = 1.17549435e-38f;  // 2^-126, smallest normal float32

template <int FMT> struct Fp8Fmt;
template <> struct Fp8Fmt<kE4M3> { static constexpr float kMax = 448.0f; };
template <> struct Fp8Fmt<kE5M2> { static constexpr float kMax = 57344.0f; };

__device__ __forceinline__ float clamp_fmax(float v, float fmax) {
  return __builtin_amdgcn_fmed3f(v, -fmax, fmax);
}

// Two saturating RNE casts packed into 16-bit half `hi` of `old`. CLAMP = false
// leaves out the clamp to +-fmax: only for finite values whose magnitude is at
// most one float32 ulp above fmax, which the conversion's nearest-even rounding
// takes to fmax by itself (the next magnitude either format encodes lies 2^-4
// (E4M3) or 2^-3 (E5M2) of fmax above it; checked on the device).
template <int FMT, bool HI, bool CLAMP = true>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t old) {
  constexpr float F = Fp8Fmt<FMT>::kMax;
  const float ca = CLAMP ? clamp_fmax(a, F) : a, cb = CLAMP ? clamp_fmax(b, F) : b;
  if (FMT == kE4M3) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, (int)old, HI);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(ca, cb, (int)old, HI);
}

// Four floats -> four codes in one dword (element i in byte i). The two
// conversions fill the low and then the high half of one register, so its
// starting value never reaches the result; passing a register the caller no
// longer needs (`dead`) saves the move that zeroes a fresh one.
template <int FMT, bool CLAMP = true>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d, uint32_t dead = 0u) {
  uint32_t w = cvt2<FMT, false, CLAMP>(a, b, dead);
  return cvt2<FMT, true, CLAMP>(c, d, w);
}

// Replace byte i of `codes` by 0x7F where element i is NaN.
__device__ __forceinline__ uint32_t patch_nan4(uint32_t codes, float a, float b, float c, float d) {
  const float v[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (v[i] != v[i]) codes = (codes & ~(0xffu << (8 * i))) | (0x7fu << (8 * i));
  return codes;
}

// ---- high-precision input vectors (16 bytes) ----------------------------------

// Number of elements in a 16-byte vector of input type XT.
template <int XT> struct VecTraits;
template <> struct VecTraits<kBF16> { static constexpr int kElems = 8; };
template <> struct VecTraits<kF32> { static constexpr int kElems = 4; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element i of a vector as float32 (exact widening).
template <int XT>
__device__ __forceinline__ float vec_elem(const uint4& v, int i) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if (XT == kF32) return __uint_as_float(w[i]);
  return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
}

// Largest magnitude in the vector, as float32 bits, non-finite elements included
// (a result >= kInfBits means the vector holds an Inf or NaN).
template <int XT>
__device__ __forceinline__ uint32_t vec_absmax_raw(const uint4& v) {
  if (XT == kF32) {
    const uint32_t a = max(v.x & 0x7fffffffu, v.y & 0x7fffffffu);
    const uint32_t b = max(v.z & 0x7fffffffu, v.w & 0x7fffffffu);
    return max(a, b);
  }
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 m0 = __builtin_bit_cast(us2, v.x & 0x7fff7fffu);
  us2 m1 = __builtin_bit_cast(us2, v.y & 0x7fff7fffu);
  us2 m2 = __builtin_bit_cast(us2, v.z & 0x7fff7fffu);
  us2 m3 = __builtin_bit_cast(us2, v.w & 0x7fff7fffu);
  us2 m = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1), __builtin_elementwise_max(m2, m3));
  return (uint32_t)max(m[0], m[1]) << 16;
}

// Largest magnitude over the finite elements only, as float32 bits.
template <int XT>
__device__ __forceinline__ uint32_t vec_absmax_finite(const uint4& v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < VecTraits<XT>::kElems; ++i) {
    const uint32_t a = __float_as_uint(vec_elem<XT>(v, i)) & 0x7fffffffu;
    m = max(m, a < kInfBits ? a : 0u);
  }
  return m;
}

// Cast the vector's elements times r. Output: bytes in element order, in
// `out[0 .. kElems/4 - 1]`. `patch` adds the NaN fix-up; CLAMP = false (see
// cvt2) only for finite elements with |x * r| <= fmax * (1 + 2^-23).
template <int XT, int FMT, bool CLAMP = true>
__device__ __forceinline__ void vec_cast(const uint4& v, float r, bool patch, uint32_t* out) {
#pragma unroll
  for (int d = 0; d < VecTraits<XT>::kElems / 4; ++d) {
    const float a = vec_elem<XT>(v, 4 * d + 0) * r;
    const float b = vec_elem<XT>(v, 4 * d + 1) * r;
    const float c = vec_elem<XT>(v, 4 * d + 2) * r;
    const float e = vec_elem<XT>(v, 4 * d + 3) * r;
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};  // element 4d's input word, dead after the widening
    uint32_t w = cvt4<FMT, CLAMP>(a, b, c, e, in[d]);
    if (patch) w = patch_nan4(w, a, b, c, e);
    out[d] = w;
  }
}

// Cast a whole vector; applies the NaN patch only when the vector holds a
// non-finite element (raw >= kInfBits), so the common path is branch-free.
// OWN: r comes from the amax of a group the vector's elements belong to
// (dynamic scaling), so every finite element has |x| <= amax and, with
// s = fl32(amax / fmax) and r = fl32(1 / s), |fl32(x * r)| <= fmax * (1 + 2^-23):
// a vector without Inf or NaN then needs no clamp.
template <int XT, int FMT, bool OWN = false>
__device__ __forceinline__ void vec_cast_checked(const uint4& v, float r, uint32_t raw, uint32_t* out) {
  if (raw >= kInfBits) vec_cast<XT, FMT>(v, r, true, out);
  else vec_cast<XT, FMT, !OWN>(v, r, false, out);
}

// ---- stochastic rounding to E5M2 -------------------------------------------------
// (hip-quant README, "Stochastic E5M2 Backward Gradients": round to one of the
// two adjacent E5M2 values, up with probability proportional to the distance
// from the lower one, from a stateless hash of (seed, element index).) The
// hash is Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): element i uses
// word i % 4 of Philox(counter = (i/4 low, i/4 high, 0, 0), key = seed) and
// u = (word >> 8) * 2^-24. Every quantity the decision compares is exact in
// float32, so the choice is deterministic given (seed, i).

struct SrSeed {
  uint32_t k0, k1;  // seed, low and high 32 bits
};

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // each 32 x 32 -> 64-bit product as one v_mad_u64_u32 (both halves at once)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The four hash words of elements i .. i+3 (i a multiple of 4).
__device__ __forceinline__ uint4 sr_words(SrSeed sd, size_t i) {
  const uint64_t blk = (uint64_t)i >> 2;
  return philox4x32_10(make_uint4((uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u), sd.k0, sd.k1);
}

// E5M2 code of the scaled value y with hash word `word`. lo <= |y| < hi are the
// adjacent E5M2 magnitudes (ulp = hi - lo, a power of two: 2^(e-2) in binade
// e >= -14, 2^-16 below); p = (|y| - lo) / ulp and u are exact, and the
// magnitude is hi when u < p. |y| >= 57344 (Inf too) saturates, NaN -> 0x7F,
// the sign is kept. The chosen value is exact in E5M2, so the nearest-even
// conversion returns its code.
__device__ __forceinline__ uint32_t e5m2_sr_code(float y, uint32_t word) {
  const float a = fabsf(y);
  if (!(a < 57344.0f)) return a != a ? 0x7Fu : ((__float_as_uint(y) >> 24) & 0x80u) | 0x7Bu;
  float lo, ulp, inv;
  if (a >= 6.103515625e-05f) {  // 2^-14: normal E5M2 range
    const uint32_t b = __float_as_uint(a), e = b & 0x7F800000u;
    lo = __uint_as_float(b & 0xFFE00000u);          // keep two mantissa bits
    ulp = __uint_as_float(e - (2u << 23));           // 2^(e-2)
    inv = __uint_as_float((256u << 23) - e);         // 2^(2-e)
  } else {
    lo = floorf(a * 65536.0f) * 1.52587890625e-05f;  // multiples of 2^-16
    ulp = 1.52587890625e-05f;
    inv = 65536.0f;
  }
  const float p = (a - lo) * inv;
  const float u = (float)(word >> 8) * 5.9604644775390625e-08f;  // 2^-24
  const float m = __builtin_copysignf(u < p ? lo + ulp : lo, y);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(m, 0.0f, 0, false) & 0xFFu;
}

// Four scaled values (elements i .. i+3) to four stochastic E5M2 codes.
__device__ __forceinline__ uint32_t e5m2_sr4(float a, float b, float c, float d, SrSeed sd, size_t i) {
  const uint4 w = sr_words(sd, i);
  return e5m2_sr_code(a, w.x) | (e5m2_sr_code(b, w.y) << 8) | (e5m2_sr_code(c, w.z) << 16) |
         (e5m2_sr_code(d, w.w) << 24);
}

// Cast a whole vector whose first element has flat index `elem`: nearest-even
// (SR = false, vec_cast_checked, OWN as there) or stochastic E5M2 (SR = true).
template <int XT, int FMT, bool SR, bool OWN = false>
__device__ __forceinline__ void cast_vec(const uint4& v, float r, uint32_t raw, uint32_t* out, SrSeed sd,
                                         size_t elem) {
  if constexpr (!SR) {
    vec_cast_checked<XT, FMT, OWN>(v, r, raw, out);
  } else {
    static_assert(FMT == kE5M2, "stochastic rounding produces E5M2");
#pragma unroll
    for (int d = 0; d < VecTraits<XT>::kElems / 4; ++d)
      out[d] = e5m2_sr4(vec_elem<XT>(v, 4 * d) * r, vec_elem<XT>(v, 4 * d + 1) * r, vec_elem<XT>(v, 4 * d + 2) * r,
                        vec_elem<XT>(v, 4 * d + 3) * r, sd, elem + 4 * d);
  }
}

// ---- code stores -----------------------------------------------------------------

typedef unsigned int hq_u2v __attribute__((ext_vector_type(2)));
typedef unsigned int hq_u4v __attribute__((ext_vector_type(4)));

// E codes (E/4 words in w) to p. The codes are written once and read by a later
// kernel, so they go out as non-temporal stores: streamed to memory without
// displacing the input lines still being read (measured: the per-row quantize
// of a 4096 x 4096 bf16 tensor drops from 12.0 to 9.6 us).
template <int E>
__device__ __forceinline__ void store_codes(uint8_t* p, const uint32_t* w) {
  if constexpr (E == 8) {
    const hq_u2v v = {w[0], w[1]};
    __builtin_nontemporal_store(v, reinterpret_cast<hq_u2v*>(p));
  } else {
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
  }
}

// The same with ordinary stores, for outputs whose 128-byte lines are filled by
// several wavefronts of a workgroup and should meet in L2 before write-back.
template <int E>
__device__ __forceinline__ void store_codes_temporal(uint8_t* p, const uint32_t* w) {
  if constexpr (E == 8) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
    *reinterpret_cast<uint32_t*>(p) = w[0];
  }
}

// ---- reductions ----------------------------------------------------------------

// Max over the 64 lanes of a wavefront, returned to every lane. DPP lane moves
// only (no LDS round trips): within each row of 16 lanes, the quad swaps and
// the half-row and row mirrors leave the row max in every lane; the row
// broadcasts then fold row 0 into row 1 and row 2 into row 3 (lane 15 of a row
// to the next row), and rows 0-1 into rows 2-3 (lane 31), so lane 63 ends with
// the wavefront max, read back as a uniform value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
  constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kQuadSwap1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kQuadSwap2, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kRowHalfMirror, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kRowMirror, 0xF, 0xF, false));
  // rows outside the row mask keep `old` (= v), so max leaves them unchanged
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kRowBcast15, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Block-wide max of a uint32; every thread gets the result. `lds` needs
// BLOCK/64 entries. Contains __syncthreads (all threads must call it).
template <int BLOCK>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds) {
  v = wave_max_u32(v);
  if (BLOCK == 64) return v;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();  // lds may still be read by a previous call
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  uint32_t m = lds[0];
#pragma unroll
  for (int i = 1; i < BLOCK / 64; ++i) m = max(m, lds[i]);
  return m;
}

// Dequant scale from an amax given as float32 bits: s = max(amax / fmax, 2^-126)
// (correctly rounded float32 division).
template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax) {
  return fmaxf(amax / Fp8Fmt<FMT>::kMax, kScaleFloor);
}

// ---- bf16 output ---------------------------------------------------------------

// float32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > kInfBits) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace hq
