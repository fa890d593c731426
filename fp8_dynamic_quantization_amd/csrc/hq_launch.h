// Internal launcher interface between the C ABI (hq_api.cpp) and the kernels.
// All sizes here have been validated by the caller; launchers only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hq {

constexpr int kNumCUs = 256;              // compute units of an MI355X / MI350X (gfx950)
constexpr int kMaxTensorPartials = 1024;  // blocks of the per-tensor partial pass
// Delayed scaling counts its blocks in through kArrivalGroups arrival counters
// (one per 128-byte line, after the partials) whose last arrivals then count
// into the ring's own counter: one counter for every block serialised the
// blocks' device-scope increments (17 us instead of 6 us for 8M elements).
constexpr int kArrivalGroups = 32;
constexpr int kArrivalStride = 32;        // uint32 words between arrival counters (128 bytes)
// The single-pass per-tensor kernel's grid barrier follows the arrival
// counters, one 128-byte line each: a 64-bit word (generation in the high
// half, the last call's tensor amax bits in the low half), the top arrival
// counter, and a sticky status word whose bit 0 a single-pass kernel sets when
// one of its blocks gave up its bounded wait (the call's scales are then NaN;
// the bit stays set until the workspace is zero-filled again).
constexpr int kBarGen = 0, kBarTop = kArrivalStride, kBarStatus = 2 * kArrivalStride, kBarWords = 3 * kArrivalStride;
// Line 0, words 8-9: the one-pass per-channel kernel's tensor-wide non-finite
// flag, a 64-bit word (generation in the high half, 1 in the low half when a
// tile of that launch held an Inf or NaN).
constexpr int kBarColFlag = 8;
constexpr uint32_t kGaveUpBit = 1u;
constexpr size_t kArrivalOffsetWords = kMaxTensorPartials;
constexpr size_t kBarrierOffsetWords = kArrivalOffsetWords + (size_t)kArrivalGroups * kArrivalStride;
constexpr size_t kTensorWorkspaceBytes = (kBarrierOffsetWords + kBarWords) * 4;
constexpr int kColChunkRows = 128;        // rows per partial in the per-column pass

int tensor_partial_blocks(size_t nvec);   // partials written by the per-tensor passes
int col_chunks(int rows);                 // partial rows of the per-column pass

// `sr`: stochastic rounding to E5M2 (fmt must be E5M2) with hash key `seed`.
hipError_t launch_quant_rows(const void* x, int xt, int rows, int cols, int fmt, uint8_t* q, float* scale,
                             float* amax, bool sr, uint64_t seed, hipStream_t st);
// Per-row dynamic quantization of a weight [rows, cols] straight into the
// pre-shuffled layout qp (and row-major codes into q when non-null).
hipError_t launch_quant_rows_pre(const void* x, int xt, int rows, int cols, int fmt, uint8_t* q, uint8_t* qp,
                                 float* scale, float* amax, hipStream_t st);
hipError_t launch_quant_tensor(const void* x, int xt, size_t numel, int fmt, uint8_t* q, float* scale,
                               float* amax, void* ws, bool sr, uint64_t seed, hipStream_t st);
hipError_t launch_quant_cols(const void* x, int xt, int rows, int cols, int fmt, uint8_t* q, float* scale,
                             float* amax, void* ws, bool sr, uint64_t seed, hipStream_t st);
hipError_t launch_quant_delayed(const void* x, int xt, size_t numel, int fmt, uint8_t* q, float* scale,
                                float* amax, float* state, int len, int idx, int margin, int32_t* flag, void* ws,
                                bool sr, uint64_t seed, hipStream_t st);
// Per-tensor codes of a row-major [rows, cols] tensor in up to four layouts
// (null pointers are skipped): row-major, transposed [cols, rows], and the
// pre-shuffled weight layout of either (N = rows, K = cols, or N = cols,
// K = rows; np_* = N padded to 32, kb_* = K blocks of 128).
struct LayoutOut {
  uint8_t* q;
  uint8_t* qt;
  uint8_t* qp;
  uint8_t* qtp;
  int np_q, kb_q;
  int np_t, kb_t;
};
// Scale: scale_in (given), else the ring in state (delayed), else dynamic
// (a partial-amax pass first, partials in ws).
hipError_t launch_quant_layouts(const void* x, int xt, int rows, int cols, int fmt, const LayoutOut& o,
                                const float* scale_in, float* scale_out, float* amax, float* state, int len, int idx,
                                int margin, int32_t* flag, void* ws, bool sr, uint64_t seed, hipStream_t st);
hipError_t launch_ring_update(float* state, int len, int idx, int margin, int32_t* flag, const float* amax,
                              int fmt, hipStream_t st);

hipError_t launch_preshuffle(const uint8_t* wq, int n, int k, uint8_t* out, hipStream_t st);
hipError_t launch_stream_rows_probe(const void* x, int64_t rows, int row_vecs, int waves, uint8_t* q,
                                    hipStream_t st);

// Epilogue bias kinds (GemmArgs::bias_kind).
constexpr int kBiasNone = 0, kBiasBF16 = 1, kBiasE4M3 = 2, kBiasE5M2 = 3;

struct GemmArgs {
  const uint8_t* xq;      // [m, k] row-major
  const uint8_t* wq_pre;  // pre-shuffled weight(s)
  const float* x_scale;   // [1] or [m]
  const float* w_scale;   // [1] or [n] (per expert in the grouped form)
  void* out;              // bf16 [m, n]; FP8 codes [m, n] when out_scale is set
  int m, n, k;
  int x_scale_per_row;    // 0: x_scale[0] for every row
  int w_scale_per_col;    // 0: w_scale[0] (per expert) for every column
  // Epilogue (all zero: bf16 output, no bias). v = fl32(fl32(acc * x_s) * w_s);
  // with a bias v = fl32(v + bias[col]); out = bf16(v), or with out_scale the
  // FP8 (out_fmt) code of fl32(v * fl32(1 / out_scale[0])).
  const void* bias;        // [n]: bf16 bits or FP8 codes, per bias_kind
  int bias_kind;           // kBias*
  const float* bias_scale; // [1]: dequant scale of an FP8 bias
  const float* out_scale;  // [1] or null
  int out_fmt;             // kE4M3 / kE5M2 (with out_scale)
  // Block-scaled form only (launch_gemm_bsf): the number of K blocks; x_scale
  // is then [m, nblk] and w_scale [n, nblk], row-major.
  int nblk;
  // Strict form (launch_gemm, launch_grouped_gemm): products on the float16
  // matrix-core instructions, which keep every product bit, instead of the FP8
  // ones, whose 8-product runs drop bits 13 below the run's largest exponent.
  int strict;
};

// Decode-shape (small M) launch plan: MB 16-row activation blocks, F weight
// fragments per group, KPW K blocks per wavefront chunk, `groups` fragment
// groups, each split over `splits` workgroups; workspace_bytes is what the
// split needs (0 when splits == 1).
// halves = 2: each group is one half (8 of the 16 slots) of a weight fragment,
// so a narrow N still gives every CU a group without splitting K.
struct SkinnyPlan {
  int mb, f, kpw, groups, splits, halves, waves, kb;  // kb: 128-deep K blocks
  size_t workspace_bytes;
};
SkinnyPlan skinny_plan(int m, int n, int k);

// Scratch the GEMM can use for m x n x k (0: none). With less (or none) the
// launch runs unsplit. Its leading counters must be zero before first use and
// are left zero by every launch.
size_t gemm_workspace_bytes(int m, int n, int k);
hipError_t launch_gemm(const GemmArgs& a, int xf, int wf, void* workspace, size_t workspace_bytes, hipStream_t st);

// Library-held GEMM scratch for callers that cannot allocate: a file-scope
// device array of kNoAllocScratchBytes per GPU (the largest split plan needs
// under 4.1 MiB). noalloc_scratch returns the current device's address of it,
// looked up once per device with hipGetSymbolAddress, whose counter region is
// zeroed at that first lookup by a kernel on `st`.
constexpr size_t kNoAllocScratchBytes = (size_t)4352 << 10;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(hipStream_t st, void** ptr);

// Block-wise quantization: scales [rows, ceil(cols / bs)], bs in {16, 32, 64, 128}.
hipError_t launch_quant_blocks(const void* x, int xt, int rows, int cols, int fmt, int bs, bool sr, uint64_t seed,
                               uint8_t* q, float* scale, float* amax, hipStream_t st);

// Block-scaled GEMM on row-major codes: xs [m, nb], ws [n, nb], nb = ceil(k / bs), bs in {32, 64, 128}.
struct BlockGemmArgs {
  const uint8_t* xq;  // [m, k]
  const uint8_t* wq;  // [n, k]
  const float* xs;    // [m, nb]
  const float* ws;    // [n, nb]
  const uint16_t* bias;  // bf16 [n], or null
  uint16_t* out;      // bf16 [m, n]
  int m, n, k, nb;
};
hipError_t launch_gemm_blockscaled(const BlockGemmArgs& a, int xf, int wf, int bs, hipStream_t st);
// Block-scaled GEMM with blocks of bs (32, 64, 128) along K over the
// pre-shuffled weight (the plain GEMM's data path, each block's sums folded
// with its two scales).
hipError_t launch_gemm_bsf(const GemmArgs& a, int xf, int wf, int bs, hipStream_t st);

// Grouped form: rows [offsets[e], offsets[e+1]) use expert e's weight at
// wq_pre + e * preshuffled_bytes(n, k) and scales w_scale + e * (per_col ? n : 1).
hipError_t launch_grouped_gemm(const GemmArgs& a, const int32_t* offsets, int experts, int xf, int wf,
                               hipStream_t st);

}  // namespace hq
