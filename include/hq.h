/*
 * hq.h -- C ABI of the MI355X (gfx950) FP8 dynamic-quantization + scaled FP8
 * (a8w8) GEMM library, libhq.so.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device; host pointers are marked "host". The caller allocates
 *    and owns every buffer (inputs, outputs, workspaces, ring state). The
 *    library allocates nothing, frees nothing and keeps no pointer after a call
 *    returns (the caller-owned output of the aiter PR "gemm_a8w8_bpreshuffle_out",
 *    Technical Details).
 *  - Every call is asynchronous on `stream` (0 = the null stream): it validates
 *    its arguments on the host, then enqueues kernels and returns.
 *  - Errors: a status code, plus a thread-local message from hq_last_error().
 *    All argument checks run before any launch, and on any error nothing is
 *    written (aiter PR, Technical Details and Test Plan). The architecture check
 *    (gfx950 only, cached per device) runs after the argument checks, so an
 *    invalid argument always reports HQ_ERR_INVALID_ARGUMENT.
 *  - Not checked (documented preconditions, since checking needs a device sync):
 *    that device pointers are device memory of the current device (operands on
 *    a non-current device faulted in the aiter PR's review), that scale values
 *    are positive and finite (hip-quant README, "Memory Safety"), and that
 *    grouped-GEMM offsets are valid (the kernels clamp them, so invalid offsets
 *    give wrong rows but never an out-of-bounds access).
 *  - Sizes are int64 on the ABI and must fit int32 where the kernels index with
 *    32-bit math (hip-quant README, "Memory Safety": checked narrowing).
 *  - Enum-typed parameters are passed as C `int`.
 */
#ifndef HQ_H
#define HQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hq_status {
  HQ_OK = 0,
  HQ_ERR_INVALID_ARGUMENT = 1,   /* bad pointer, size, alignment, overlap, enum  */
  HQ_ERR_UNSUPPORTED_DEVICE = 2, /* no HIP device, or the current one is not gfx950 */
  HQ_ERR_LAUNCH = 3              /* the HIP runtime rejected a kernel launch     */
} hq_status;

/* FP8 formats (hip-quant README, table "FP8 Formats (both APIs)"): E4M3 bias 7,
 * max 448, NaN only; E5M2 bias 15, max 57344, +-Inf and NaN. Casts are
 * saturating round-to-nearest-even; NaN encodes to 0x7F; +-Inf saturates. */
typedef enum hq_fp8 { HQ_E4M3 = 0, HQ_E5M2 = 1 } hq_fp8;

/* Element type of a high-precision input tensor. */
typedef enum hq_dtype { HQ_F32 = 0, HQ_BF16 = 1 } hq_dtype;

/* Scale granularity (fuel-ir 0.22.4 quant_scale.rs, ScaleGranularity): one scale
 * for the tensor, one per row ("token"), or one per column ("channel") of a
 * row-major [rows, cols] tensor. A GEMM weight W [N, K] gets its
 * per-output-channel scales from the per-row call (HQ_PER_TOKEN) on W. */
typedef enum hq_gran { HQ_PER_TENSOR = 0, HQ_PER_TOKEN = 1, HQ_PER_CHANNEL = 2 } hq_gran;

/* Delayed-scaling state (AstrAI ops.cu, pack_quantize_params and the commit
 * "finalize fp8 scale rings inside quantize kernels"): `state` is a device
 * float32 buffer of len + 2 entries laid out as
 *     [hist[0 .. len-1] | scale | counter]
 * Initialise it to hist = 0, scale = 1.0, counter = 0 (all bits zero); the
 * counter is 0 again after every call. `idx` is this step's history slot
 * (0 <= idx < len), `margin` the power-of-two headroom of the next scale
 * (-64 <= margin <= 64). `nonfinite_flag` is an optional device int32 that a
 * call sets to 1 (never clears) when it sees a NaN or Inf amax sample
 * (hip-quant README, "Training-path numerical guards"). */
typedef struct hq_ring {
  float* state;
  int32_t len;
  int32_t idx;
  int32_t margin;
  int32_t* nonfinite_flag;
} hq_ring;

/* Number of float32 scales for a [rows, cols] tensor: 1, rows or cols
 * (fuel-ir quant_scale.rs, ScaleGranularity::scale_count). Returns -1 for an
 * unknown granularity or negative sizes. */
int64_t hq_scale_count(int gran, int64_t rows, int64_t cols);

/* Bytes of device workspace hq_quantize_fp8 needs for this granularity and
 * shape: 0 for HQ_PER_TOKEN; for HQ_PER_TENSOR (dynamic or delayed) a fixed
 * 8576-byte region of block partials, arrival counters, the single-pass grid
 * barrier and its status word; for HQ_PER_CHANNEL that region plus (ceil(rows/128) + 1) * cols * 8
 * bytes of column partials and per-column words after it (so one workspace
 * sized for the largest call serves every granularity). Returns 0 for invalid arguments (hq_quantize_fp8
 * then reports the error). */
size_t hq_quantize_workspace_bytes(int gran, int64_t rows, int64_t cols);

/* Dynamic (or delayed) FP8 quantization of a row-major [rows, cols] tensor.
 *
 * Dynamic (ring == NULL), for each group of the granularity:
 *   amax  = max |x| over the group's finite elements
 *   s     = max(fl32(amax / fmax), 2^-126)        fmax = 448 (E4M3) or 57344 (E5M2)
 *   r     = fl32(1 / s)
 *   q     = saturating RNE cast of fl32(x * r)
 * (the method statement: amax reduction, scale = amax / 448, saturating RNE cast;
 * hip-quant README "Training-path numerical guards": the reciprocal of the
 * pre-quant multiplier is the dequant scale). x ~= decode(q) * s.
 *
 * Delayed (ring != NULL, gran must be HQ_PER_TENSOR): s is the ring's scale as
 * read when the call starts, q is cast with r = fl32(1/s); the tensor's amax is
 * then folded into the ring in the same launch (last-block epilogue), exactly as
 * hq_scale_ring_update would: hist[idx] = amax, next scale =
 * max(hist) * 2^margin / fmax. A tensor holding any NaN/Inf leaves the ring
 * unchanged and sets *nonfinite_flag.
 *
 *   x          device, [rows, cols] of `xt`, row-major, 16-byte aligned
 *   q          device, [rows, cols] uint8 FP8 codes, row-major, 16-byte aligned
 *   scale_out  device, float32 [hq_scale_count(gran, rows, cols)]: the dequant
 *              scales s used for the codes (in delayed mode, the ring's s_t)
 *   amax_out   device, optional (NULL), float32 [scale_count]: the group amax
 *   ring       host pointer to an hq_ring, or NULL for dynamic scaling
 *   workspace  device, at least hq_quantize_workspace_bytes(gran, rows, cols)
 *              bytes (may be NULL when that is 0). Zero-fill it once before
 *              its first call: its counters (delayed scaling, and the grid
 *              barrier of the single-pass per-tensor kernel) start from zero,
 *              and every call leaves them ready for the next. Calls that share
 *              a workspace must not run concurrently. Dynamic per-tensor
 *              quantization of up to 2^24 bf16 (2^23 float32) elements, and
 *              per-channel quantization whose tiles of 128 rows x 256 bf16
 *              (128 float32) columns number at most 512, run as one pass over
 *              x whose blocks agree on the maxima through the workspace;
 *              other sizes take a partial-max pass first. The one-pass form
 *              needs its whole grid resident at once (checked by an occupancy
 *              query before the launch); a block that still waits longer than
 *              0.5 s (other work holding the device) gives up, the call's
 *              affected scales come out NaN, and a sticky bit in the workspace
 *              records it (hq_quantize_workspace_status).
 * Requires cols % 16 == 0 (16-byte vector rows), 1 <= rows, cols <= 2^31 - 1024,
 * rows * cols < 2^40. rows == 0 returns HQ_OK without a launch. Outputs must not
 * overlap inputs. */
hq_status hq_quantize_fp8(const void* x, int xt, int64_t rows, int64_t cols,
                          int fmt, int gran, uint8_t* q, float* scale_out,
                          float* amax_out, const hq_ring* ring,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Whether any one-pass per-tensor or per-channel call on this quantize
 * workspace (since it was last zero-filled) gave up its grid wait: *gave_up = 1
 * if so (that call's scales, or those of the columns it covered, are NaN and
 * the call should be repeated after zero-filling the workspace), else 0. Reads
 * the workspace's status word after the work already on `stream` (a
 * synchronous device-to-host copy: not for the hot path).
 *   workspace  device, a quantize workspace of workspace_bytes >=
 *              hq_quantize_workspace_bytes(HQ_PER_TENSOR, 1, 16) bytes
 *   gave_up    host pointer */
hq_status hq_quantize_workspace_status(const void* workspace, size_t workspace_bytes, int32_t* gave_up,
                                       hipStream_t stream);

/* hq_quantize_fp8 to E5M2 with stochastic rounding (hip-quant README,
 * "Stochastic E5M2 Backward Gradients": each value rounds to one of the two
 * adjacent E5M2 values, up with probability proportional to its distance from
 * the lower one, drawn from a stateless hash of (seed, element index), so the
 * result is reproducible). Scales, granularities, the ring and every argument
 * rule are those of hq_quantize_fp8 with fmt = HQ_E5M2; only the cast of
 * y = fl32(x * r) differs:
 *   u = (w >> 8) * 2^-24, w = word i % 4 of Philox-4x32-10 (Salmon et al.,
 *       SC 2011) with counter (i/4 low 32 bits, i/4 high 32 bits, 0, 0) and
 *       key (seed low, seed high), i = row-major flat index of the element
 *   lo <= |y| < hi adjacent E5M2 magnitudes; the code's magnitude is hi when
 *       u < (|y| - lo) / (hi - lo), else lo; the sign of y is kept
 *   |y| >= 57344 or Inf saturates to +-57344, NaN gives 0x7F. */
hq_status hq_quantize_fp8_stochastic(const void* x, int xt, int64_t rows, int64_t cols, int gran,
                                     uint64_t seed, uint8_t* q, float* scale_out,
                                     float* amax_out, const hq_ring* ring,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Per-tensor FP8 quantization of a row-major [rows, cols] tensor written, in
 * one pass over x, to any of four layouts (the fused quantize-plus-transpose
 * of the hip-quant README, "Runtime codebooks and GPU execution features").
 * Per-tensor codes do not depend on where they are stored, so each layout
 * holds exactly the codes hq_quantize_fp8 would give (transposed or
 * reordered):
 *   q        [rows, cols] row-major codes
 *   q_t      [cols, rows] row-major codes of the transpose
 *   q_pre    hq_preshuffle_weight of q     (a GEMM weight with N = rows, K = cols)
 *   q_t_pre  hq_preshuffle_weight of q_t   (N = cols, K = rows)
 * Any of them may be NULL; at least one must not be. The pre-shuffled forms
 * are sized hq_preshuffled_bytes(rows, cols) and hq_preshuffled_bytes(cols,
 * rows), padding included (written as zero codes). For the backward GEMMs of a
 * linear layer this replaces the transposed copies and the pre-shuffle passes.
 *
 * The scale comes from exactly one source:
 *   scale_in != NULL  a given per-tensor dequant scale s (device float32 [1]):
 *                     q = cast(fl32(x * fl32(1/s))), no reduction (AstrAI
 *                     ops.cu, linear_backward_fp8: the weight and input are
 *                     quantized again with their forward scales, no ring);
 *                     amax_out must be NULL; no workspace is used
 *   ring != NULL      delayed scaling, exactly as hq_quantize_fp8 with a ring
 *   both NULL         dynamic per-tensor, exactly as hq_quantize_fp8 with
 *                     HQ_PER_TENSOR (a partial-amax pass, then this pass)
 * scale_out (device float32 [1]) receives the scale used; amax_out (optional)
 * the tensor amax. workspace: hq_quantize_workspace_bytes(HQ_PER_TENSOR, rows,
 * cols) bytes for the ring and dynamic forms, under the same zero-fill-once
 * rule as hq_quantize_fp8 (may be NULL with scale_in).
 * Requires cols % 16 == 0, and rows % 16 == 0 when q_t or q_t_pre is asked
 * for; rows, cols <= 2^31 - 1024, rows * cols < 2^40; 16-byte aligned x and
 * code buffers; no output may overlap another
 * buffer. rows == 0 returns HQ_OK without a launch. */
hq_status hq_quantize_fp8_layouts(const void* x, int xt, int64_t rows, int64_t cols, int fmt,
                                  const float* scale_in, const hq_ring* ring,
                                  uint8_t* q, uint8_t* q_t, uint8_t* q_pre, uint8_t* q_t_pre,
                                  float* scale_out, float* amax_out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The layouts call with stochastic rounding to E5M2 (hip-quant README,
 * "Stochastic E5M2 Backward Gradients": a gradient is the tensor rounded
 * stochastically, and the backward pass needs it row-major for one GEMM and
 * transposed for the other). Codes are those of hq_quantize_fp8_stochastic:
 * element (r, c) of x draws from its row-major index r * cols + c, so every
 * layout of an element carries the same code, and with a dynamic scale the
 * row-major codes equal hq_quantize_fp8_stochastic's per-tensor codes for the
 * same seed. Other arguments, the scale modes and the requirements are those
 * of hq_quantize_fp8_layouts with fmt = HQ_E5M2. */
hq_status hq_quantize_fp8_layouts_stochastic(const void* x, int xt, int64_t rows, int64_t cols, uint64_t seed,
                                             const float* scale_in, const hq_ring* ring, uint8_t* q, uint8_t* q_t,
                                             uint8_t* q_pre, uint8_t* q_t_pre, float* scale_out, float* amax_out,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Block-wise FP8 quantization (hip-quant README, "Block-wise FP8 Scaling"):
 * FP8 codes plus one float32 dequant scale per block of block_size consecutive
 * elements along each row, value ~= code * block_scale. Each block follows the
 * rule of hq_quantize_fp8 (amax over its finite elements, s = max(amax / fmax,
 * 2^-126), q = saturating RNE cast of fl32(x * fl32(1/s))); the last block of a
 * row holds cols mod block_size elements when that is not zero. With
 * `stochastic` != 0 the cast is the stochastic E5M2 of
 * hq_quantize_fp8_stochastic (fmt must be HQ_E5M2; element index = row-major
 * flat index) - the README's quantize_e5m2_blockwise_stochastic.
 *   x         device, [rows, cols] of `xt`, row-major, 16-byte aligned
 *   q         device, [rows, cols] uint8 codes, 16-byte aligned
 *   scales    device, float32 [rows, ceil(cols / block_size)] row-major
 *   amax_out  device, optional, float32 of the same shape: the block amax
 * Requires block_size in {16, 32, 64, 128}, cols % 16 == 0, 1 <= rows,
 * cols <= 2^31 - 1024, rows * cols < 2^40; no output may overlap an input. rows == 0
 * returns HQ_OK without a launch. */
hq_status hq_quantize_fp8_blockwise(const void* x, int xt, int64_t rows, int64_t cols, int fmt,
                                    int block_size, int stochastic, uint64_t seed,
                                    uint8_t* q, float* scales, float* amax_out,
                                    hipStream_t stream);

/* Block-scaled FP8 GEMM (hip-quant README, "Block-scaled Linear ...": the
 * pre-quantized path consumes FP8 bytes, both block-scale tensors and an
 * optional bias):
 *   out[m, n] = bf16( sum_b x_scales[m, b] * w_scales[n, b] *
 *                     sum_{k in block b} dec(XQ[m, k]) * dec(WQ[n, k])  + bias[n] )
 * Each block's partial sum (float32 MFMAs) is folded into the float32 result
 * with one fused multiply-add by the float32 product of the two scales; the
 * bias (bf16, output units) is then added in float32.
 *   xq        device, uint8 [m, k] codes in format xf, row-major, 16-byte aligned
 *   wq        device, uint8 [n, k] codes in format wf, row-major (not
 *             pre-shuffled), 16-byte aligned
 *   x_scales  device, float32 [m, ceil(k / block_size)]
 *   w_scales  device, float32 [n, ceil(k / block_size)]
 *   bias      device, bf16 bits [n], 2-byte aligned, or NULL for none
 *   out       device, bf16 bits [m, n], caller-owned, must not overlap an input
 * Requires block_size in {32, 64, 128}, k % 16 == 0, 16 <= k < 2^24. m == 0 or
 * n == 0 returns HQ_OK without a launch. */
hq_status hq_gemm_a8w8_blockscaled(const uint8_t* xq, int xf, const uint8_t* wq, int wf,
                                   const float* x_scales, const float* w_scales, int block_size,
                                   int64_t m, int64_t n, int64_t k, const uint16_t* bias,
                                   uint16_t* out, hipStream_t stream);

/* hq_gemm_a8w8_blockscaled with the weight pre-shuffled (hq_preshuffle_weight
 * of WQ [n, k]; as in hq_gemm_a8w8): the same operation and the same per-block
 * fold in K order,
 *   out[m, n] = bf16( fl32-fold over b of fma(S_b[m,n], fl32(xs[m,b] * ws[n,b]), . ) + bias[n] )
 * with S_b the float32 MFMA sum over block b, on the plain GEMM's data path.
 * Blocks of 128 give the same bits as hq_gemm_a8w8_blockscaled; blocks of 32
 * and 64 sum each block on the 128-deep MFMA (the other chunks scaled out),
 * within the same error bound.
 *   wq_pre      device, hq_preshuffled_bytes(n, k) bytes, 16-byte aligned
 *   block_size  32, 64 or 128; x_scales [m, ceil(k/bs)], w_scales [n, ceil(k/bs)]
 *   out         device bf16 [m, n], 16-byte aligned
 * All other arguments and requirements are those of hq_gemm_a8w8_blockscaled. */
hq_status hq_gemm_a8w8_blockscaled_preshuffled(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf,
                                               const float* x_scales, const float* w_scales, int block_size,
                                               int64_t m, int64_t n, int64_t k, const uint16_t* bias,
                                               uint16_t* out, hipStream_t stream);

/* Fold one amax sample into a ring and publish the next scale (the delayed
 * update of hq_quantize_fp8, as its own launch). `amax` is a device float32
 * scalar; a NaN or Inf sample leaves the ring unchanged and sets the flag. */
hq_status hq_scale_ring_update(const hq_ring* ring, const float* amax, int fmt,
                               hipStream_t stream);

/* Bytes of the pre-shuffled form of an [n, k] FP8 weight:
 * ceil(n/32)*32 * ceil(k/128)*128. Returns -1 for invalid sizes. */
int64_t hq_preshuffled_bytes(int64_t n, int64_t k);

/* Reorder a row-major FP8 weight WQ [n, k] into the GEMM's pre-shuffled layout
 * (the aiter PR has the GEMM read a pre-shuffled, optionally K-padded weight;
 * the order is this library's). n is padded to a multiple of 32 and k to a
 * multiple of 128 with zero bytes. Row n = 32*G + 8*g + 4*p + r (g < 4, p < 2,
 * r < 4) becomes slot s = 4*g + r of fragment nb = 2*G + p; fragment (nb, kb)
 * holds 16 slots x 128 columns at byte (nb * ceil(k/128) + kb) * 2048, and the
 * byte of (slot s, column k_in) sits at h*1024 + (q*16 + s)*16 + b with
 * q = k_in/32, h = (k_in%32)/16, b = k_in%16.
 *   wq      device, uint8 [n, k] row-major, 16-byte aligned, k % 16 == 0
 *   wq_pre  device, hq_preshuffled_bytes(n, k) bytes, 16-byte aligned */
hq_status hq_preshuffle_weight(const uint8_t* wq, int64_t n, int64_t k,
                               uint8_t* wq_pre, hipStream_t stream);

/* Per-row dynamic quantization of a weight x [rows, cols] (rows = the GEMM's
 * output channels N, cols = K) written straight into the pre-shuffled layout:
 * the codes, scales and amax are exactly those of hq_quantize_fp8 with
 * HQ_PER_TOKEN (per output channel of the weight, the PTPC weight side of the
 * aiter PR), and q_pre is byte for byte hq_preshuffle_weight of those codes,
 * padding included (zero codes), without the row-major copy in between.
 *   x          device, fp32 / bf16 [rows, cols] row-major, 16-byte aligned
 *   q          device uint8 [rows, cols] row-major codes, or NULL for none
 *   q_pre      device, hq_preshuffled_bytes(rows, cols) bytes, 16-byte aligned
 *   scale_out  device float32 [rows]; amax_out device float32 [rows] or NULL
 * Requires cols % 16 == 0, rows, cols <= 2^31 - 1024; no output may overlap another
 * buffer. rows == 0 returns HQ_OK without a launch. */
hq_status hq_quantize_fp8_preshuffled(const void* x, int xt, int64_t rows, int64_t cols, int fmt,
                                      uint8_t* q, uint8_t* q_pre, float* scale_out, float* amax_out,
                                      hipStream_t stream);

/* Bytes of GEMM workspace worth passing to hq_gemm_a8w8 for an m x n x k
 * product: nonzero only for the decode shapes (1 <= m <= 64) whose weight
 * stream is split over several workgroups per column group. Returns -1 for
 * invalid sizes. */
int64_t hq_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Scaled FP8 GEMM into a caller-owned bf16 buffer (the method statement; the
 * operand set of the aiter PR's gemm_a8w8_bpreshuffle_out):
 *   out[m, n] = bf16_rne( fp32( sum_k dec(XQ[m,k]) * dec(WQ[n,k]) ) * x_scale[m] * w_scale[n] )
 * accumulated in fp32 on gfx950 FP8 MFMA.
 *   xq        device, uint8 [m, k] codes in format xf, row-major, 16-byte aligned
 *   wq_pre    device, hq_preshuffle_weight(WQ [n, k]) in format wf
 *   x_scale   device, float32 [x_scale_count], x_scale_count = 1 or m
 *   w_scale   device, float32 [w_scale_count], w_scale_count = 1 or n
 *   out       device, bf16 bits [m, n] dense row-major, 16-byte aligned; must not
 *             overlap any input. Written in full; nothing else is touched.
 *   workspace device scratch of workspace_bytes bytes, 16-byte aligned, or NULL
 *             with workspace_bytes == 0. Zero-fill it once before its first
 *             use: its first 1024 bytes are per-column-group arrival counters
 *             that every call leaves at zero again, the rest holds partial sums
 *             and needs no reset (the layout does not depend on the shape, so
 *             one workspace serves calls of any shapes). With at least
 *             hq_gemm_workspace_bytes(m, n, k) bytes the decode shapes split
 *             their weight stream over more workgroups; with less they run
 *             unsplit, slower but with the same output bits (the order of the
 *             sums depends only on m, n and k).
 *             Calls that share a workspace must not run concurrently.
 * Requires k % 16 == 0, 16 <= k < 2^24, m, n <= 2^31 - 1024. m == 0 or n == 0 returns HQ_OK
 * without a launch (aiter PR: an empty out is a no-op). */
hq_status hq_gemm_a8w8(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf,
                       const float* x_scale, int64_t x_scale_count,
                       const float* w_scale, int64_t w_scale_count,
                       int64_t m, int64_t n, int64_t k, uint16_t* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* hq_gemm_a8w8 for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation, arguments, requirements and output bits, with no workspace
 * argument. The split decode launches (1 <= m <= 64) take their scratch from
 * a device array the library holds for each GPU (4.25 MiB, kept until the
 * process ends; its address is looked up once per device, and the first call
 * on a device also enqueues a small kernel on `stream` that zeroes the
 * array's counters). The call allocates nothing: no hipMalloc, no hipFree. A
 * shape whose split plan needs more scratch than that is rejected with
 * HQ_ERR_INVALID_ARGUMENT (no valid shape does today: the largest plan needs
 * under 4.1 MiB). Every call on a GPU shares that GPU's array, which keeps the
 * last call's partial sums: calls that overlap on one GPU (concurrent
 * streams, host threads) race and must not be made. */
hq_status hq_gemm_a8w8_noalloc(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf,
                               const float* x_scale, int64_t x_scale_count,
                               const float* w_scale, int64_t w_scale_count,
                               int64_t m, int64_t n, int64_t k, uint16_t* out,
                               hipStream_t stream);

/* Kinds of GEMM epilogue bias (AstrAI ops.cu, linear_forward_fp8: a bf16 bias
 * as is, or a pre-quantized FP8 bias with its bias_scale). */
typedef enum hq_bias { HQ_BIAS_BF16 = 0, HQ_BIAS_E4M3 = 1, HQ_BIAS_E5M2 = 2 } hq_bias;

/* GEMM epilogue options (host struct):
 *   bias        device [n], one value per output column: bf16 bits
 *               (HQ_BIAS_BF16) or FP8 codes (HQ_BIAS_E4M3 / HQ_BIAS_E5M2);
 *               NULL for no bias
 *   bias_type   an hq_bias value
 *   bias_scale  device float32 [1]: dequant scale of an FP8 bias (required
 *               for FP8, must be NULL for bf16)
 *   out_scale   device float32 [1]: when non-NULL the output is FP8 codes
 *               (AstrAI ops.cu, mm_fp8: FP8 E4M3 output "requires out_scale,
 *               the output quantization step"); NULL for bf16 output
 *   out_fmt     HQ_E4M3 or HQ_E5M2, the FP8 output format (with out_scale) */
typedef struct hq_epilogue {
  const void* bias;
  int32_t bias_type;
  const float* bias_scale;
  const float* out_scale;
  int32_t out_fmt;
} hq_epilogue;

/* hq_gemm_a8w8 with an epilogue. Per output element, in float32:
 *   v = fl32(fl32(acc * x_scale[m]) * w_scale[n])
 *   v = fl32(v + b[n])        with a bias, b = bf16 value or fl32(dec(code) * bias_scale)
 *   out[m, n] = bf16_rne(v), or with out_scale the saturating RNE FP8 code of
 *               fl32(v * fl32(1 / out_scale))   (NaN -> 0x7F)
 * `ep` is a host pointer (NULL = plain bf16 output, exactly hq_gemm_a8w8).
 * `out` is bf16 [m, n] (2 bytes per element) or uint8 codes [m, n] with
 * out_scale; 16-byte aligned, caller-owned, must not overlap any input. All
 * other arguments, the workspace rule and the requirements are those of
 * hq_gemm_a8w8. */
hq_status hq_gemm_a8w8_epilogue(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf,
                                const float* x_scale, int64_t x_scale_count,
                                const float* w_scale, int64_t w_scale_count,
                                int64_t m, int64_t n, int64_t k, const hq_epilogue* ep,
                                void* out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* hq_gemm_a8w8_epilogue whose products are summed without the FP8 matrix
 * cores' run window: the same operation, arguments, requirements, workspace
 * rule and epilogue, computed with every product exact.
 * The GEMM the method states accumulates in float32 and is compared with the
 * exact sum within 2 bf16 ulp + 2^-22 * sum_k |x_scale * w_scale * dec * dec|
 * per element. The gfx950 FP8 instructions (hq_gemm_a8w8) add each run of 8
 * consecutive-k products in a fixed-point window: a product is truncated
 * toward zero at 2^(P - 13), P the largest exponent sum e(x) + e(w) of the
 * run's non-zero products, so a run holding one product 2^14 times larger
 * than the others loses the others' low bits, and ~0.1 % of the elements of a
 * GEMM with outlier activations fall outside that bound. This entry point
 * converts each operand byte to float16 (exact for E4M3 and E5M2, NaN and Inf
 * included) and runs the float16 matrix-core instructions, which keep every
 * product bit; sums are float32. Costs about twice the FP8 path's time at
 * large shapes (half the matrix-core rate); decode shapes (m <= 64) stay
 * bound by the weight stream. */
hq_status hq_gemm_a8w8_strict(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf,
                              const float* x_scale, int64_t x_scale_count,
                              const float* w_scale, int64_t w_scale_count,
                              int64_t m, int64_t n, int64_t k, const hq_epilogue* ep,
                              void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Grouped (per-expert) scaled FP8 GEMM over row ranges (megablocks-hip grouped
 * GEMM notes: per-expert products of concatenated tokens, written over, never
 * accumulated into, the output). For each expert e with rows
 * [offsets[e], offsets[e+1]):
 *   out[t, :] = gemm_a8w8 row t of XQ with expert e's weight and scales
 *   xq             device, uint8 [total_rows, k] row-major, 16-byte aligned
 *   wq_pre         device, num_experts consecutive pre-shuffled weights, each
 *                  hq_preshuffled_bytes(n, k) bytes
 *   x_scale        device, float32 [x_scale_count], 1 or total_rows
 *   w_scale        device, float32 [w_scale_count], num_experts (one per expert)
 *                  or num_experts * n (per expert, per output channel)
 *   group_offsets  device, int32 [num_experts + 1], 0 = offsets[0] <= ... <=
 *                  offsets[num_experts] = total_rows (precondition; clamped)
 *   out            device, bf16 bits [total_rows, n], 16-byte aligned. Rows of
 *                  no group are left untouched.
 * Requires 1 <= num_experts <= 1024, k % 16 == 0, 16 <= k < 2^24. total_rows == 0 or n == 0
 * returns HQ_OK without a launch. */
hq_status hq_grouped_gemm_a8w8(const uint8_t* xq, int xf, const uint8_t* wq_pre,
                               int wf, const float* x_scale, int64_t x_scale_count,
                               const float* w_scale, int64_t w_scale_count,
                               const int32_t* group_offsets, int32_t num_experts,
                               int64_t total_rows, int64_t n, int64_t k,
                               uint16_t* out, hipStream_t stream);

/* hq_grouped_gemm_a8w8 with an epilogue (the hq_gemm_a8w8_epilogue arithmetic
 * per row range; AstrAI ops.cu, linear_forward_fp8 for the bias and output
 * options). Each expert has its own bias row:
 *   ep->bias        device [num_experts, n]: expert e's rows add bias[e, :]
 *                   (bf16 bits, or FP8 codes with a bias_scale)
 *   ep->bias_scale  device float32 [num_experts], one per expert (FP8 bias)
 *   ep->out_scale   device float32 [1], shared by every expert; the output is
 *                   then uint8 codes [total_rows, n] in ep->out_fmt
 * `ep` is a host pointer; NULL is exactly hq_grouped_gemm_a8w8. All other
 * arguments and requirements are those of hq_grouped_gemm_a8w8. */
hq_status hq_grouped_gemm_a8w8_epilogue(const uint8_t* xq, int xf, const uint8_t* wq_pre,
                                        int wf, const float* x_scale, int64_t x_scale_count,
                                        const float* w_scale, int64_t w_scale_count,
                                        const int32_t* group_offsets, int32_t num_experts,
                                        int64_t total_rows, int64_t n, int64_t k,
                                        const hq_epilogue* ep, void* out, hipStream_t stream);

/* hq_grouped_gemm_a8w8_epilogue with exact products (the float16 matrix-core
 * form of hq_gemm_a8w8_strict). Same arguments and requirements. */
hq_status hq_grouped_gemm_a8w8_strict(const uint8_t* xq, int xf, const uint8_t* wq_pre,
                                      int wf, const float* x_scale, int64_t x_scale_count,
                                      const float* w_scale, int64_t w_scale_count,
                                      const int32_t* group_offsets, int32_t num_experts,
                                      int64_t total_rows, int64_t n, int64_t k,
                                      const hq_epilogue* ep, void* out, hipStream_t stream);

/* Row-streaming probe: a measurement aid, not a step of the quantization (no
 * page defines it). It moves the bytes of a per-token quantize pass without
 * its arithmetic: for each of `rows` rows of 16-bit elements it writes the
 * high byte of every element, out[r, i] = x[r, i] >> 8, with the per-token
 * kernel's access pattern (one wavefront per row, 16-byte loads, the next
 * row's loads in flight while the current row is stored, non-temporal 8-byte
 * stores) over a grid of `waves` wavefronts. Timed at the per-token kernel's
 * own grid (12 wavefronts per compute unit) it is the HBM ceiling of a pass of
 * that size and shape.
 *   x          device, 16-bit elements [rows, row_bytes / 2], 16-byte aligned
 *   out        device, uint8 [rows, row_bytes / 2], 8-byte aligned, must not
 *              overlap x
 * Requires row_bytes % 16 == 0, 16 <= row_bytes <= 8192, 1 <= waves <= 2^20,
 * 0 <= rows <= 2^31 - 1024. rows == 0 returns HQ_OK without a launch. */
hq_status hq_stream_rows_probe(const void* x, int64_t rows, int64_t row_bytes, int32_t waves, uint8_t* out,
                               hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* hq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H */
