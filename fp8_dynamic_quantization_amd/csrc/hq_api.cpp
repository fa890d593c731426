// C ABI of libhq: argument validation, the gfx950 gate and kernel dispatch.
//
// Order of checks (aiter PR "gemm_a8w8_bpreshuffle_out", Technical Details):
// every argument check runs on the host before any launch and reports
// HQ_ERR_INVALID_ARGUMENT; then the architecture check (gfx950 only, cached per
// device under a mutex as AstrAI's ops.cu caches its capability check); empty
// problems return HQ_OK without a launch. The memory-safety list of the
// hip-quant README ("Memory Safety": checked narrowing, grid limits, empty
// tensors) is applied to every entry point.
#include "hq.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "hq_launch.h"

namespace {

thread_local std::string g_err;

hq_status fail(hq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hq_status ok() {
  g_err.clear();
  return HQ_OK;
}

constexpr int64_t kI32Max = 2147483647;
// Largest row or column count a launch accepts: grid sizes and tile bounds
// round a dimension up to a multiple of at most 1024 in 32-bit arithmetic.
constexpr int64_t kMaxDim = kI32Max - 1023;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

// Returns the name pair of the first overlapping ranges, or nullptr.
const char* find_overlap(const Range* r, int n, const char** other) {
  for (int i = 0; i < n; ++i) {
    if (!r[i].p || !r[i].bytes) continue;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(r[i].p), a1 = a0 + r[i].bytes;
    for (int j = i + 1; j < n; ++j) {
      if (!r[j].p || !r[j].bytes) continue;
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(r[j].p), b1 = b0 + r[j].bytes;
      if (a0 < b1 && b0 < a1) {
        *other = r[j].name;
        return r[i].name;
      }
    }
  }
  return nullptr;
}

// gfx950 gate for the current device, cached per device in a fixed table (no
// allocation on any call).
hq_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(HQ_ERR_UNSUPPORTED_DEVICE, "no HIP device is available (libhq requires an MI355X / gfx950)");
  }
  if (dev < 0 || dev >= hq::kMaxDevices) return fail(HQ_ERR_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
  static std::mutex mu;
  static int8_t cache[hq::kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
  {
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] != 0) {
      if (cache[dev] < 0) return fail(HQ_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
      return HQ_OK;
    }
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(HQ_ERR_UNSUPPORTED_DEVICE, "cannot query HIP device %d", dev);
  }
  const bool is950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                     (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
  {
    std::lock_guard<std::mutex> lk(mu);
    cache[dev] = is950 ? 1 : -1;
  }
  if (!is950) return fail(HQ_ERR_UNSUPPORTED_DEVICE, "device %d is %s, libhq requires gfx950", dev, prop.gcnArchName);
  return HQ_OK;
}

hq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HQ_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

bool valid_fmt(int f) { return f == HQ_E4M3 || f == HQ_E5M2; }

int64_t padded_bytes(int64_t n, int64_t k) { return ((n + 31) / 32 * 32) * ((k + 127) / 128 * 128); }

hq_status check_ring(const hq_ring* ring) {
  if (!ring->state) return fail(HQ_ERR_INVALID_ARGUMENT, "ring->state is NULL");
  if (!aligned(ring->state, 4)) return fail(HQ_ERR_INVALID_ARGUMENT, "ring->state must be 4-byte aligned");
  if (ring->len < 1 || ring->len > (1 << 20)) return fail(HQ_ERR_INVALID_ARGUMENT, "ring->len must be in [1, 2^20], got %d", ring->len);
  if (ring->idx < 0 || ring->idx >= ring->len)
    return fail(HQ_ERR_INVALID_ARGUMENT, "ring->idx must be in [0, len), got %d (len %d)", ring->idx, ring->len);
  if (ring->margin < -64 || ring->margin > 64)
    return fail(HQ_ERR_INVALID_ARGUMENT, "ring->margin must be in [-64, 64], got %d", ring->margin);
  if (ring->nonfinite_flag && !aligned(ring->nonfinite_flag, 4))
    return fail(HQ_ERR_INVALID_ARGUMENT, "ring->nonfinite_flag must be 4-byte aligned");
  return HQ_OK;
}

}  // namespace

extern "C" {

const char* hq_last_error(void) { return g_err.c_str(); }

int64_t hq_scale_count(int gran, int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return -1;
  switch (gran) {
    case HQ_PER_TENSOR: return 1;
    case HQ_PER_TOKEN: return rows;
    case HQ_PER_CHANNEL: return cols;
    default: return -1;
  }
}

size_t hq_quantize_workspace_bytes(int gran, int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0 || rows > kI32Max || cols > kI32Max) return 0;
  switch (gran) {
    case HQ_PER_TENSOR: return hq::kTensorWorkspaceBytes;
    case HQ_PER_TOKEN: return 0;
    case HQ_PER_CHANNEL: return hq::kTensorWorkspaceBytes + ((size_t)hq::col_chunks((int)rows) + 1) * (size_t)cols * 8;
    default: return 0;
  }
}

int64_t hq_preshuffled_bytes(int64_t n, int64_t k) {
  if (n < 0 || k < 0 || n > kI32Max || k > kI32Max) return -1;
  return padded_bytes(n, k);
}

static hq_status quantize_impl(const void* x, int xt, int64_t rows, int64_t cols, int fmt, int gran, uint8_t* q,
                               float* scale_out, float* amax_out, const hq_ring* ring, void* workspace,
                               size_t workspace_bytes, bool sr, uint64_t seed, hipStream_t stream,
                               const char* name);

hq_status hq_quantize_fp8(const void* x, int xt, int64_t rows, int64_t cols, int fmt, int gran, uint8_t* q,
                          float* scale_out, float* amax_out, const hq_ring* ring, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return quantize_impl(x, xt, rows, cols, fmt, gran, q, scale_out, amax_out, ring, workspace, workspace_bytes, false,
                       0, stream, "hq_quantize_fp8");
}

hq_status hq_quantize_fp8_stochastic(const void* x, int xt, int64_t rows, int64_t cols, int gran, uint64_t seed,
                                     uint8_t* q, float* scale_out, float* amax_out, const hq_ring* ring,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return quantize_impl(x, xt, rows, cols, HQ_E5M2, gran, q, scale_out, amax_out, ring, workspace, workspace_bytes,
                       true, seed, stream, "hq_quantize_fp8_stochastic");
}

static hq_status quantize_impl(const void* x, int xt, int64_t rows, int64_t cols, int fmt, int gran, uint8_t* q,
                               float* scale_out, float* amax_out, const hq_ring* ring, void* workspace,
                               size_t workspace_bytes, bool sr, uint64_t seed, hipStream_t stream,
                               const char* name) {
  if (xt != HQ_F32 && xt != HQ_BF16) return fail(HQ_ERR_INVALID_ARGUMENT, "xt must be HQ_F32 or HQ_BF16, got %d", xt);
  if (!valid_fmt(fmt)) return fail(HQ_ERR_INVALID_ARGUMENT, "fmt must be HQ_E4M3 or HQ_E5M2, got %d", fmt);
  if (gran != HQ_PER_TENSOR && gran != HQ_PER_TOKEN && gran != HQ_PER_CHANNEL)
    return fail(HQ_ERR_INVALID_ARGUMENT, "unknown granularity %d", gran);
  if (rows < 0 || rows > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31 - 1024], got %lld", (long long)rows);
  if (cols < 16 || cols > kMaxDim || cols % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "cols must be a positive multiple of 16, at most 2^31 - 1024, got %lld",
                (long long)cols);
  if ((double)rows * (double)cols > 1099511627776.0) return fail(HQ_ERR_INVALID_ARGUMENT, "rows * cols exceeds 2^40");
  if (ring) {
    if (gran != HQ_PER_TENSOR) return fail(HQ_ERR_INVALID_ARGUMENT, "a delayed-scaling ring requires HQ_PER_TENSOR");
    hq_status st = check_ring(ring);
    if (st != HQ_OK) return st;
  }
  if (gran == HQ_PER_CHANNEL && hq::col_chunks((int)rows) > 65535)
    return fail(HQ_ERR_INVALID_ARGUMENT, "per-channel quantization supports at most %d rows", 65535 * hq::kColChunkRows);
  if (rows == 0) return ok();
  if (!x || !q || !scale_out) return fail(HQ_ERR_INVALID_ARGUMENT, "x, q and scale_out must be non-NULL");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(HQ_ERR_INVALID_ARGUMENT, "x and q must be 16-byte aligned");
  if (!aligned(scale_out, 4) || (amax_out && !aligned(amax_out, 4)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "scale_out and amax_out must be 4-byte aligned");
  const size_t need = ring ? hq::kTensorWorkspaceBytes : hq_quantize_workspace_bytes(gran, rows, cols);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(HQ_ERR_INVALID_ARGUMENT, "workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                  workspace ? "" : " (NULL)");
    if (!aligned(workspace, 4)) return fail(HQ_ERR_INVALID_ARGUMENT, "workspace must be 4-byte aligned");
  }
  const size_t numel = (size_t)rows * (size_t)cols;
  const size_t nscale = (size_t)hq_scale_count(gran, rows, cols);
  const Range rg[] = {
      {x, numel * (xt == HQ_BF16 ? 2 : 4), "x"},
      {q, numel, "q"},
      {scale_out, nscale * 4, "scale_out"},
      {amax_out, amax_out ? nscale * 4 : 0, "amax_out"},
      {workspace, need, "workspace"},
      {ring ? ring->state : nullptr, ring ? ((size_t)ring->len + 2) * 4 : 0, "ring->state"},
      {ring ? ring->nonfinite_flag : nullptr, ring && ring->nonfinite_flag ? 4u : 0u, "ring->nonfinite_flag"},
  };
  const char* other = nullptr;
  if (const char* a = find_overlap(rg, 7, &other)) return fail(HQ_ERR_INVALID_ARGUMENT, "%s overlaps %s", a, other);
  hq_status st = check_device();
  if (st != HQ_OK) return st;
  (void)hipGetLastError();
  hipError_t e;
  if (ring) {
    e = hq::launch_quant_delayed(x, xt, numel, fmt, q, scale_out, amax_out, ring->state, ring->len, ring->idx,
                                 ring->margin, ring->nonfinite_flag, workspace, sr, seed, stream);
  } else if (gran == HQ_PER_TOKEN) {
    e = hq::launch_quant_rows(x, xt, (int)rows, (int)cols, fmt, q, scale_out, amax_out, sr, seed, stream);
  } else if (gran == HQ_PER_TENSOR) {
    e = hq::launch_quant_tensor(x, xt, numel, fmt, q, scale_out, amax_out, workspace, sr, seed, stream);
  } else {
    e = hq::launch_quant_cols(x, xt, (int)rows, (int)cols, fmt, q, scale_out, amax_out, workspace, sr, seed, stream);
  }
  return launched(e, name);
}

static hq_status layouts_impl(const void* x, int xt, int64_t rows, int64_t cols, int fmt, const float* scale_in,
                              const hq_ring* ring, uint8_t* q, uint8_t* q_t, uint8_t* q_pre, uint8_t* q_t_pre,
                              float* scale_out, float* amax_out, void* workspace, size_t workspace_bytes, bool sr,
                              uint64_t seed, hipStream_t stream, const char* name) {
  if (xt != HQ_F32 && xt != HQ_BF16) return fail(HQ_ERR_INVALID_ARGUMENT, "xt must be HQ_F32 or HQ_BF16, got %d", xt);
  if (!valid_fmt(fmt)) return fail(HQ_ERR_INVALID_ARGUMENT, "fmt must be HQ_E4M3 or HQ_E5M2, got %d", fmt);
  if (rows < 0 || rows > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31 - 1024], got %lld", (long long)rows);
  if (cols < 16 || cols > kMaxDim || cols % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "cols must be a positive multiple of 16, at most 2^31 - 1024, got %lld",
                (long long)cols);
  if ((double)rows * (double)cols > 1099511627776.0) return fail(HQ_ERR_INVALID_ARGUMENT, "rows * cols exceeds 2^40");
  if (scale_in && ring) return fail(HQ_ERR_INVALID_ARGUMENT, "give scale_in or ring, not both");
  if (ring) {
    hq_status st = check_ring(ring);
    if (st != HQ_OK) return st;
  }
  if (!q && !q_t && !q_pre && !q_t_pre) return fail(HQ_ERR_INVALID_ARGUMENT, "no output layout requested");
  if ((q_t || q_t_pre) && rows % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "transposed outputs need rows %% 16 == 0, got %lld", (long long)rows);
  if (scale_in && amax_out) return fail(HQ_ERR_INVALID_ARGUMENT, "amax_out is not reported with a given scale_in");
  if (rows == 0) return ok();
  if (!x || !scale_out) return fail(HQ_ERR_INVALID_ARGUMENT, "x and scale_out must be non-NULL");
  if (!aligned(x, 16) || (q && !aligned(q, 16)) || (q_t && !aligned(q_t, 16)) || (q_pre && !aligned(q_pre, 16)) ||
      (q_t_pre && !aligned(q_t_pre, 16)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "x and the code buffers must be 16-byte aligned");
  if (!aligned(scale_out, 4) || (amax_out && !aligned(amax_out, 4)) || (scale_in && !aligned(scale_in, 4)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "scale_in, scale_out and amax_out must be 4-byte aligned");
  const size_t need = scale_in ? 0 : hq::kTensorWorkspaceBytes;
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(HQ_ERR_INVALID_ARGUMENT, "workspace needs %zu bytes, got %zu%s", need, workspace_bytes,
                  workspace ? "" : " (NULL)");
    if (!aligned(workspace, 4)) return fail(HQ_ERR_INVALID_ARGUMENT, "workspace must be 4-byte aligned");
  }
  const size_t numel = (size_t)rows * (size_t)cols;
  const Range rg[] = {
      {x, numel * (xt == HQ_BF16 ? 2 : 4), "x"},
      {q, q ? numel : 0, "q"},
      {q_t, q_t ? numel : 0, "q_t"},
      {q_pre, q_pre ? (size_t)padded_bytes(rows, cols) : 0, "q_pre"},
      {q_t_pre, q_t_pre ? (size_t)padded_bytes(cols, rows) : 0, "q_t_pre"},
      {scale_in, scale_in ? 4u : 0u, "scale_in"},
      {scale_out, 4, "scale_out"},
      {amax_out, amax_out ? 4u : 0u, "amax_out"},
      {workspace, need, "workspace"},
      {ring ? ring->state : nullptr, ring ? ((size_t)ring->len + 2) * 4 : 0, "ring->state"},
      {ring ? ring->nonfinite_flag : nullptr, ring && ring->nonfinite_flag ? 4u : 0u, "ring->nonfinite_flag"},
  };
  const char* other = nullptr;
  if (const char* a = find_overlap(rg, 11, &other)) return fail(HQ_ERR_INVALID_ARGUMENT, "%s overlaps %s", a, other);
  hq_status st = check_device();
  if (st != HQ_OK) return st;
  (void)hipGetLastError();
  hq::LayoutOut o;
  o.q = q;
  o.qt = q_t;
  o.qp = q_pre;
  o.qtp = q_t_pre;
  o.np_q = (int)((rows + 31) / 32 * 32);
  o.kb_q = (int)((cols + 127) / 128);
  o.np_t = (int)((cols + 31) / 32 * 32);
  o.kb_t = (int)((rows + 127) / 128);
  return launched(hq::launch_quant_layouts(x, xt, (int)rows, (int)cols, fmt, o, scale_in, scale_out, amax_out,
                                           ring ? ring->state : nullptr, ring ? ring->len : 0, ring ? ring->idx : 0,
                                           ring ? ring->margin : 0, ring ? ring->nonfinite_flag : nullptr, workspace,
                                           sr, seed, stream),
                  name);
}

hq_status hq_quantize_fp8_layouts(const void* x, int xt, int64_t rows, int64_t cols, int fmt, const float* scale_in,
                                  const hq_ring* ring, uint8_t* q, uint8_t* q_t, uint8_t* q_pre, uint8_t* q_t_pre,
                                  float* scale_out, float* amax_out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  return layouts_impl(x, xt, rows, cols, fmt, scale_in, ring, q, q_t, q_pre, q_t_pre, scale_out, amax_out, workspace,
                      workspace_bytes, false, 0, stream, "hq_quantize_fp8_layouts");
}

hq_status hq_quantize_fp8_layouts_stochastic(const void* x, int xt, int64_t rows, int64_t cols, uint64_t seed,
                                             const float* scale_in, const hq_ring* ring, uint8_t* q, uint8_t* q_t,
                                             uint8_t* q_pre, uint8_t* q_t_pre, float* scale_out, float* amax_out,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return layouts_impl(x, xt, rows, cols, HQ_E5M2, scale_in, ring, q, q_t, q_pre, q_t_pre, scale_out, amax_out,
                      workspace, workspace_bytes, true, seed, stream, "hq_quantize_fp8_layouts_stochastic");
}

hq_status hq_quantize_fp8_blockwise(const void* x, int xt, int64_t rows, int64_t cols, int fmt, int block_size,
                                    int stochastic, uint64_t seed, uint8_t* q, float* scales, float* amax_out,
                                    hipStream_t stream) {
  if (xt != HQ_F32 && xt != HQ_BF16) return fail(HQ_ERR_INVALID_ARGUMENT, "xt must be HQ_F32 or HQ_BF16, got %d", xt);
  if (!valid_fmt(fmt)) return fail(HQ_ERR_INVALID_ARGUMENT, "fmt must be HQ_E4M3 or HQ_E5M2, got %d", fmt);
  if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128)
    return fail(HQ_ERR_INVALID_ARGUMENT, "block_size must be 16, 32, 64 or 128, got %d", block_size);
  if (stochastic && fmt != HQ_E5M2) return fail(HQ_ERR_INVALID_ARGUMENT, "stochastic rounding produces E5M2");
  if (rows < 0 || rows > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31 - 1024], got %lld", (long long)rows);
  if (cols < 16 || cols > kMaxDim || cols % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "cols must be a positive multiple of 16, at most 2^31 - 1024, got %lld",
                (long long)cols);
  if ((double)rows * (double)cols > 1099511627776.0) return fail(HQ_ERR_INVALID_ARGUMENT, "rows * cols exceeds 2^40");
  if (rows == 0) return ok();
  if (!x || !q || !scales) return fail(HQ_ERR_INVALID_ARGUMENT, "x, q and scales must be non-NULL");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(HQ_ERR_INVALID_ARGUMENT, "x and q must be 16-byte aligned");
  if (!aligned(scales, 4) || (amax_out && !aligned(amax_out, 4)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "scales and amax_out must be 4-byte aligned");
  const size_t numel = (size_t)rows * (size_t)cols;
  const size_t nscale = (size_t)rows * (size_t)((cols + block_size - 1) / block_size);
  const Range rg[] = {
      {x, numel * (xt == HQ_BF16 ? 2 : 4), "x"},
      {q, numel, "q"},
      {scales, nscale * 4, "scales"},
      {amax_out, amax_out ? nscale * 4 : 0, "amax_out"},
  };
  const char* other = nullptr;
  if (const char* a = find_overlap(rg, 4, &other)) return fail(HQ_ERR_INVALID_ARGUMENT, "%s overlaps %s", a, other);
  hq_status st = check_device();
  if (st != HQ_OK) return st;
  (void)hipGetLastError();
  return launched(hq::launch_quant_blocks(x, xt, (int)rows, (int)cols, fmt, block_size, stochastic != 0, seed, q,
                                          scales, amax_out, stream),
                  "hq_quantize_fp8_blockwise");
}

hq_status hq_scale_ring_update(const hq_ring* ring, const float* amax, int fmt, hipStream_t stream) {
  if (!ring) return fail(HQ_ERR_INVALID_ARGUMENT, "ring is NULL");
  if (!valid_fmt(fmt)) return fail(HQ_ERR_INVALID_ARGUMENT, "fmt must be HQ_E4M3 or HQ_E5M2, got %d", fmt);
  hq_status st = check_ring(ring);
  if (st != HQ_OK) return st;
  if (!amax || !aligned(amax, 4)) return fail(HQ_ERR_INVALID_ARGUMENT, "amax must be a non-NULL, 4-byte aligned device float");
  const Range rg[] = {
      {ring->state, ((size_t)ring->len + 2) * 4, "ring->state"},
      {amax, 4, "amax"},
      {ring->nonfinite_flag, ring->nonfinite_flag ? 4u : 0u, "ring->nonfinite_flag"},
  };
  const char* other = nullptr;
  if (const char* a = find_overlap(rg, 3, &other)) return fail(HQ_ERR_INVALID_ARGUMENT, "%s overlaps %s", a, other);
  st = check_device();
  if (st != HQ_OK) return st;
  (void)hipGetLastError();
  return launched(hq::launch_ring_update(ring->state, ring->len, ring->idx, ring->margin, ring->nonfinite_flag, amax,
                                         fmt, stream),
                  "hq_scale_ring_update");
}

hq_status hq_quantize_fp8_preshuffled(const void* x, int xt, int64_t rows, int64_t cols, int fmt, uint8_t* q,
                                      uint8_t* q_pre, float* scale_out, float* amax_out, hipStream_t stream) {
  if (xt != HQ_F32 && xt != HQ_BF16) return fail(HQ_ERR_INVALID_ARGUMENT, "xt must be HQ_F32 or HQ_BF16, got %d", xt);
  if (!valid_fmt(fmt)) return fail(HQ_ERR_INVALID_ARGUMENT, "fmt must be HQ_E4M3 or HQ_E5M2, got %d", fmt);
  if (rows < 0 || rows > kMaxDim)
    return fail(HQ_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31 - 1024], got %lld", (long long)rows);
  if (cols < 16 || cols > kMaxDim || cols % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "cols must be a positive multiple of 16, at most 2^31 - 1024, got %lld",
                (long long)cols);
  if ((double)rows * (double)cols > 1099511627776.0) return fail(HQ_ERR_INVALID_ARGUMENT, "rows * cols exceeds 2^40");
  if (rows == 0) return ok();
  if (!x || !q_pre || !scale_out) return fail(HQ_ERR_INVALID_ARGUMENT, "x, q_pre and scale_out must be non-NULL");
  if (!aligned(x, 16) || !aligned(q_pre, 16) || (q && !aligned(q, 16)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "x, q and q_pre must be 16-byte aligned");
  if (!aligned(scale_out, 4) || (amax_out && !aligned(amax_out, 4)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "scale_out and amax_out must be 4-byte aligned");
  const size_t numel = (size_t)rows * (size_t)cols;
  const Range rg[] = {
      {x, numel * (xt == HQ_BF16 ? 2 : 4), "x"},
      {q, q ? numel : 0, "q"},
      {q_pre, (size_t)padded_bytes(rows, cols), "q_pre"},
      {scale_out, (size_t)rows * 4, "scale_out"},
      {amax_out, amax_out ? (size_t)rows * 4 : 0, "amax_out"},
  };
  const char* other = nullptr;
  if (const char* a = find_overlap(rg, 5, &other)) return fail(HQ_ERR_INVALID_ARGUMENT, "%s overlaps %s", a, other);
  hq_status st = check_device();
  if (st != HQ_OK) return st;
  (void)hipGetLastError();
  return launched(hq::launch_quant_rows_pre(x, xt, (int)rows, (int)cols, fmt, q, q_pre, scale_out, amax_out, stream),
                  "hq_quantize_fp8_preshuffled");
}

hq_status hq_preshuffle_weight(const uint8_t* wq, int64_t n, int64_t k, uint8_t* wq_pre, hipStream_t stream) {
  if (n < 0 || n > kMaxDim) return fail(HQ_ERR_INVALID_ARGUMENT, "n must be in [0, 2^31 - 1024], got %lld", (long long)n);
  if (k < 16 || k > kMaxDim || k % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "k must be a positive multiple of 16, at most 2^31 - 1024, got %lld",
                (long long)k);
  if ((double)padded_bytes(n, k) / 16.0 / 256.0 > (double)kI32Max) return fail(HQ_ERR_INVALID_ARGUMENT, "weight too large");
  if (n == 0) return ok();
  if (!wq || !wq_pre) return fail(HQ_ERR_INVALID_ARGUMENT, "wq and wq_pre must be non-NULL");
  if (!aligned(wq, 16) || !aligned(wq_pre, 16)) return fail(HQ_ERR_INVALID_ARGUMENT, "wq and wq_pre must be 16-byte aligned");
  const Range rg[] = {{wq, (size_t)n * (size_t)k, "wq"}, {wq_pre, (size_t)padded_bytes(n, k), "wq_pre"}};
  const char* other = nullptr;
  if (const char* a = find_overlap(rg, 2, &other)) return fail(HQ_ERR_INVALID_ARGUMENT, "%s overlaps %s", a, other);
  hq_status st = check_device();
  if (st != HQ_OK) return st;
  (void)hipGetLastError();
  return launched(hq::launch_preshuffle(wq, (int)n, (int)k, wq_pre, stream), "hq_preshuffle_weight");
}

hq_status hq_stream_rows_probe(const void* x, int64_t rows, int64_t row_bytes, int32_t waves, uint8_t* out,
                               hipStream_t stream) {
  if (rows < 0 || rows > kMaxDim) return fail(HQ_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31 - 1024], got %lld", (long long)rows);
  if (row_bytes < 16 || row_bytes > 8192 || row_bytes % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "row_bytes must be a multiple of 16 in [16, 8192], got %lld", (long long)row_bytes);
  if (waves < 1 || waves > (1 << 20)) return fail(HQ_ERR_INVALID_ARGUMENT, "waves must be in [1, 2^20], got %d", waves);
  if (rows == 0) return ok();
  if (!x || !out) return fail(HQ_ERR_INVALID_ARGUMENT, "x and out must be non-NULL");
  if (!aligned(x, 16) || !aligned(out, 8)) return fail(HQ_ERR_INVALID_ARGUMENT, "x must be 16-byte and out 8-byte aligned");
  const Range rg[] = {{x, (size_t)rows * (size_t)row_bytes, "x"}, {out, (size_t)rows * (size_t)row_bytes / 2, "out"}};
  const char* other = nullptr;
  if (const char* a = find_overlap(rg, 2, &other)) return fail(HQ_ERR_INVALID_ARGUMENT, "%s overlaps %s", a, other);
  hq_status st = check_device();
  if (st != HQ_OK) return st;
  (void)hipGetLastError();
  return launched(hq::launch_stream_rows_probe(x, rows, (int)(row_bytes / 16), waves, out, stream), "hq_stream_rows_probe");
}

// Epilogue arguments shared by the plain and grouped forms: bias kind, pointers
// and the validation of their combination. Returns HQ_OK and fills the outputs.
static hq_status epilogue_args(const hq_epilogue* ep, const void** bias, int* bias_kind, const float** bias_scale,
                               const float** out_scale, int* out_fmt) {
  *bias = ep ? ep->bias : nullptr;
  *bias_scale = ep ? ep->bias_scale : nullptr;
  *out_scale = ep ? ep->out_scale : nullptr;
  *bias_kind = hq::kBiasNone;
  *out_fmt = 0;
  if (*bias) {
    switch (ep->bias_type) {
      case HQ_BIAS_BF16: *bias_kind = hq::kBiasBF16; break;
      case HQ_BIAS_E4M3: *bias_kind = hq::kBiasE4M3; break;
      case HQ_BIAS_E5M2: *bias_kind = hq::kBiasE5M2; break;
      default: return fail(HQ_ERR_INVALID_ARGUMENT, "unknown bias_type %d", ep->bias_type);
    }
    if ((*bias_kind == hq::kBiasBF16) != (*bias_scale == nullptr))
      return fail(HQ_ERR_INVALID_ARGUMENT, "an FP8 bias requires bias_scale and a bf16 bias takes none");
  } else if (*bias_scale) {
    return fail(HQ_ERR_INVALID_ARGUMENT, "bias_scale given without a bias");
  }
  if (*out_scale) {
    if (!valid_fmt(ep->out_fmt)) return fail(HQ_ERR_INVALID_ARGUMENT, "out_fmt must be HQ_E4M3 or HQ_E5M2, got %d", ep->out_fmt);
    *out_fmt = ep->out_fmt;
  }
  return HQ_OK;
}

static hq_status check_gemm_common(int xf, int wf, int64_t m, int64_t n, int64_t k) {
  if (!valid_fmt(xf) || !valid_fmt(wf)) return fail(HQ_ERR_INVALID_ARGUMENT, "xf and wf must be HQ_E4M3 or HQ_E5M2");
  if (m < 0 || m > kMaxDim) return fail(HQ_ERR_INVALID_ARGUMENT, "m must be in [0, 2^31 - 1024], got %lld", (long long)m);
  if (n < 0 || n > kMaxDim) return fail(HQ_ERR_INVALID_ARGUMENT, "n must be in [0, 2^31 - 1024], got %lld", (long long)n);
  if (k < 16 || k >= (1 << 24) || k % 16 != 0)
    return fail(HQ_ERR_INVALID_ARGUMENT, "k must be a positive multiple of 16 below 2^24, got %lld", (long long)k);
  if ((double)((m + 127) / 128) * (double)((n + 127) / 128) > 1.0e9)
    return fail(HQ_ERR_INVALID_ARGUMENT, "output too large for one launch");
  return HQ_OK;
}

int64_t hq_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k < 16 || k % 16 != 0 || k >= (int64_t(1) << 24) || m > kMaxDim || n > kMaxDim) return -1;
  if (m == 0 || n == 0) return 0;
  return (int64_t)hq::gemm_workspace_bytes((int)m, (int)n, (int)k);
}

hq_status hq_gemm_a8w8(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf, const float* x_scale,
                       int64_t x_scale_count, const float* w_scale, int64_t w_scale_count, int64_t m, int64_t n,
                       int64_t k, uint16_t* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return hq_gemm_a8w8_epilogue(xq, xf, wq_pre, wf, x_scale, x_scale_count, w_scale, w_scale_count, m, n, k, nullptr,
                               out, workspace, workspace_bytes, stream);
}

// library_scratch: take the split workspace from the library's device array
// (hq_gemm_a8w8_noalloc) instead of `workspace`, which is then NULL / 0.
static hq_status gemm_impl(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf, const float* x_scale,
                           int64_t x_scale_count, const float* w_scale, int64_t w_scale_count, int64_t m, int64_t n,
                           int64_t k, const hq_epilogue* ep, void* out, void* workspace, size_t workspace_bytes,
                           bool strict, const char* name, hipStream_t stream, bool library_scratch = false) {
  hq_status st = check_gemm_common(xf, wf, m, n, k);
  if (st != HQ_OK) return st;
  if (workspace_bytes > 0 && workspace == nullptr)
    return fail(HQ_ERR_INVALID_ARGUMENT, "workspace is NULL but workspace_bytes is %zu", workspace_bytes);
  if (workspace_bytes > 0 && !aligned(workspace, 16))
    return fail(HQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (x_scale_count != 1 && x_scale_count != m)
    return fail(HQ_ERR_INVALID_ARGUMENT, "x_scale_count must be 1 or m (%lld), got %lld", (long long)m, (long long)x_scale_count);
  if (w_scale_count != 1 && w_scale_count != n)
    return fail(HQ_ERR_INVALID_ARGUMENT, "w_scale_count must be 1 or n (%lld), got %lld", (long long)n, (long long)w_scale_count);
  const void* bias;
  int bias_kind, out_fmt;
  const float *bias_scale, *out_scale;
  st = epilogue_args(ep, &bias, &bias_kind, &bias_scale, &out_scale, &out_fmt);
  if (st != HQ_OK) return st;
  if (m == 0 || n == 0) return ok();
  if (!xq || !wq_pre || !x_scale || !w_scale || !out)
    return fail(HQ_ERR_INVALID_ARGUMENT, "xq, wq_pre, x_scale, w_scale and out must be non-NULL");
  if (!aligned(xq, 16) || !aligned(wq_pre, 16)) return fail(HQ_ERR_INVALID_ARGUMENT, "xq and wq_pre must be 16-byte aligned");
  if (!aligned(out, 16)) return fail(HQ_ERR_INVALID_ARGUMENT, "out must be 16-byte aligned");
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || (bias_scale && !aligned(bias_scale, 4)) ||
      (out_scale && !aligned(out_scale, 4)) || (bias_kind == hq::kBiasBF16 && !aligned(bias, 2)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "scales must be 4-byte aligned and a bf16 bias 2-byte aligned");
  const size_t ws_used = workspace_bytes > 0 ? workspace_bytes : 0;
  const Range rg[] = {
      {out, (size_t)m * (size_t)n * (out_scale ? 1 : 2), "out"},
      {workspace, ws_used, "workspace"},
      {xq, (size_t)m * (size_t)k, "xq"},
      {wq_pre, (size_t)padded_bytes(n, k), "wq_pre"},
      {x_scale, (size_t)x_scale_count * 4, "x_scale"},
      {w_scale, (size_t)w_scale_count * 4, "w_scale"},
      {bias, bias ? (size_t)n * (bias_kind == hq::kBiasBF16 ? 2 : 1) : 0, "bias"},
      {bias_scale, bias_scale ? 4u : 0u, "bias_scale"},
      {out_scale, out_scale ? 4u : 0u, "out_scale"},
  };
  const char* other = nullptr;
  const char* a = find_overlap(rg, 9, &other);
  if (a && (strcmp(a, "out") == 0 || strcmp(a, "workspace") == 0))
    return fail(HQ_ERR_INVALID_ARGUMENT, "%s overlaps %s", a, other);
  size_t scratch_need = 0;
  if (library_scratch) {
    scratch_need = hq::gemm_workspace_bytes((int)m, (int)n, (int)k);
    if (scratch_need > hq::kNoAllocScratchBytes)
      return fail(HQ_ERR_INVALID_ARGUMENT, "%s: m=%lld n=%lld k=%lld needs %zu bytes of scratch, more than the %zu the "
                  "library holds", name, (long long)m, (long long)n, (long long)k, scratch_need,
                  hq::kNoAllocScratchBytes);
  }
  st = check_device();
  if (st != HQ_OK) return st;
  hq::GemmArgs g{xq, wq_pre, x_scale, w_scale, out, (int)m, (int)n, (int)k, x_scale_count != 1, w_scale_count != 1,
                 bias, bias_kind, bias_scale, out_scale, out_fmt};
  g.strict = strict;
  (void)hipGetLastError();
  if (library_scratch) {
    void* scratch = nullptr;
    if (scratch_need > 0) {
      const hipError_t e = hq::noalloc_scratch(stream, &scratch);
      if (e != hipSuccess) return fail(HQ_ERR_LAUNCH, "%s: library scratch: %s", name, hipGetErrorString(e));
    }
    return launched(hq::launch_gemm(g, xf, wf, scratch, scratch_need, stream), name);
  }
  return launched(hq::launch_gemm(g, xf, wf, ws_used ? workspace : nullptr, ws_used, stream), name);
}

hq_status hq_quantize_workspace_status(const void* workspace, size_t workspace_bytes, int32_t* gave_up,
                                       hipStream_t stream) {
  if (!gave_up) return fail(HQ_ERR_INVALID_ARGUMENT, "gave_up must be non-NULL");
  if (!workspace) return fail(HQ_ERR_INVALID_ARGUMENT, "workspace must be non-NULL");
  if (workspace_bytes < hq::kTensorWorkspaceBytes)
    return fail(HQ_ERR_INVALID_ARGUMENT, "workspace_bytes %zu is less than the %zu of a quantize workspace",
                workspace_bytes, hq::kTensorWorkspaceBytes);
  if (!aligned(workspace, 16)) return fail(HQ_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  hq_status st = check_device();
  if (st != HQ_OK) return st;
  uint32_t word = 0;
  const uint8_t* src = static_cast<const uint8_t*>(workspace) + (hq::kBarrierOffsetWords + hq::kBarStatus) * 4;
  hipError_t e = hipMemcpyAsync(&word, src, 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(HQ_ERR_LAUNCH, "hq_quantize_workspace_status: %s", hipGetErrorString(e));
  *gave_up = (word & hq::kGaveUpBit) ? 1 : 0;
  return ok();
}

hq_status hq_gemm_a8w8_noalloc(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf, const float* x_scale,
                               int64_t x_scale_count, const float* w_scale, int64_t w_scale_count, int64_t m,
                               int64_t n, int64_t k, uint16_t* out, hipStream_t stream) {
  return gemm_impl(xq, xf, wq_pre, wf, x_scale, x_scale_count, w_scale, w_scale_count, m, n, k, nullptr, out, nullptr,
                   0, false, "hq_gemm_a8w8_noalloc", stream, true);
}

hq_status hq_gemm_a8w8_epilogue(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf, const float* x_scale,
                                int64_t x_scale_count, const float* w_scale, int64_t w_scale_count, int64_t m,
                                int64_t n, int64_t k, const hq_epilogue* ep, void* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return gemm_impl(xq, xf, wq_pre, wf, x_scale, x_scale_count, w_scale, w_scale_count, m, n, k, ep, out, workspace,
                   workspace_bytes, false, ep ? "hq_gemm_a8w8_epilogue" : "hq_gemm_a8w8", stream);
}

hq_status hq_gemm_a8w8_strict(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf, const float* x_scale,
                              int64_t x_scale_count, const float* w_scale, int64_t w_scale_count, int64_t m, int64_t n,
                              int64_t k, const hq_epilogue* ep, void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return gemm_impl(xq, xf, wq_pre, wf, x_scale, x_scale_count, w_scale, w_scale_count, m, n, k, ep, out, workspace,
                   workspace_bytes, true, "hq_gemm_a8w8_strict", stream);
}

hq_status hq_grouped_gemm_a8w8(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf, const float* x_scale,
                               int64_t x_scale_count, const float* w_scale, int64_t w_scale_count,
                               const int32_t* group_offsets, int32_t num_experts, int64_t total_rows, int64_t n,
                               int64_t k, uint16_t* out, hipStream_t stream) {
  return hq_grouped_gemm_a8w8_epilogue(xq, xf, wq_pre, wf, x_scale, x_scale_count, w_scale, w_scale_count,
                                       group_offsets, num_experts, total_rows, n, k, nullptr, out, stream);
}

static hq_status grouped_impl(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf, const float* x_scale,
                              int64_t x_scale_count, const float* w_scale, int64_t w_scale_count,
                              const int32_t* group_offsets, int32_t num_experts, int64_t total_rows, int64_t n,
                              int64_t k, const hq_epilogue* ep, void* out, bool strict, const char* name,
                              hipStream_t stream) {
  hq_status st = check_gemm_common(xf, wf, total_rows, n, k);
  if (st != HQ_OK) return st;
  if (num_experts < 1 || num_experts > 1024)
    return fail(HQ_ERR_INVALID_ARGUMENT, "num_experts must be in [1, 1024], got %d", num_experts);
  if (x_scale_count != 1 && x_scale_count != total_rows)
    return fail(HQ_ERR_INVALID_ARGUMENT, "x_scale_count must be 1 or total_rows (%lld), got %lld", (long long)total_rows,
                (long long)x_scale_count);
  if (w_scale_count != num_experts && w_scale_count != (int64_t)num_experts * n)
    return fail(HQ_ERR_INVALID_ARGUMENT, "w_scale_count must be num_experts or num_experts * n, got %lld",
                (long long)w_scale_count);
  if ((double)((total_rows + 127) / 128 + num_experts) * (double)((n + 127) / 128) > 1.0e9)
    return fail(HQ_ERR_INVALID_ARGUMENT, "output too large for one launch");
  const void* bias;
  int bias_kind, out_fmt;
  const float *bias_scale, *out_scale;
  st = epilogue_args(ep, &bias, &bias_kind, &bias_scale, &out_scale, &out_fmt);
  if (st != HQ_OK) return st;
  if (total_rows == 0 || n == 0) return ok();
  if (!xq || !wq_pre || !x_scale || !w_scale || !group_offsets || !out)
    return fail(HQ_ERR_INVALID_ARGUMENT, "xq, wq_pre, x_scale, w_scale, group_offsets and out must be non-NULL");
  if (!aligned(xq, 16) || !aligned(wq_pre, 16) || !aligned(out, 16))
    return fail(HQ_ERR_INVALID_ARGUMENT, "xq, wq_pre and out must be 16-byte aligned");
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(group_offsets, 4) ||
      (bias_scale && !aligned(bias_scale, 4)) || (out_scale && !aligned(out_scale, 4)) ||
      (bias_kind == hq::kBiasBF16 && !aligned(bias, 2)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "scales and group_offsets must be 4-byte aligned and a bf16 bias 2-byte aligned");
  const size_t bias_bytes = bias ? (size_t)num_experts * (size_t)n * (bias_kind == hq::kBiasBF16 ? 2 : 1) : 0;
  const Range rg[] = {
      {out, (size_t)total_rows * (size_t)n * (out_scale ? 1 : 2), "out"},
      {xq, (size_t)total_rows * (size_t)k, "xq"},
      {wq_pre, (size_t)padded_bytes(n, k) * (size_t)num_experts, "wq_pre"},
      {x_scale, (size_t)x_scale_count * 4, "x_scale"},
      {w_scale, (size_t)w_scale_count * 4, "w_scale"},
      {group_offsets, ((size_t)num_experts + 1) * 4, "group_offsets"},
      {bias, bias_bytes, "bias"},
      {bias_scale, bias_scale ? (size_t)num_experts * 4 : 0, "bias_scale"},
      {out_scale, out_scale ? 4u : 0u, "out_scale"},
  };
  const char* other = nullptr;
  const char* a = find_overlap(rg, 9, &other);
  if (a && strcmp(a, "out") == 0) return fail(HQ_ERR_INVALID_ARGUMENT, "out overlaps %s", other);
  st = check_device();
  if (st != HQ_OK) return st;
  hq::GemmArgs g{xq, wq_pre, x_scale, w_scale, out, (int)total_rows, (int)n, (int)k, x_scale_count != 1,
                 w_scale_count != num_experts, bias, bias_kind, bias_scale, out_scale, out_fmt};
  g.strict = strict;
  (void)hipGetLastError();
  return launched(hq::launch_grouped_gemm(g, group_offsets, num_experts, xf, wf, stream), name);
}

hq_status hq_grouped_gemm_a8w8_epilogue(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf,
                                        const float* x_scale, int64_t x_scale_count, const float* w_scale,
                                        int64_t w_scale_count, const int32_t* group_offsets, int32_t num_experts,
                                        int64_t total_rows, int64_t n, int64_t k, const hq_epilogue* ep, void* out,
                                        hipStream_t stream) {
  return grouped_impl(xq, xf, wq_pre, wf, x_scale, x_scale_count, w_scale, w_scale_count, group_offsets, num_experts,
                      total_rows, n, k, ep, out, false,
                      ep ? "hq_grouped_gemm_a8w8_epilogue" : "hq_grouped_gemm_a8w8", stream);
}

hq_status hq_grouped_gemm_a8w8_strict(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf,
                                      const float* x_scale, int64_t x_scale_count, const float* w_scale,
                                      int64_t w_scale_count, const int32_t* group_offsets, int32_t num_experts,
                                      int64_t total_rows, int64_t n, int64_t k, const hq_epilogue* ep, void* out,
                                      hipStream_t stream) {
  return grouped_impl(xq, xf, wq_pre, wf, x_scale, x_scale_count, w_scale, w_scale_count, group_offsets, num_experts,
                      total_rows, n, k, ep, out, true, "hq_grouped_gemm_a8w8_strict", stream);
}

hq_status hq_gemm_a8w8_blockscaled(const uint8_t* xq, int xf, const uint8_t* wq, int wf, const float* x_scales,
                                   const float* w_scales, int block_size, int64_t m, int64_t n, int64_t k,
                                   const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  hq_status st = check_gemm_common(xf, wf, m, n, k);
  if (st != HQ_OK) return st;
  if (block_size != 32 && block_size != 64 && block_size != 128)
    return fail(HQ_ERR_INVALID_ARGUMENT, "block_size must be 32, 64 or 128, got %d", block_size);
  if (m == 0 || n == 0) return ok();
  if (!xq || !wq || !x_scales || !w_scales || !out)
    return fail(HQ_ERR_INVALID_ARGUMENT, "xq, wq, x_scales, w_scales and out must be non-NULL");
  if (!aligned(xq, 16) || !aligned(wq, 16)) return fail(HQ_ERR_INVALID_ARGUMENT, "xq and wq must be 16-byte aligned");
  if (!aligned(out, 2) || !aligned(x_scales, 4) || !aligned(w_scales, 4) || (bias && !aligned(bias, 2)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "out and bias must be 2-byte and the scales 4-byte aligned");
  const int64_t nb = (k + block_size - 1) / block_size;
  const Range rg[] = {
      {out, (size_t)m * (size_t)n * 2, "out"},
      {xq, (size_t)m * (size_t)k, "xq"},
      {wq, (size_t)n * (size_t)k, "wq"},
      {x_scales, (size_t)m * (size_t)nb * 4, "x_scales"},
      {w_scales, (size_t)n * (size_t)nb * 4, "w_scales"},
      {bias, bias ? (size_t)n * 2 : 0, "bias"},
  };
  const char* other = nullptr;
  const char* a = find_overlap(rg, 6, &other);
  if (a && strcmp(a, "out") == 0) return fail(HQ_ERR_INVALID_ARGUMENT, "out overlaps %s", other);
  st = check_device();
  if (st != HQ_OK) return st;
  hq::BlockGemmArgs g{xq, wq, x_scales, w_scales, bias, out, (int)m, (int)n, (int)k, (int)nb};
  (void)hipGetLastError();
  return launched(hq::launch_gemm_blockscaled(g, xf, wf, block_size, stream), "hq_gemm_a8w8_blockscaled");
}

hq_status hq_gemm_a8w8_blockscaled_preshuffled(const uint8_t* xq, int xf, const uint8_t* wq_pre, int wf,
                                               const float* x_scales, const float* w_scales, int block_size,
                                               int64_t m, int64_t n, int64_t k, const uint16_t* bias, uint16_t* out,
                                               hipStream_t stream) {
  hq_status st = check_gemm_common(xf, wf, m, n, k);
  if (st != HQ_OK) return st;
  if (block_size != 32 && block_size != 64 && block_size != 128)
    return fail(HQ_ERR_INVALID_ARGUMENT, "block_size must be 32, 64 or 128, got %d", block_size);
  if (m == 0 || n == 0) return ok();
  if (!xq || !wq_pre || !x_scales || !w_scales || !out)
    return fail(HQ_ERR_INVALID_ARGUMENT, "xq, wq_pre, x_scales, w_scales and out must be non-NULL");
  if (!aligned(xq, 16) || !aligned(wq_pre, 16) || !aligned(out, 16))
    return fail(HQ_ERR_INVALID_ARGUMENT, "xq, wq_pre and out must be 16-byte aligned");
  if (!aligned(x_scales, 4) || !aligned(w_scales, 4) || (bias && !aligned(bias, 2)))
    return fail(HQ_ERR_INVALID_ARGUMENT, "the scales must be 4-byte and bias 2-byte aligned");
  const int64_t nb = (k + block_size - 1) / block_size;
  const Range rg[] = {
      {out, (size_t)m * (size_t)n * 2, "out"},
      {xq, (size_t)m * (size_t)k, "xq"},
      {wq_pre, (size_t)padded_bytes(n, k), "wq_pre"},
      {x_scales, (size_t)m * (size_t)nb * 4, "x_scales"},
      {w_scales, (size_t)n * (size_t)nb * 4, "w_scales"},
      {bias, bias ? (size_t)n * 2 : 0, "bias"},
  };
  const char* other = nullptr;
  const char* a = find_overlap(rg, 6, &other);
  if (a && strcmp(a, "out") == 0) return fail(HQ_ERR_INVALID_ARGUMENT, "out overlaps %s", other);
  st = check_device();
  if (st != HQ_OK) return st;
  hq::GemmArgs g{xq, wq_pre, x_scales, w_scales, out, (int)m, (int)n, (int)k, 1, 1,
                 bias, bias ? hq::kBiasBF16 : hq::kBiasNone, nullptr, nullptr, 0, (int)nb};
  (void)hipGetLastError();
  return launched(hq::launch_gemm_bsf(g, xf, wf, block_size, stream), "hq_gemm_a8w8_blockscaled_preshuffled");
}

}  // extern "C"
