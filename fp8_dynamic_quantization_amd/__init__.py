"""MI355X (gfx950) dynamic FP8 quantization and scaled FP8 (a8w8) GEMM.

The computation lives in libhq.so (HIP kernels behind the C ABI of
include/hq.h); this package is its thin Python binding.
"""
from ._lib import (HQ_BF16, HQ_BIAS_BF16, HQ_BIAS_E4M3, HQ_BIAS_E5M2, HQ_E4M3, HQ_E5M2, HQ_ERR_INVALID_ARGUMENT, HQ_ERR_LAUNCH,
                   HQ_ERR_UNSUPPORTED_DEVICE, HQ_F32, HQ_OK, HQ_PER_CHANNEL, HQ_PER_TENSOR,
                   HQ_PER_TOKEN, HQError, HQInvalidArgument, HQLaunchError,
                   HQUnsupportedDevice, LIB_PATH, SIGNATURES, hq_epilogue, hq_ring, load)
from .api import (Ring, gemm_workspace, hq_gemm_a8w8, hq_gemm_a8w8_blockscaled, hq_gemm_a8w8_epilogue,
                  hq_gemm_a8w8_blockscaled_preshuffled,
                  hq_gemm_workspace_bytes, hq_quantize_fp8_blockwise, hq_grouped_gemm_a8w8,
                  hq_grouped_gemm_a8w8_epilogue, hq_quantize_fp8_preshuffled, hq_gemm_a8w8_strict,
                  hq_grouped_gemm_a8w8_strict, hq_gemm_a8w8_noalloc,
                  hq_quantize_workspace_status, hq_stream_rows_probe,
                  hq_last_error, hq_preshuffle_weight, hq_preshuffled_bytes, hq_quantize_fp8,
                  hq_quantize_fp8_layouts, hq_quantize_fp8_layouts_stochastic, hq_quantize_fp8_stochastic,
                  hq_quantize_workspace_bytes, hq_scale_count,
                  hq_scale_ring_update)

__all__ = [
    "HQ_OK", "HQ_ERR_INVALID_ARGUMENT", "HQ_ERR_UNSUPPORTED_DEVICE", "HQ_ERR_LAUNCH",
    "HQ_E4M3", "HQ_E5M2", "HQ_F32", "HQ_BF16", "HQ_PER_TENSOR", "HQ_PER_TOKEN",
    "HQ_PER_CHANNEL", "HQError", "HQInvalidArgument", "HQUnsupportedDevice", "HQLaunchError",
    "LIB_PATH", "SIGNATURES", "hq_ring", "load", "Ring", "hq_scale_count",
    "hq_quantize_workspace_bytes", "hq_preshuffled_bytes", "hq_quantize_fp8", "hq_quantize_fp8_layouts", "hq_quantize_fp8_layouts_stochastic", "hq_quantize_fp8_stochastic", "hq_quantize_fp8_blockwise", "hq_gemm_a8w8_blockscaled", "hq_gemm_a8w8_blockscaled_preshuffled",
    "hq_scale_ring_update", "hq_preshuffle_weight", "hq_gemm_workspace_bytes", "hq_gemm_a8w8",
    "hq_gemm_a8w8_epilogue", "hq_epilogue", "HQ_BIAS_BF16", "HQ_BIAS_E4M3", "HQ_BIAS_E5M2",
    "hq_grouped_gemm_a8w8", "hq_grouped_gemm_a8w8_epilogue", "hq_quantize_fp8_preshuffled", "hq_last_error", "gemm_workspace",
    "hq_gemm_a8w8_strict", "hq_grouped_gemm_a8w8_strict", "hq_gemm_a8w8_noalloc", "hq_quantize_workspace_status",
    "hq_stream_rows_probe",
]
