"""ctypes loader for libhq.so: declares every exported C symbol of include/hq.h.

The library must have been built (``python -m fp8_dynamic_quantization_amd.build``);
loading fails loudly otherwise. There is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhq.so")

HQ_OK = 0
HQ_ERR_INVALID_ARGUMENT = 1
HQ_ERR_UNSUPPORTED_DEVICE = 2
HQ_ERR_LAUNCH = 3

HQ_E4M3 = 0
HQ_E5M2 = 1
HQ_F32 = 0
HQ_BF16 = 1
HQ_PER_TENSOR = 0
HQ_PER_TOKEN = 1
HQ_PER_CHANNEL = 2
HQ_BIAS_BF16 = 0
HQ_BIAS_E4M3 = 1
HQ_BIAS_E5M2 = 2


class hq_ring(ctypes.Structure):
    _fields_ = [
        ("state", ctypes.c_void_p),
        ("len", ctypes.c_int32),
        ("idx", ctypes.c_int32),
        ("margin", ctypes.c_int32),
        ("nonfinite_flag", ctypes.c_void_p),
    ]


class hq_epilogue(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("bias_type", ctypes.c_int32), ("bias_scale", ctypes.c_void_p),
                ("out_scale", ctypes.c_void_p), ("out_fmt", ctypes.c_int32)]


class HQError(RuntimeError):
    """A non-OK status from libhq. ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[hq status {status}] {message}")
        self.status = status


class HQInvalidArgument(HQError, ValueError):
    pass


class HQUnsupportedDevice(HQError, NotImplementedError):
    pass


class HQLaunchError(HQError):
    pass


_P = ctypes.c_void_p
_I = ctypes.c_int
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); the complete export list of include/hq.h
SIGNATURES = {
    "hq_scale_count": (_I64, [_I, _I64, _I64]),
    "hq_quantize_workspace_bytes": (_SZ, [_I, _I64, _I64]),
    "hq_quantize_fp8": (_I, [_P, _I, _I64, _I64, _I, _I, _P, _P, _P, ctypes.POINTER(hq_ring), _P, _SZ, _P]),
    "hq_quantize_fp8_stochastic": (_I, [_P, _I, _I64, _I64, _I, ctypes.c_uint64, _P, _P, _P,
                                        ctypes.POINTER(hq_ring), _P, _SZ, _P]),
    "hq_quantize_fp8_blockwise": (_I, [_P, _I, _I64, _I64, _I, _I, _I, ctypes.c_uint64, _P, _P, _P, _P]),
    "hq_gemm_a8w8_blockscaled": (_I, [_P, _I, _P, _I, _P, _P, _I, _I64, _I64, _I64, _P, _P, _P]),
    "hq_gemm_a8w8_blockscaled_preshuffled": (_I, [_P, _I, _P, _I, _P, _P, _I, _I64, _I64, _I64, _P, _P, _P]),
    "hq_quantize_fp8_layouts": (_I, [_P, _I, _I64, _I64, _I, _P, ctypes.POINTER(hq_ring), _P, _P, _P, _P, _P, _P,
                                     _P, _SZ, _P]),
    "hq_quantize_fp8_layouts_stochastic": (_I, [_P, _I, _I64, _I64, ctypes.c_uint64, _P, ctypes.POINTER(hq_ring), _P,
                                                _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "hq_scale_ring_update": (_I, [ctypes.POINTER(hq_ring), _P, _I, _P]),
    "hq_preshuffled_bytes": (_I64, [_I64, _I64]),
    "hq_preshuffle_weight": (_I, [_P, _I64, _I64, _P, _P]),
    "hq_quantize_fp8_preshuffled": (_I, [_P, _I, _I64, _I64, _I, _P, _P, _P, _P, _P]),
    "hq_gemm_workspace_bytes": (_I64, [_I64, _I64, _I64]),
    "hq_gemm_a8w8": (_I, [_P, _I, _P, _I, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "hq_gemm_a8w8_epilogue": (_I, [_P, _I, _P, _I, _P, _I64, _P, _I64, _I64, _I64, _I64, ctypes.POINTER(hq_epilogue),
                                   _P, _P, _SZ, _P]),
    "hq_grouped_gemm_a8w8": (_I, [_P, _I, _P, _I, _P, _I64, _P, _I64, _P, _I32, _I64, _I64, _I64, _P, _P]),
    "hq_grouped_gemm_a8w8_epilogue": (_I, [_P, _I, _P, _I, _P, _I64, _P, _I64, _P, _I32, _I64, _I64, _I64,
                                           ctypes.POINTER(hq_epilogue), _P, _P]),
    "hq_quantize_workspace_status": (_I, [_P, _SZ, ctypes.POINTER(_I32), _P]),
    "hq_gemm_a8w8_noalloc": (_I, [_P, _I, _P, _I, _P, _I64, _P, _I64, _I64, _I64, _I64, _P, _P]),
    "hq_gemm_a8w8_strict": (_I, [_P, _I, _P, _I, _P, _I64, _P, _I64, _I64, _I64, _I64, ctypes.POINTER(hq_epilogue),
                                 _P, _P, _SZ, _P]),
    "hq_grouped_gemm_a8w8_strict": (_I, [_P, _I, _P, _I, _P, _I64, _P, _I64, _P, _I32, _I64, _I64, _I64,
                                         ctypes.POINTER(hq_epilogue), _P, _P]),
    "hq_stream_rows_probe": (_I, [_P, _I64, _I64, _I32, _P, _P]),
    "hq_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libhq.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libhq.so not found at {LIB_PATH}; build it with "
            "`python -m fp8_dynamic_quantization_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int) -> None:
    if status == HQ_OK:
        return
    msg = load().hq_last_error().decode(errors="replace")
    if status == HQ_ERR_INVALID_ARGUMENT:
        raise HQInvalidArgument(status, msg)
    if status == HQ_ERR_UNSUPPORTED_DEVICE:
        raise HQUnsupportedDevice(status, msg)
    if status == HQ_ERR_LAUNCH:
        raise HQLaunchError(status, msg)
    raise HQError(status, msg)
