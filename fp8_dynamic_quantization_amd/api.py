"""Thin torch-facing binding of libhq: the same entry points as include/hq.h.

Each function only marshals arguments (tensor -> pointer, current HIP stream,
optional output allocation with ``torch.empty``) and calls the C ABI; every
step of the computation runs in the library's HIP kernels. With ``stream=``
every buffer the binding allocates (outputs, zero-filled workspaces) is made
and filled on that stream, so the launch is ordered after it. Errors come back as
``HQInvalidArgument`` (ValueError), ``HQUnsupportedDevice``
(NotImplementedError) or ``HQLaunchError``.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools

import torch

from ._lib import (HQ_BF16, HQ_BIAS_BF16, HQ_E4M3, HQ_E5M2, HQ_F32, HQ_PER_CHANNEL, HQ_PER_TENSOR,
                   HQ_PER_TOKEN, check, hq_epilogue, hq_ring, load)

__all__ = [
    "Ring", "hq_scale_count", "hq_quantize_workspace_bytes", "hq_preshuffled_bytes",
    "hq_quantize_fp8", "hq_quantize_fp8_layouts", "hq_quantize_fp8_layouts_stochastic", "hq_quantize_fp8_stochastic",
    "hq_quantize_fp8_blockwise",
    "hq_gemm_a8w8_blockscaled", "hq_gemm_a8w8_blockscaled_preshuffled", "hq_scale_ring_update", "hq_preshuffle_weight", "hq_gemm_a8w8",
    "hq_gemm_a8w8_epilogue",
    "hq_grouped_gemm_a8w8", "hq_grouped_gemm_a8w8_epilogue", "hq_quantize_fp8_preshuffled", "hq_last_error",
    "hq_gemm_a8w8_strict", "hq_grouped_gemm_a8w8_strict", "hq_gemm_a8w8_noalloc",
    "hq_quantize_workspace_status", "hq_stream_rows_probe",
]

_XT = {torch.float32: HQ_F32, torch.bfloat16: HQ_BF16}


def _on_stream(fn):
    """Run `fn` with its `stream=` argument (if any) as torch's current stream,
    so the binding's allocations and fills are ordered before the launch."""
    @functools.wraps(fn)
    def wrapped(*args, stream=None, **kwargs):
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, stream=stream, **kwargs)
    return wrapped


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device, stream=None):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def hq_last_error() -> str:
    return load().hq_last_error().decode(errors="replace")


def hq_scale_count(gran: int, rows: int, cols: int) -> int:
    return int(load().hq_scale_count(gran, rows, cols))


def hq_quantize_workspace_bytes(gran: int, rows: int, cols: int) -> int:
    return int(load().hq_quantize_workspace_bytes(gran, rows, cols))


def hq_preshuffled_bytes(n: int, k: int) -> int:
    return int(load().hq_preshuffled_bytes(n, k))


def hq_gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(load().hq_gemm_workspace_bytes(m, n, k))


class Ring:
    """Device state of a delayed-scaling amax-history ring.

    ``state`` is float32 [length + 2] = [hist | scale | counter], initialised to
    hist = 0, scale = 1, counter = 0; ``flag`` is the sticky int32 non-finite flag.
    """

    def __init__(self, length: int = 16, margin: int = 0, device="cuda"):
        self.length = int(length)
        self.margin = int(margin)
        self.state = torch.zeros(self.length + 2, dtype=torch.float32, device=device)
        self.state[self.length] = 1.0
        self.flag = torch.zeros(1, dtype=torch.int32, device=device)

    def c_struct(self, idx: int) -> hq_ring:
        return hq_ring(self.state.data_ptr(), self.length, int(idx), self.margin, self.flag.data_ptr())


@_on_stream
def hq_quantize_fp8(x: torch.Tensor, fmt: int = HQ_E4M3, gran: int = HQ_PER_TOKEN, *,
                    ring: Ring | None = None, ring_idx: int = 0, q=None, scale_out=None,
                    amax_out=None, workspace=None, stream=None):
    """Quantize a 2-D bf16/fp32 tensor; returns (q uint8, scale_out fp32, amax_out fp32)."""
    if x.dtype not in _XT:
        raise ValueError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    x = x.contiguous()
    rows, cols = x.shape
    lib = load()
    count = max(int(lib.hq_scale_count(gran, rows, cols)), 0)
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scale_out is None:
        scale_out = torch.empty(count, dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.empty(count, dtype=torch.float32, device=dev)
    need = int(lib.hq_quantize_workspace_bytes(gran, rows, cols))
    if workspace is None and need > 0:
        # zero-filled: delayed scaling keeps arrival counters there
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ring_c = ctypes.byref(ring.c_struct(ring_idx)) if ring is not None else None
    st = lib.hq_quantize_fp8(_ptr(x), _XT[x.dtype], rows, cols, fmt, gran, _ptr(q), _ptr(scale_out),
                             _ptr(amax_out), ring_c, _ptr(workspace), ws_bytes, _stream(dev, stream))
    check(st)
    return q, scale_out, amax_out


@_on_stream
def hq_quantize_fp8_stochastic(x: torch.Tensor, gran: int = HQ_PER_TOKEN, seed: int = 0, *,
                               ring: Ring | None = None, ring_idx: int = 0, q=None, scale_out=None,
                               amax_out=None, workspace=None, stream=None):
    """E5M2 quantization with stochastic rounding (reproducible for a seed);
    returns (q uint8, scale_out fp32, amax_out fp32) like hq_quantize_fp8."""
    if x.dtype not in _XT:
        raise ValueError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    x = x.contiguous()
    rows, cols = x.shape
    lib = load()
    count = max(int(lib.hq_scale_count(gran, rows, cols)), 0)
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scale_out is None:
        scale_out = torch.empty(count, dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.empty(count, dtype=torch.float32, device=dev)
    need = int(lib.hq_quantize_workspace_bytes(gran, rows, cols))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ring_c = ctypes.byref(ring.c_struct(ring_idx)) if ring is not None else None
    st = lib.hq_quantize_fp8_stochastic(_ptr(x), _XT[x.dtype], rows, cols, gran, int(seed) & (2 ** 64 - 1), _ptr(q),
                                        _ptr(scale_out), _ptr(amax_out), ring_c, _ptr(workspace), ws_bytes,
                                        _stream(dev, stream))
    check(st)
    return q, scale_out, amax_out


@_on_stream
def hq_quantize_fp8_blockwise(x: torch.Tensor, fmt: int = HQ_E4M3, block_size: int = 32, *, stochastic: bool = False,
                              seed: int = 0, q=None, scales=None, amax_out=None, stream=None):
    """Block-wise quantization: returns (q uint8 [rows, cols], scales fp32
    [rows, ceil(cols / block_size)], amax fp32 of the same shape)."""
    if x.dtype not in _XT:
        raise ValueError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    x = x.contiguous()
    rows, cols = x.shape
    nb = -(-cols // int(block_size))
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows, nb), dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.empty((rows, nb), dtype=torch.float32, device=dev)
    check(load().hq_quantize_fp8_blockwise(_ptr(x), _XT[x.dtype], rows, cols, fmt, int(block_size), int(bool(stochastic)),
                                           int(seed) & (2 ** 64 - 1), _ptr(q), _ptr(scales), _ptr(amax_out),
                                           _stream(dev, stream)))
    return q, scales, amax_out


@_on_stream
def hq_gemm_a8w8_blockscaled(xq: torch.Tensor, xf: int, wq: torch.Tensor, wf: int, x_scales: torch.Tensor,
                             w_scales: torch.Tensor, block_size: int = 32, bias=None, out=None,
                             stream=None) -> torch.Tensor:
    """Block-scaled GEMM of row-major codes xq [m, k], wq [n, k] with block
    scales [m, nb], [n, nb] and an optional bf16 bias [n]; returns bf16 [m, n]."""
    xq, wq = xq.contiguous(), wq.contiguous()
    x_scales, w_scales = x_scales.contiguous(), w_scales.contiguous()
    m, k = xq.shape
    n = wq.shape[0]
    if bias is not None:
        if bias.dtype != torch.bfloat16 or bias.numel() != n:
            raise ValueError("bias must be bf16 with n elements")
        bias = bias.contiguous()
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=xq.device)
    check(load().hq_gemm_a8w8_blockscaled(_ptr(xq), xf, _ptr(wq), wf, _ptr(x_scales), _ptr(w_scales), int(block_size),
                                          m, n, k, _ptr(bias), _ptr(out), _stream(xq.device, stream)))
    return out


@_on_stream
def hq_gemm_a8w8_blockscaled_preshuffled(xq: torch.Tensor, xf: int, wq_pre: torch.Tensor, wf: int,
                                         x_scales: torch.Tensor, w_scales: torch.Tensor, n: int, block_size: int = 128,
                                         bias=None, out=None, stream=None) -> torch.Tensor:
    """Block-scaled GEMM (blocks of 32, 64 or 128) of row-major codes xq [m, k] and the
    pre-shuffled weight wq_pre (hq_preshuffle_weight of [n, k]) with block
    scales [m, nb], [n, nb] and an optional bf16 bias [n]; returns bf16 [m, n]."""
    xq = xq.contiguous()
    x_scales, w_scales = x_scales.contiguous(), w_scales.contiguous()
    m, k = xq.shape
    if bias is not None:
        if bias.dtype != torch.bfloat16 or bias.numel() != n:
            raise ValueError("bias must be bf16 with n elements")
        bias = bias.contiguous()
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=xq.device)
    check(load().hq_gemm_a8w8_blockscaled_preshuffled(_ptr(xq), xf, _ptr(wq_pre), wf, _ptr(x_scales), _ptr(w_scales),
                                                      int(block_size), m, n, k, _ptr(bias), _ptr(out),
                                                      _stream(xq.device, stream)))
    return out


@_on_stream
def hq_quantize_fp8_layouts(x: torch.Tensor, fmt: int = HQ_E4M3, *, scale_in: torch.Tensor | None = None,
                            ring: Ring | None = None, ring_idx: int = 0, q=False, q_t=False, q_pre=False,
                            q_t_pre=False, scale_out=None, amax_out=None, workspace=None, stream=None):
    """Per-tensor quantization of a 2-D bf16/fp32 tensor into the requested
    layouts in one pass. Each of q, q_t, q_pre, q_t_pre is False (skip), True
    (allocate) or a uint8 tensor to write. Returns a dict with the written
    layouts plus "scale" and "amax" (None with scale_in)."""
    return _layouts(x, fmt, None, scale_in, ring, ring_idx, q, q_t, q_pre, q_t_pre, scale_out, amax_out, workspace,
                    stream)


@_on_stream
def hq_quantize_fp8_layouts_stochastic(x: torch.Tensor, seed: int, *, scale_in: torch.Tensor | None = None,
                                       ring: Ring | None = None, ring_idx: int = 0, q=False, q_t=False, q_pre=False,
                                       q_t_pre=False, scale_out=None, amax_out=None, workspace=None, stream=None):
    """hq_quantize_fp8_layouts with stochastic rounding to E5M2 keyed by `seed`."""
    return _layouts(x, HQ_E5M2, int(seed) & (2 ** 64 - 1), scale_in, ring, ring_idx, q, q_t, q_pre, q_t_pre,
                    scale_out, amax_out, workspace, stream)


def _layouts(x, fmt, seed, scale_in, ring, ring_idx, q, q_t, q_pre, q_t_pre, scale_out, amax_out, workspace,
             stream):
    if x.dtype not in _XT:
        raise ValueError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    x = x.contiguous()
    rows, cols = x.shape
    lib = load()
    dev = x.device
    sizes = {"q": rows * cols, "q_t": rows * cols, "q_pre": max(int(lib.hq_preshuffled_bytes(rows, cols)), 0),
             "q_t_pre": max(int(lib.hq_preshuffled_bytes(cols, rows)), 0)}
    shapes = {"q": (rows, cols), "q_t": (cols, rows), "q_pre": (sizes["q_pre"],), "q_t_pre": (sizes["q_t_pre"],)}
    outs = {}
    for name, want in (("q", q), ("q_t", q_t), ("q_pre", q_pre), ("q_t_pre", q_t_pre)):
        if want is True:
            outs[name] = torch.empty(shapes[name], dtype=torch.uint8, device=dev)
        elif want is not False and want is not None:
            outs[name] = want
    if scale_out is None:
        scale_out = torch.empty(1, dtype=torch.float32, device=dev)
    if amax_out is None and scale_in is None:
        amax_out = torch.empty(1, dtype=torch.float32, device=dev)
    need = 0 if scale_in is not None else int(lib.hq_quantize_workspace_bytes(HQ_PER_TENSOR, rows, cols))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ring_c = ctypes.byref(ring.c_struct(ring_idx)) if ring is not None else None
    tail = (_ptr(outs.get("q")), _ptr(outs.get("q_t")), _ptr(outs.get("q_pre")), _ptr(outs.get("q_t_pre")),
            _ptr(scale_out), _ptr(amax_out), _ptr(workspace), ws_bytes, _stream(dev, stream))
    if seed is None:
        st = lib.hq_quantize_fp8_layouts(_ptr(x), _XT[x.dtype], rows, cols, fmt, _ptr(scale_in), ring_c, *tail)
    else:
        st = lib.hq_quantize_fp8_layouts_stochastic(_ptr(x), _XT[x.dtype], rows, cols, seed, _ptr(scale_in), ring_c,
                                                    *tail)
    check(st)
    outs["scale"] = scale_out
    outs["amax"] = amax_out
    return outs


@_on_stream
def hq_scale_ring_update(ring: Ring, amax: torch.Tensor, fmt: int = HQ_E4M3, ring_idx: int = 0,
                         stream=None) -> None:
    """Fold a device float32 amax scalar into the ring and publish the next scale."""
    lib = load()
    st = lib.hq_scale_ring_update(ctypes.byref(ring.c_struct(ring_idx)), _ptr(amax), fmt,
                                  _stream(ring.state.device, stream))
    check(st)


@_on_stream
def hq_preshuffle_weight(wq: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """Pre-shuffle FP8 codes WQ [n, k] (uint8); returns the flat uint8 buffer."""
    if wq.dim() != 2:
        raise ValueError("wq must be 2-D [n, k]")
    wq = wq.contiguous()
    n, k = wq.shape
    lib = load()
    nbytes = int(lib.hq_preshuffled_bytes(n, k))
    if out is None:
        out = torch.empty(max(nbytes, 0), dtype=torch.uint8, device=wq.device)
    check(lib.hq_preshuffle_weight(_ptr(wq), n, k, _ptr(out), _stream(wq.device, stream)))
    return out


@_on_stream
def hq_stream_rows_probe(x: torch.Tensor, waves: int, out=None, stream=None) -> torch.Tensor:
    """Row-streaming probe over a 2-D 16-bit tensor X [rows, cols] (a
    measurement aid): returns uint8 [rows, cols] holding the high byte of each
    element, written with the per-token quantize's access pattern over a grid
    of `waves` wavefronts."""
    if x.dim() != 2 or x.element_size() != 2:
        raise ValueError("x must be a 2-D tensor of 16-bit elements")
    x = x.contiguous()
    rows, cols = x.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    check(load().hq_stream_rows_probe(_ptr(x), rows, 2 * cols, waves, _ptr(out), _stream(x.device, stream)))
    return out


@_on_stream
def hq_quantize_fp8_preshuffled(x: torch.Tensor, fmt: int = HQ_E4M3, *, row_major: bool = False, q=None,
                                q_pre=None, scale_out=None, amax_out=None, stream=None):
    """Per-row quantization of a weight [n, k] straight into the pre-shuffled
    layout; returns (q_pre uint8 flat, scale_out fp32 [n], amax_out fp32 [n],
    q uint8 [n, k] or None). Row-major codes are written too when `q` is given
    or `row_major` is set."""
    if x.dtype not in _XT:
        raise ValueError(f"x must be float32 or bfloat16, got {x.dtype}")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    x = x.contiguous()
    rows, cols = x.shape
    lib = load()
    dev = x.device
    if q is None and row_major:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if q_pre is None:
        q_pre = torch.empty(max(int(lib.hq_preshuffled_bytes(rows, cols)), 0), dtype=torch.uint8, device=dev)
    if scale_out is None:
        scale_out = torch.empty(rows, dtype=torch.float32, device=dev)
    if amax_out is None:
        amax_out = torch.empty(rows, dtype=torch.float32, device=dev)
    check(lib.hq_quantize_fp8_preshuffled(_ptr(x), _XT[x.dtype], rows, cols, fmt, _ptr(q), _ptr(q_pre),
                                          _ptr(scale_out), _ptr(amax_out), _stream(dev, stream)))
    return q_pre, scale_out, amax_out, q


_GEMM_WORKSPACE = {}


def gemm_workspace(device, nbytes: int) -> torch.Tensor | None:
    """A GEMM workspace of at least `nbytes` for `device` and torch's current
    stream, zero-filled on that stream when made and kept for reuse (the
    kernels leave its counters at zero). Launches on one stream are ordered,
    so they may share it; each stream gets its own."""
    if nbytes <= 0:
        return None
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (dev.type, idx, torch.cuda.current_stream(idx).cuda_stream)
    ws = _GEMM_WORKSPACE.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _GEMM_WORKSPACE[key] = ws
    return ws


@_on_stream
def hq_gemm_a8w8(xq: torch.Tensor, xf: int, wq_pre: torch.Tensor, wf: int, x_scale: torch.Tensor,
                 w_scale: torch.Tensor, n: int, out=None, workspace=None, stream=None,
                 strict: bool = False) -> torch.Tensor:
    """out[m, n] = bf16(x_scale[m] * w_scale[n] * sum_k XQ[m,k] WQ[n,k]); returns out.

    `workspace`: None (a shared zero-filled buffer of the size the shape wants),
    False (run without one) or a zero-filled uint8 device tensor.
    `strict`: exact products (hq_gemm_a8w8_strict) instead of the FP8
    matrix-core window."""
    xq = xq.contiguous()
    m, k = xq.shape
    x_scale = x_scale.contiguous()
    w_scale = w_scale.contiguous()
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=xq.device)
    lib = load()
    if workspace is None:
        workspace = gemm_workspace(xq.device, int(lib.hq_gemm_workspace_bytes(m, n, k)))
    elif workspace is False:
        workspace = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if strict:
        check(lib.hq_gemm_a8w8_strict(_ptr(xq), xf, _ptr(wq_pre), wf, _ptr(x_scale), x_scale.numel(),
                                      _ptr(w_scale), w_scale.numel(), m, n, k, None, _ptr(out), _ptr(workspace),
                                      ws_bytes, _stream(xq.device, stream)))
        return out
    check(lib.hq_gemm_a8w8(_ptr(xq), xf, _ptr(wq_pre), wf, _ptr(x_scale), x_scale.numel(),
                           _ptr(w_scale), w_scale.numel(), m, n, k, _ptr(out), _ptr(workspace), ws_bytes,
                           _stream(xq.device, stream)))
    return out


@_on_stream
def hq_quantize_workspace_status(workspace: torch.Tensor, stream=None) -> bool:
    """True if a one-pass per-tensor / per-channel call on this quantize
    workspace gave up its grid wait since the workspace was zero-filled (its
    scales are NaN). Synchronises with the stream."""
    flag = ctypes.c_int32(0)
    check(load().hq_quantize_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                              ctypes.byref(flag), _stream(workspace.device, stream)))
    return bool(flag.value)


@_on_stream
def hq_gemm_a8w8_noalloc(xq: torch.Tensor, xf: int, wq_pre: torch.Tensor, wf: int, x_scale: torch.Tensor,
                         w_scale: torch.Tensor, n: int, out: torch.Tensor, stream=None) -> torch.Tensor:
    """hq_gemm_a8w8 with the library's own device scratch (no workspace, no
    allocation in the call; `out` is required). Calls that overlap on one GPU
    race on that scratch."""
    for t in (xq, wq_pre, x_scale, w_scale, out):
        if not t.is_contiguous():
            raise ValueError("hq_gemm_a8w8_noalloc takes contiguous tensors (it makes no copies)")
    m, k = xq.shape
    check(load().hq_gemm_a8w8_noalloc(_ptr(xq), xf, _ptr(wq_pre), wf, _ptr(x_scale), x_scale.numel(),
                                      _ptr(w_scale), w_scale.numel(), m, n, k, _ptr(out),
                                      _stream(xq.device, stream)))
    return out


def hq_gemm_a8w8_strict(*args, **kwargs) -> torch.Tensor:
    """hq_gemm_a8w8 with exact products (float16 matrix cores); same arguments."""
    return hq_gemm_a8w8(*args, strict=True, **kwargs)


@_on_stream
def hq_gemm_a8w8_epilogue(xq: torch.Tensor, xf: int, wq_pre: torch.Tensor, wf: int, x_scale: torch.Tensor,
                          w_scale: torch.Tensor, n: int, *, bias: torch.Tensor | None = None,
                          bias_type: int = HQ_BIAS_BF16, bias_scale: torch.Tensor | None = None,
                          out_scale: torch.Tensor | None = None, out_fmt: int = HQ_E4M3, out=None,
                          workspace=None, stream=None, strict: bool = False) -> torch.Tensor:
    """hq_gemm_a8w8 with a bias (bf16 tensor, or uint8 FP8 codes with
    bias_scale) added after the scales, and bf16 output or, with out_scale,
    FP8 (out_fmt) codes of v / out_scale. Returns out (bf16 or uint8 [m, n])."""
    xq = xq.contiguous()
    m, k = xq.shape
    x_scale = x_scale.contiguous()
    w_scale = w_scale.contiguous()
    if bias is not None:
        bias = bias.contiguous()
    if out is None:
        out = torch.empty((m, n), dtype=torch.uint8 if out_scale is not None else torch.bfloat16, device=xq.device)
    lib = load()
    if workspace is None:
        workspace = gemm_workspace(xq.device, int(lib.hq_gemm_workspace_bytes(m, n, k)))
    elif workspace is False:
        workspace = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ep = hq_epilogue(0 if bias is None else bias.data_ptr(), int(bias_type),
                     0 if bias_scale is None else bias_scale.data_ptr(),
                     0 if out_scale is None else out_scale.data_ptr(), int(out_fmt))
    fn = lib.hq_gemm_a8w8_strict if strict else lib.hq_gemm_a8w8_epilogue
    check(fn(_ptr(xq), xf, _ptr(wq_pre), wf, _ptr(x_scale), x_scale.numel(),
             _ptr(w_scale), w_scale.numel(), m, n, k, ctypes.byref(ep), _ptr(out),
             _ptr(workspace), ws_bytes, _stream(xq.device, stream)))
    return out


@_on_stream
def hq_grouped_gemm_a8w8(xq: torch.Tensor, xf: int, wq_pre: torch.Tensor, wf: int,
                         x_scale: torch.Tensor, w_scale: torch.Tensor, group_offsets: torch.Tensor,
                         num_experts: int, n: int, out=None, stream=None, strict: bool = False) -> torch.Tensor:
    """Per-expert GEMM over row ranges [offsets[e], offsets[e+1]); returns out [T, n].
    `strict`: exact products (hq_grouped_gemm_a8w8_strict)."""
    xq = xq.contiguous()
    t, k = xq.shape
    x_scale = x_scale.contiguous()
    w_scale = w_scale.contiguous()
    group_offsets = group_offsets.contiguous()
    if out is None:
        out = torch.empty((t, n), dtype=torch.bfloat16, device=xq.device)
    if strict:
        check(load().hq_grouped_gemm_a8w8_strict(_ptr(xq), xf, _ptr(wq_pre), wf, _ptr(x_scale), x_scale.numel(),
                                                 _ptr(w_scale), w_scale.numel(), _ptr(group_offsets),
                                                 int(num_experts), t, n, k, None, _ptr(out),
                                                 _stream(xq.device, stream)))
        return out
    check(load().hq_grouped_gemm_a8w8(_ptr(xq), xf, _ptr(wq_pre), wf, _ptr(x_scale), x_scale.numel(),
                                      _ptr(w_scale), w_scale.numel(), _ptr(group_offsets),
                                      int(num_experts), t, n, k, _ptr(out),
                                      _stream(xq.device, stream)))
    return out


def hq_grouped_gemm_a8w8_strict(*args, **kwargs) -> torch.Tensor:
    """hq_grouped_gemm_a8w8 with exact products (float16 matrix cores)."""
    return hq_grouped_gemm_a8w8(*args, strict=True, **kwargs)


@_on_stream
def hq_grouped_gemm_a8w8_epilogue(xq: torch.Tensor, xf: int, wq_pre: torch.Tensor, wf: int,
                                  x_scale: torch.Tensor, w_scale: torch.Tensor, group_offsets: torch.Tensor,
                                  num_experts: int, n: int, *, bias: torch.Tensor | None = None,
                                  bias_type: int = HQ_BIAS_BF16, bias_scale: torch.Tensor | None = None,
                                  out_scale: torch.Tensor | None = None, out_fmt: int = HQ_E4M3, out=None,
                                  stream=None, strict: bool = False) -> torch.Tensor:
    """hq_grouped_gemm_a8w8 with a per-expert bias [E, n] (bf16, or uint8 FP8
    codes with bias_scale [E]) and bf16 output or, with out_scale, FP8 codes.
    Returns out (bf16 or uint8 [T, n])."""
    xq = xq.contiguous()
    t, k = xq.shape
    x_scale = x_scale.contiguous()
    w_scale = w_scale.contiguous()
    group_offsets = group_offsets.contiguous()
    if bias is not None:
        bias = bias.contiguous()
    if bias_scale is not None:
        bias_scale = bias_scale.contiguous()
    if out is None:
        out = torch.empty((t, n), dtype=torch.uint8 if out_scale is not None else torch.bfloat16, device=xq.device)
    ep = hq_epilogue(0 if bias is None else bias.data_ptr(), int(bias_type),
                     0 if bias_scale is None else bias_scale.data_ptr(),
                     0 if out_scale is None else out_scale.data_ptr(), int(out_fmt))
    lib = load()
    fn = lib.hq_grouped_gemm_a8w8_strict if strict else lib.hq_grouped_gemm_a8w8_epilogue
    check(fn(_ptr(xq), xf, _ptr(wq_pre), wf, _ptr(x_scale), x_scale.numel(),
             _ptr(w_scale), w_scale.numel(), _ptr(group_offsets),
             int(num_experts), t, n, k, ctypes.byref(ep), _ptr(out),
             _stream(xq.device, stream)))
    return out
