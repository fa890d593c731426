"""Benchmark of the dynamic-FP8 quantize + a8w8 GEMM hot path on one MI355X.

Workload (the PTPC square configuration): X bf16 [4096, 4096] N(0,1) with 0.1%
of entries x50, W bf16 [4096, 4096] N(0, 0.02^2). One step is one pass of the
whole path: per-token E4M3 quantization of X, per-output-channel E4M3
quantization of W (row reduction on [N, K]) written straight into the GEMM's
pre-shuffled weight layout (the quantize and pre-shuffle in one pass), and the
a8w8 GEMM M = N = K = 4096 into bf16. The two-launch form of the weight side
(row-major codes, then the pre-shuffle) is timed beside it. Inputs are resident in HBM before timing;
``--rotate`` input/output sets (default 8, ~1.2 GB) cycle so that neither a step
nor a single kernel's timing loop finds its data in the 256 MB Infinity Cache.

Prints one JSON line (stdout). ``value`` = 2*M*N*K / step time (TFLOP/s of the
whole step). ``roofline`` refers to the dominant kernel (the GEMM), timed with
HIP events on the stream it runs on. ``cpu_baseline`` times the CPU oracle on
the same workload for a bounded time (see --cpu-seconds): the whole step at
full size with the quantizations on a process pool over row blocks and the
float64 GEMM on the BLAS threads, plus the quantize oracle on one core.

    python bench.py [--gpus 1] [--steps 50] [--warmup 200]

Helpers for the rocprofv3 summaries kept with the sources (they read
``--output-format csv`` output and run on any host):

    python bench.py --summarize DIR            # markdown table of a trace/PMC run
    python bench.py --write-traffic NAME KERNEL FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "a8w8 GEMM TFLOP/s + quantize GB/s (% of MI355X roofline), PTPC 4096³"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 MFMA (the strict GEMM's instruction)
M = N = K = 4096
COPY_PROBE_BYTES = 1 << 30
NUM_CUS = 256
QUANT_ROW_WAVES_PER_CU = 12         # the per-token quantize's grid (wavefronts per compute unit)
ROW_PROBE_WAVES_PER_CU = (4, 8, 12, 16)
COPY_PROBE_KERNEL = "bitwise_not"
KERNEL_SOURCES = ["fp8_dynamic_quantization_amd/csrc/gemm.hip", "fp8_dynamic_quantization_amd/csrc/quantize.hip",
                  "fp8_dynamic_quantization_amd/csrc/hq_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Buffers:
    """One rotating set of device buffers for a step."""

    def __init__(self, torch, x_bits, w_bits, pre_bytes):
        dev = "cuda"
        self.x = torch.from_numpy(x_bits.view("int16")).to(dev).view(torch.bfloat16)
        self.w = torch.from_numpy(w_bits.view("int16")).to(dev).view(torch.bfloat16)
        self.xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        self.wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        self.xs = torch.empty(M, dtype=torch.float32, device=dev)
        self.ws = torch.empty(N, dtype=torch.float32, device=dev)
        self.xa = torch.empty(M, dtype=torch.float32, device=dev)
        self.wa = torch.empty(N, dtype=torch.float32, device=dev)
        self.wpre = torch.empty(pre_bytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.p = {k: p(getattr(self, k)) for k in ("x", "w", "xq", "wq", "xs", "ws", "xa", "wa", "wpre", "out")}


def make_ops(hq, lib, stream):
    """Per-kernel launch closures calling the C ABI with pre-marshalled pointers
    (on `stream` unless a stream handle is passed)."""
    E4M3, BF16, TOK = hq.HQ_E4M3, hq.HQ_BF16, hq.HQ_PER_TOKEN

    def quant_x(b, h=None):
        st = lib.hq_quantize_fp8(b.p["x"], BF16, M, K, E4M3, TOK, b.p["xq"], b.p["xs"], b.p["xa"], None, None, 0,
                                 h or stream)
        assert st == 0, hq.hq_last_error()

    def quant_w(b, h=None):
        st = lib.hq_quantize_fp8(b.p["w"], BF16, N, K, E4M3, TOK, b.p["wq"], b.p["ws"], b.p["wa"], None, None, 0,
                                 h or stream)
        assert st == 0, hq.hq_last_error()

    def preshuffle(b, h=None):
        st = lib.hq_preshuffle_weight(b.p["wq"], N, K, b.p["wpre"], h or stream)
        assert st == 0, hq.hq_last_error()

    def quant_w_pre(b, h=None):
        st = lib.hq_quantize_fp8_preshuffled(b.p["w"], BF16, N, K, E4M3, None, b.p["wpre"], b.p["ws"], b.p["wa"],
                                             h or stream)
        assert st == 0, hq.hq_last_error()

    def gemm(b, h=None):
        st = lib.hq_gemm_a8w8(b.p["xq"], E4M3, b.p["wpre"], E4M3, b.p["xs"], M, b.p["ws"], N, M, N, K, b.p["out"],
                              None, 0, h or stream)
        assert st == 0, hq.hq_last_error()

    step = {"quant_x": quant_x, "quant_w_pre": quant_w_pre, "gemm": gemm}
    # the two-launch form of quant_w_pre (row-major codes, then the pre-shuffle),
    # timed for comparison only
    two_launch = {"quant_w": quant_w, "preshuffle": preshuffle}
    return step, two_launch


def time_kernel(torch, fn, sets, reps):
    """Average duration (ms) of `fn` over `reps` launches on the current stream."""
    for i in range(3):
        fn(sets[i % len(sets)])
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(reps):
        fn(sets[i % len(sets)])
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def traffic_from_profile(name):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash():
        return None
    return d.get("bytes_per_launch")


_POOL_X = None


def _pool_init():
    """Worker set-up (untimed): the seeded PTPC inputs, made by the generator."""
    global _POOL_X
    import workloads
    _POOL_X = workloads.ptpc_square(1)


def _pool_quant(task):
    """Oracle per-token quantization of rows [lo, hi) of X (which = 0) or W (1)."""
    from oracle import fp8, quantize as Q
    which, lo, hi = task
    q, s, _ = Q.quantize_dynamic(_POOL_X[which][lo:hi], Q.BF16, fp8.E4M3, Q.PER_TOKEN)
    return which, lo, q, s


def cpu_baseline(min_seconds: float):
    """Time the CPU oracle on the PTPC 4096^3 workload:
      * the quantize oracle (per-token E4M3 of X bf16 [4096, 4096]) on one core,
        in GB/s of the same algorithmic bytes as the GPU quantize;
      * the whole step: per-token quantization of X and W on a process pool
        over 64-row blocks (min(16, cpu count) workers), the pre-shuffle of WQ,
        and the float64 GEMM on the BLAS threads, repeated for at least
        `min_seconds`; `value` is 2*M*N*K / step time."""
    import multiprocessing as mp

    import numpy as np

    import workloads
    from oracle import fp8, gemm as G, preshuffle as P, quantize as Q
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    x, w = workloads.ptpc_square(1)
    quant_bytes = M * K * 3 + M * 8
    # one core: 1024 rows at a time, repeated for about 2 s
    rows, reps, t1 = 1024, 0, 0.0
    while reps == 0 or t1 < 2.0:
        t0 = time.perf_counter()
        Q.quantize_dynamic(x[:rows], Q.BF16, fp8.E4M3, Q.PER_TOKEN)
        t1 += time.perf_counter() - t0
        reps += 1
    gbs_1 = quant_bytes * rows / M / (t1 / reps) / 1e9
    workers = max(1, min(16, os.cpu_count() or 1))
    ctx = mp.get_context("spawn")  # fresh interpreters: no GPU state in the workers
    with ctx.Pool(workers, initializer=_pool_init) as pool:
        pool.map(_pool_quant, [(0, 0, 1)] * workers)  # workers up (untimed)
        tasks = [(which, lo, lo + 64) for which in (0, 1) for lo in range(0, M, 64)]
        steps, t_all, t_quant, t_gemm = 0, 0.0, 0.0, 0.0
        while steps == 0 or t_all < min_seconds:
            t0 = time.perf_counter()
            xq = np.empty((M, K), np.uint8)
            wq = np.empty((N, K), np.uint8)
            xs = np.empty(M, np.float32)
            ws = np.empty(N, np.float32)
            for which, lo, q, sc in pool.imap_unordered(_pool_quant, tasks, chunksize=4):
                (xq if which == 0 else wq)[lo:lo + len(q)] = q
                (xs if which == 0 else ws)[lo:lo + len(sc)] = sc
            t_q = time.perf_counter()
            P.preshuffle(wq)
            G.gemm_a8w8(xq, fp8.E4M3, wq, fp8.E4M3, xs, ws)
            t_e = time.perf_counter()
            t_quant += t_q - t0
            t_gemm += t_e - t_q
            t_all += t_e - t0
            steps += 1
    per = t_all / steps
    return {
        "value": round(2.0 * M * N * K / per / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(max(workers, blas)),
        "kind": "oracle",
        "sample": (f"the whole step at full size: oracle per-token quantization of X and W on {workers} worker "
                   f"processes (64-row blocks), pre-shuffle of WQ, float64 {M}x{N}x{K} GEMM on {blas} BLAS threads; "
                   f"{steps} steps, {t_all:.1f} s in total, {per:.2f} s each; plus the quantize oracle on one core "
                   f"over {rows} rows x {reps}"),
        "os_cpu_count": os.cpu_count(),
        "quantize_x": {"gbs_1core": round(gbs_1, 4),
                       "gbs_all_workers": round(2 * quant_bytes / (t_quant / steps) / 1e9, 4),
                       "workers": workers, "algorithmic_bytes": quant_bytes},
        "gemm_float64": {"tflops": round(2.0 * M * N * K / (t_gemm / steps) / 1e12, 6), "blas_threads": blas},
    }


# Untimed replays before the timed ones: at least this much GPU time of the
# same launches, so each kernel is timed at the clock it settles at under its
# own load whatever ran before it (from a cold start the PTPC step takes about
# 150 steps, 12 ms, to settle).
GRAPH_WARM_MS = 25.0
GRAPH_WARM_MAX_REPLAYS = 2000


def time_graph(torch, launch, reps, replays=5, info=None):
    """Average duration (ms) of one launch: `reps` launches captured in a HIP
    graph (launch(i, stream_handle)), replayed back to back, so host launch
    overhead does not hide short kernels. The graph is first replayed untimed
    until GRAPH_WARM_MS have passed (the count goes to info["untimed_replays"]
    when a dict is given)."""
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(reps):
            launch(i, h)
    warm = 0
    t_warm = time.perf_counter()
    while True:
        g.replay()
        warm += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t_warm) * 1e3 >= GRAPH_WARM_MS or warm >= GRAPH_WARM_MAX_REPLAYS:
            break
    if info is not None:
        info["untimed_replays"] = warm
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (replays * reps)


class MoeSets:
    """The grouped MoE workload on the device: 8 experts, N = 2048, K = 1024,
    8192 rows, per-token x per-expert-channel E4M3; 5 rotating (codes,
    pre-shuffled weights, output) sets, 141 MB together."""

    def __init__(self, torch, hq, lib):
        import workloads
        x, w, offs = workloads.grouped_moe()
        self.e, self.n, self.k = w.shape
        self.t = x.shape[0]
        self.offs = offs
        e4 = hq.HQ_E4M3
        gx, self.xs, _ = hq.hq_quantize_fp8(torch.from_numpy(x.view("int16")).cuda().view(torch.bfloat16), e4,
                                            hq.HQ_PER_TOKEN)
        gw, self.ws, _ = hq.hq_quantize_fp8(torch.from_numpy(w.reshape(self.e * self.n, self.k).view("int16"))
                                            .cuda().view(torch.bfloat16), e4, hq.HQ_PER_TOKEN)
        pre = torch.cat([hq.hq_preshuffle_weight(gw[i * self.n:(i + 1) * self.n]) for i in range(self.e)])
        self.off = torch.from_numpy(offs).cuda()
        self.sets = [(gx.clone(), pre.clone(), torch.empty((self.t, self.n), dtype=torch.bfloat16, device="cuda"))
                     for _ in range(5)]
        self.lib, self.hq = lib, hq

    def launch(self, i, h):
        P = ctypes.c_void_p
        a, b, o = self.sets[i % len(self.sets)]
        st = self.lib.hq_grouped_gemm_a8w8(P(a.data_ptr()), self.hq.HQ_E4M3, P(b.data_ptr()), self.hq.HQ_E4M3,
                                           P(self.xs.data_ptr()), self.t, P(self.ws.data_ptr()), self.e * self.n,
                                           P(self.off.data_ptr()), self.e, self.t, self.n, self.k, P(o.data_ptr()), h)
        assert st == 0, self.hq.hq_last_error()


def other_workloads(torch, hq, lib, reps):
    """Decode-skinny GEMM, grouped MoE GEMM and per-tensor / per-channel
    quantize, each timed on rotating buffers larger than the Infinity Cache."""
    import numpy as np

    import workloads
    P = ctypes.c_void_p
    E4M3, BF16 = hq.HQ_E4M3, hq.HQ_BF16
    res = {}

    # decode: X [m, 7168] x W [2048, 7168], 24 weight copies (353 MB)
    dn, dk, copies = 2048, 7168, 24
    dec = {}
    for m in (1, 8, 32):
        x, w = workloads.decode_skinny(m)
        gx, gxs, _ = hq.hq_quantize_fp8(torch.from_numpy(x.view("int16")).cuda().view(torch.bfloat16), E4M3,
                                        hq.HQ_PER_TOKEN)
        if m == 1:
            gw, gws, _ = hq.hq_quantize_fp8(torch.from_numpy(w.view("int16")).cuda().view(torch.bfloat16), E4M3,
                                            hq.HQ_PER_TOKEN)
            pre = hq.hq_preshuffle_weight(gw)
            pres = [pre.clone() for _ in range(copies)]
            del gw
        out = torch.empty((m, dn), dtype=torch.bfloat16, device="cuda")
        wsb = hq.hq_gemm_workspace_bytes(m, dn, dk)
        work = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")

        def launch(i, h, gx=gx, gxs=gxs, out=out, m=m, work=work, wsb=wsb):
            st = lib.hq_gemm_a8w8(P(gx.data_ptr()), E4M3, P(pres[i % copies].data_ptr()), E4M3, P(gxs.data_ptr()),
                                  m, P(gws.data_ptr()), dn, m, dn, dk, P(out.data_ptr()), P(work.data_ptr()), wsb, h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, launch, 2 * copies)
        alg = dn * dk + m * dk + 2 * m * dn + 4 * (m + dn)

        def slaunch(i, h, gx=gx, gxs=gxs, out=out, m=m, work=work, wsb=wsb):
            st = lib.hq_gemm_a8w8_strict(P(gx.data_ptr()), E4M3, P(pres[i % copies].data_ptr()), E4M3,
                                         P(gxs.data_ptr()), m, P(gws.data_ptr()), dn, m, dn, dk, None,
                                         P(out.data_ptr()), P(work.data_ptr()), wsb, h)
            assert st == 0, hq.hq_last_error()
        sms = time_graph(torch, slaunch, 2 * copies)
        dec[f"m{m}"] = {"us": round(ms * 1e3, 3), "gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg,
                        "strict_us": round(sms * 1e3, 3)}
    res["decode_skinny"] = {"shape": "M in {1,8,32}, N=2048, K=7168, per-token x per-channel E4M3",
                            "rotating_weight_copies": copies, **dec}
    del pres

    # grouped MoE: 8 experts, N=2048, K=1024, 8192 rows; 5 rotating sets
    moe = MoeSets(torch, hq, lib)
    gsets, gxs, gws, off_d, offs = moe.sets, moe.xs, moe.ws, moe.off, moe.offs
    e_, gn, gk, t = moe.e, moe.n, moe.k, moe.t
    ms = time_graph(torch, moe.launch, 10)

    def gslaunch(i, h):
        a, b, o = gsets[i % len(gsets)]
        st = lib.hq_grouped_gemm_a8w8_strict(P(a.data_ptr()), E4M3, P(b.data_ptr()), E4M3, P(gxs.data_ptr()), t,
                                             P(gws.data_ptr()), e_ * gn, P(off_d.data_ptr()), e_, t, gn, gk, None,
                                             P(o.data_ptr()), h)
        assert st == 0, hq.hq_last_error()
    strict_ms = time_graph(torch, gslaunch, 10)
    nonempty = int(np.count_nonzero(np.diff(offs)))
    flops = 2.0 * t * gn * gk
    alg = t * gk + nonempty * gn * gk + 2 * t * gn + 4 * (t + e_ * gn)
    res["grouped_moe"] = {"shape": f"{e_} experts ({nonempty} non-empty), N={gn}, K={gk}, {t} rows",
                          "us": round(ms * 1e3, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                          "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                          "gbs": round(alg / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes": alg,
                          "strict_us": round(strict_ms * 1e3, 3), "traffic": traffic_from_profile("grouped_moe")}
    del gsets, moe

    # GEMM epilogue variants on the PTPC 4096^3 operands: bf16 bias, and FP8 E4M3 output with an output scale
    x, w = workloads.ptpc_square(1)
    gx, gxs, _ = hq.hq_quantize_fp8(torch.from_numpy(x.view("int16")).cuda().view(torch.bfloat16), E4M3,
                                    hq.HQ_PER_TOKEN)
    gw, gws, _ = hq.hq_quantize_fp8(torch.from_numpy(w.view("int16")).cuda().view(torch.bfloat16), E4M3,
                                    hq.HQ_PER_TOKEN)
    pre = hq.hq_preshuffle_weight(gw)
    esets = [(gx.clone(), pre.clone()) for _ in range(4)]
    bias = torch.randn(N, device="cuda").to(torch.bfloat16)
    osc = torch.full((1,), 0.05, dtype=torch.float32, device="cuda")
    ep_res = {}
    for name, ep, obytes in (("bias_bf16_out_bf16", hq.hq_epilogue(bias.data_ptr(), hq.HQ_BIAS_BF16, None, None, 0), 2),
                             ("out_e4m3", hq.hq_epilogue(None, 0, None, osc.data_ptr(), E4M3), 1)):
        outs = [torch.empty(M * N * obytes, dtype=torch.uint8, device="cuda") for _ in range(4)]

        def elaunch(i, h, ep=ep, outs=outs):
            a_, p_ = esets[i % 4]
            st = lib.hq_gemm_a8w8_epilogue(P(a_.data_ptr()), E4M3, P(p_.data_ptr()), E4M3, P(gxs.data_ptr()), M,
                                           P(gws.data_ptr()), N, M, N, K, ctypes.byref(ep),
                                           P(outs[i % 4].data_ptr()), None, 0, h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, elaunch, 8)
        ep_res[name] = {"us": round(ms * 1e3, 3), "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
    res["gemm_epilogue_ptpc4096"] = ep_res
    # the strict GEMM (exact products on the float16 matrix cores) on the same operands
    souts = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(4)]

    def slaunch4096(i, h):
        a_, p_ = esets[i % 4]
        st = lib.hq_gemm_a8w8_strict(P(a_.data_ptr()), E4M3, P(p_.data_ptr()), E4M3, P(gxs.data_ptr()), M,
                                     P(gws.data_ptr()), N, M, N, K, None, P(souts[i % 4].data_ptr()), None, 0, h)
        assert st == 0, hq.hq_last_error()
    ms = time_graph(torch, slaunch4096, 8)
    tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    res["gemm_strict_ptpc4096"] = {"us": round(ms * 1e3, 3), "tflops": round(tf, 1),
                                   "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
                                   "frac_f16_peak": round(tf / F16_PEAK_TFLOPS, 4)}
    del souts
    del esets, gx, gw, pre

    # quantize of the PTPC X [4096, 4096] bf16 at the other two granularities
    x, _ = workloads.ptpc_square(1)
    xs_ = [torch.from_numpy(x.view("int16")).cuda().view(torch.bfloat16) for _ in range(8)]
    q = [torch.empty((M, K), dtype=torch.uint8, device="cuda") for _ in range(8)]
    qv = {}
    for name, gran in (("per_tensor", hq.HQ_PER_TENSOR), ("per_channel", hq.HQ_PER_CHANNEL)):
        cnt = int(lib.hq_scale_count(gran, M, K))
        so = torch.empty(cnt, dtype=torch.float32, device="cuda")
        ao = torch.empty(cnt, dtype=torch.float32, device="cuda")
        wsb = int(lib.hq_quantize_workspace_bytes(gran, M, K))
        wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")

        def qlaunch(i, h, gran=gran, so=so, ao=ao, wsp=wsp, wsb=wsb):
            st = lib.hq_quantize_fp8(P(xs_[i % 8].data_ptr()), BF16, M, K, E4M3, gran, P(q[i % 8].data_ptr()),
                                     P(so.data_ptr()), P(ao.data_ptr()), None, P(wsp.data_ptr()), wsb, h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, qlaunch, 24)
        alg = M * K * 3 + 8 * cnt
        qv[name] = {"us": round(ms * 1e3, 3), "gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg}
    res["quantize_x_other_granularities"] = {"shape": "X bf16 [4096,4096] -> E4M3", **qv}
    del xs_, q

    res["tiny_per_tensor"] = tiny_timings(torch, hq, lib)
    res["blockwise_ptpc4096"] = blockwise_timings(torch, hq, lib)
    res["training_linear"] = training_linear_timings(torch, hq, lib)
    return res


def tiny_timings(torch, hq, lib):
    """The tiny per-tensor workload as one step: per-tensor E4M3 quantization of
    X fp32 [16, 128] and W fp32 [64, 128] (one pass each, scale reduced on the
    device), the pre-shuffle of WQ and the GEMM 16 x 64 x 128 into bf16;
    latency-bound, so reported in microseconds per step (HIP graph)."""
    import workloads
    P = ctypes.c_void_p
    E4M3, F32, TEN = hq.HQ_E4M3, hq.HQ_F32, hq.HQ_PER_TENSOR
    x, w = workloads.tiny_per_tensor(0)
    gx, gw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    xq = torch.empty((16, 128), dtype=torch.uint8, device="cuda")
    wq = torch.empty((64, 128), dtype=torch.uint8, device="cuda")
    pre = torch.empty(hq.hq_preshuffled_bytes(64, 128), dtype=torch.uint8, device="cuda")
    xs, ws = torch.empty(1, device="cuda"), torch.empty(1, device="cuda")
    out = torch.empty((16, 64), dtype=torch.bfloat16, device="cuda")
    wsb = int(lib.hq_quantize_workspace_bytes(TEN, 64, 128))
    wx = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    ww = torch.zeros(wsb, dtype=torch.uint8, device="cuda")

    def step(i, h):
        for src, q, s, work, rows in ((gx, xq, xs, wx, 16), (gw, wq, ws, ww, 64)):
            st = lib.hq_quantize_fp8(P(src.data_ptr()), F32, rows, 128, E4M3, TEN, P(q.data_ptr()), P(s.data_ptr()),
                                     None, None, P(work.data_ptr()), wsb, h)
            assert st == 0, hq.hq_last_error()
        st = lib.hq_preshuffle_weight(P(wq.data_ptr()), 64, 128, P(pre.data_ptr()), h)
        assert st == 0, hq.hq_last_error()
        st = lib.hq_gemm_a8w8(P(xq.data_ptr()), E4M3, P(pre.data_ptr()), E4M3, P(xs.data_ptr()), 1,
                              P(ws.data_ptr()), 1, 16, 64, 128, P(out.data_ptr()), None, 0, h)
        assert st == 0, hq.hq_last_error()
    ms = time_graph(torch, step, 32)
    return {"shape": "X fp32 [16,128], W fp32 [64,128], per-tensor E4M3, GEMM 16x64x128 -> bf16",
            "us_per_step": round(ms * 1e3, 3), "launches_per_step": 4}


def blockwise_timings(torch, hq, lib):
    """Block-wise path on the PTPC operands: X bf16 [4096, 4096] quantized in
    blocks of 32 and 128 along K (codes + one float32 scale and amax per block),
    and the block-scaled GEMM 4096^3 at blocks of 32, 64 and 128 on the codes
    of X and W quantized at that block size, over the row-major and over the
    pre-shuffled weight. Rotating sets as elsewhere."""
    import workloads
    P = ctypes.c_void_p
    E4M3, BF16 = hq.HQ_E4M3, hq.HQ_BF16
    x, w = workloads.ptpc_square(1)
    xd = [torch.from_numpy(x.view("int16")).cuda().view(torch.bfloat16) for _ in range(8)]
    q = [torch.empty((M, K), dtype=torch.uint8, device="cuda") for _ in range(8)]
    quant = {}
    for bs in (32, 128):
        nb = K // bs
        so = [torch.empty((M, nb), dtype=torch.float32, device="cuda") for _ in range(8)]
        ao = [torch.empty((M, nb), dtype=torch.float32, device="cuda") for _ in range(8)]

        def qlaunch(i, h, bs=bs, so=so, ao=ao):
            st = lib.hq_quantize_fp8_blockwise(P(xd[i % 8].data_ptr()), BF16, M, K, E4M3, bs, 0, 0,
                                               P(q[i % 8].data_ptr()), P(so[i % 8].data_ptr()),
                                               P(ao[i % 8].data_ptr()), h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, qlaunch, 16)
        alg = M * K * 3 + 2 * M * nb * 4
        quant[f"bs{bs}"] = {"us": round(ms * 1e3, 3), "gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg}
    del q
    wd = torch.from_numpy(w.view("int16")).cuda().view(torch.bfloat16)
    gemm = {}
    for bs in (32, 64, 128):
        xq, xs, _ = hq.hq_quantize_fp8_blockwise(xd[0], E4M3, bs)
        wq, ws, _ = hq.hq_quantize_fp8_blockwise(wd, E4M3, bs)
        sets = [(xq.clone(), wq.clone(), xs.clone(), ws.clone(), torch.empty((M, N), dtype=torch.bfloat16,
                                                                               device="cuda")) for _ in range(4)]

        def glaunch(i, h, bs=bs, sets=sets):
            a_, b_, c_, d_, o_ = sets[i % 4]
            st = lib.hq_gemm_a8w8_blockscaled(P(a_.data_ptr()), E4M3, P(b_.data_ptr()), E4M3, P(c_.data_ptr()),
                                              P(d_.data_ptr()), bs, M, N, K, None, P(o_.data_ptr()), h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, glaunch, 8)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        # the fold: one multiply and one FMA per output element per block, wave64
        # FP32 VALU at 16 lanes x 4 SIMDs x 256 CUs x 2.4 GHz
        valu_floor_us = 2.0 * M * N * (K // bs) / (16 * 4 * 256 * 2.4e9) * 1e6
        gemm[f"bs{bs}"] = {"us": round(ms * 1e3, 3), "tflops": round(tf, 1), "frac_mfma": round(tf / FP8_PEAK_TFLOPS, 4),
                           "fold_valu_floor_us": round(valu_floor_us, 1)}
        # the same product through the pre-shuffled weight (the plain GEMM's data path)
        psets = [(a_, hq.hq_preshuffle_weight(b_), c_, d_, o_) for a_, b_, c_, d_, o_ in sets]

        def plaunch(i, h, bs=bs, psets=psets):
            a_, p_, c_, d_, o_ = psets[i % 4]
            st = lib.hq_gemm_a8w8_blockscaled_preshuffled(P(a_.data_ptr()), E4M3, P(p_.data_ptr()), E4M3,
                                                          P(c_.data_ptr()), P(d_.data_ptr()), bs, M, N, K, None,
                                                          P(o_.data_ptr()), h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, plaunch, 8)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        gemm[f"bs{bs}_preshuffled"] = {"us": round(ms * 1e3, 3), "tflops": round(tf, 1),
                                       "frac_mfma": round(tf / FP8_PEAK_TFLOPS, 4),
                                       "fold_valu_floor_us": round(valu_floor_us, 1)}
        del psets
        del sets
    return {"shape": "X, W bf16 [4096, 4096] (PTPC operands), E4M3, blocks along K", "quantize_x": quant,
            "gemm_4096": gemm}


def training_linear_timings(torch, hq, lib, copies=12):
    """One layer of the training-linear workload (X [2048,1024], W [4096,1024],
    G [2048,4096] bf16): the delayed-scaling quantizations (E4M3 X and W, E5M2
    G, each with its 16-entry ring folded in the same launch) and the three
    GEMMs (forward E4M3, dgrad and wgrad E5M2 x E5M2), each timed over `copies`
    layers' worth of distinct buffers (> 256 MB in all)."""
    import numpy as np  # noqa: F401

    import workloads
    P = ctypes.c_void_p
    E4M3, E5M2, BF16, TEN = hq.HQ_E4M3, hq.HQ_E5M2, hq.HQ_BF16, hq.HQ_PER_TENSOR
    base, factors = workloads.training_linear(4, layers=1, steps=1)
    bits = workloads.training_step_inputs(base, factors, 0, 0)
    dev = [torch.from_numpy(b.view("int16")).cuda().view(torch.bfloat16) for b in bits]
    names = ("x", "w", "g")
    fmts = (E4M3, E4M3, E5M2)
    out = {}
    for t, name, fmt in zip(dev, names, fmts):
        rows, cols = t.shape
        srcs = [t.clone() for _ in range(copies)]
        qs = [torch.empty((rows, cols), dtype=torch.uint8, device="cuda") for _ in range(copies)]
        rings = [hq.Ring(16) for _ in range(copies)]
        so = torch.empty(1, dtype=torch.float32, device="cuda")
        wsb = int(lib.hq_quantize_workspace_bytes(TEN, rows, cols))
        wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        ring_structs = [r.c_struct(0) for r in rings]

        def launch(i, h, srcs=srcs, qs=qs, rows=rows, cols=cols, fmt=fmt, so=so, wsp=wsp, wsb=wsb):
            st = lib.hq_quantize_fp8(P(srcs[i % copies].data_ptr()), BF16, rows, cols, fmt, TEN,
                                     P(qs[i % copies].data_ptr()), P(so.data_ptr()), None,
                                     ctypes.byref(ring_structs[i % copies]), P(wsp.data_ptr()), wsb, h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, launch, 2 * copies)
        alg = rows * cols * 3 + 4 * 18
        out[f"quant_{name}_delayed"] = {"shape": f"[{rows},{cols}] bf16 -> {'E4M3' if fmt == E4M3 else 'E5M2'}",
                                         "us": round(ms * 1e3, 3), "gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                                         "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del srcs, qs, rings
    # Backward operands in one pass each (hq_quantize_fp8_layouts): G (E5M2, its ring) row-major for dgrad and
    # transposed for wgrad; W and X (E5M2, their forward scales) straight into the pre-shuffled transposed
    # layouts the two GEMMs take. Algorithmic bytes: input + one byte per code written.
    sw = torch.full((1,), 0.02 * 4.5 / 448.0, dtype=torch.float32, device="cuda")
    sx = torch.full((1,), 4.5 / 448.0, dtype=torch.float32, device="cuda")
    for name, t, kw, nbytes in (
            ("g_e5m2_ring_q_and_qt", dev[2], dict(q=True, q_t=True), 2),
            ("w_e5m2_given_qt_pre", dev[1], dict(q_t_pre=True), 1),
            ("x_e5m2_given_qt_pre", dev[0], dict(q_t_pre=True), 1)):
        rows, cols = t.shape
        srcs = [t.clone() for _ in range(copies)]
        outs = [hq.hq_quantize_fp8_layouts(srcs[i], E5M2, scale_in=None if name.startswith("g") else
                                           (sw if name.startswith("w") else sx),
                                           ring=hq.Ring(16) if name.startswith("g") else None, **kw)
                for i in range(copies)]
        rings = [hq.Ring(16) for _ in range(copies)] if name.startswith("g") else None
        ring_structs = [r.c_struct(0) for r in rings] if rings else None
        wsb = int(lib.hq_quantize_workspace_bytes(TEN, rows, cols))
        wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        so = torch.empty(1, dtype=torch.float32, device="cuda")

        def llaunch(i, h, srcs=srcs, outs=outs, rows=rows, cols=cols, name=name, so=so, wsp=wsp, wsb=wsb,
                    ring_structs=ring_structs):
            o = outs[i % copies]
            given = None if name.startswith("g") else (sw if name.startswith("w") else sx)
            st = lib.hq_quantize_fp8_layouts(P(srcs[i % copies].data_ptr()), BF16, rows, cols, E5M2,
                                             P(given.data_ptr()) if given is not None else None,
                                             ctypes.byref(ring_structs[i % copies]) if ring_structs else None,
                                             P(o["q"].data_ptr()) if "q" in o else None,
                                             P(o["q_t"].data_ptr()) if "q_t" in o else None, None,
                                             P(o["q_t_pre"].data_ptr()) if "q_t_pre" in o else None,
                                             P(so.data_ptr()), None, P(wsp.data_ptr()) if given is None else None,
                                             wsb if given is None else 0, h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, llaunch, 2 * copies)
        alg = rows * cols * (2 + nbytes)
        out[f"layouts_{name}"] = {"shape": f"[{rows},{cols}] bf16", "us": round(ms * 1e3, 3),
                                  "gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del srcs, outs
    # G with stochastic rounding and its ring (hq_quantize_fp8_stochastic)
    rows, cols = dev[2].shape
    srcs = [dev[2].clone() for _ in range(copies)]
    qs = [torch.empty((rows, cols), dtype=torch.uint8, device="cuda") for _ in range(copies)]
    rings = [hq.Ring(16) for _ in range(copies)]
    ring_structs = [r.c_struct(0) for r in rings]
    wsb = int(lib.hq_quantize_workspace_bytes(TEN, rows, cols))
    wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    so = torch.empty(1, dtype=torch.float32, device="cuda")

    def slaunch(i, h):
        st = lib.hq_quantize_fp8_stochastic(P(srcs[i % copies].data_ptr()), BF16, rows, cols, TEN, 1234 + i,
                                            P(qs[i % copies].data_ptr()), P(so.data_ptr()), None,
                                            ctypes.byref(ring_structs[i % copies]), P(wsp.data_ptr()), wsb, h)
        assert st == 0, hq.hq_last_error()
    ms = time_graph(torch, slaunch, 2 * copies)
    alg = rows * cols * 3
    out["quant_g_delayed_stochastic"] = {"shape": f"[{rows},{cols}] bf16 -> E5M2 (stochastic)",
                                         "us": round(ms * 1e3, 3), "gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                                         "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # the same, written row-major (dgrad) and transposed (wgrad) in one pass
    # (hq_quantize_fp8_layouts_stochastic); algorithmic bytes: input + two codes
    qts = [torch.empty((cols, rows), dtype=torch.uint8, device="cuda") for _ in range(copies)]

    def sllaunch(i, h):
        st = lib.hq_quantize_fp8_layouts_stochastic(P(srcs[i % copies].data_ptr()), BF16, rows, cols, 1234 + i, None,
                                                    ctypes.byref(ring_structs[i % copies]),
                                                    P(qs[i % copies].data_ptr()), P(qts[i % copies].data_ptr()),
                                                    None, None, P(so.data_ptr()), None, P(wsp.data_ptr()), wsb, h)
        assert st == 0, hq.hq_last_error()
    ms = time_graph(torch, sllaunch, 2 * copies)
    alg = rows * cols * 4
    out["layouts_g_e5m2_ring_q_and_qt_stochastic"] = {"shape": f"[{rows},{cols}] bf16", "us": round(ms * 1e3, 3),
                                                      "gbs": round(alg / (ms * 1e-3) / 1e9, 1),
                                                      "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del srcs, qs, qts, rings

    # GEMM operands (made once, untimed): E4M3 X, W for the forward; E5M2 G, W^T, G^T, X^T for the backward
    def quant(t, fmt):
        return hq.hq_quantize_fp8(t, fmt, TEN)

    xq, xs, _ = quant(dev[0], E4M3)
    wq, ws, _ = quant(dev[1], E4M3)
    gq, gs, _ = quant(dev[2], E5M2)
    wq5, ws5, _ = quant(dev[1], E5M2)
    xq5, xs5, _ = quant(dev[0], E5M2)
    cases = {
        "gemm_fwd": (xq, E4M3, wq, E4M3, xs, ws),
        "gemm_dgrad": (gq, E5M2, wq5.t().contiguous(), E5M2, gs, ws5),
        "gemm_wgrad": (gq.t().contiguous(), E5M2, xq5.t().contiguous(), E5M2, gs, xs5),
    }
    for name, (a, af, b, bf, sa, sb) in cases.items():
        m, k = a.shape
        n = b.shape[0]
        pre = hq.hq_preshuffle_weight(b)
        sets = [(a.clone(), pre.clone(), torch.empty((m, n), dtype=torch.bfloat16, device="cuda"))
                for _ in range(copies)]

        def glaunch(i, h, sets=sets, m=m, n=n, k=k, af=af, bf=bf, sa=sa, sb=sb):
            a_, p_, o_ = sets[i % copies]
            st = lib.hq_gemm_a8w8(P(a_.data_ptr()), af, P(p_.data_ptr()), bf, P(sa.data_ptr()), 1,
                                  P(sb.data_ptr()), 1, m, n, k, P(o_.data_ptr()), None, 0, h)
            assert st == 0, hq.hq_last_error()
        ms = time_graph(torch, glaunch, 2 * copies)
        fl = 2.0 * m * n * k
        out[name] = {"shape": f"{m}x{n}x{k} {'E4M3' if af == E4M3 else 'E5M2'}", "us": round(ms * 1e3, 3),
                     "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                     "frac_mfma": round(fl / (ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)}
        del sets
    return out


def vendor_yardstick(torch):
    """Context only, not part of the step: the vendor FP8 GEMM behind
    torch._scaled_mm (E4M3 operands, per-tensor scales of 1, bf16 output) on the
    GEMM shapes of the bench, graph-timed like this library's kernels over
    rotating operand and output sets larger than the Infinity Cache."""
    res = {"what": "torch._scaled_mm, float8_e4m3fn x float8_e4m3fn^T, scalar scales, bf16 out"}
    for (m, n, k) in [(4096, 4096, 4096), (8192, 2048, 1024), (2048, 4096, 1024), (2048, 1024, 4096),
                      (4096, 1024, 2048), (8192, 8192, 8192)]:
        nsets = max(2, min(8, int(600e6 // (m * k + n * k + 2 * m * n))))
        sets = [(torch.randn(m, k, device="cuda").to(torch.float8_e4m3fn),
                 torch.randn(n, k, device="cuda").to(torch.float8_e4m3fn),
                 torch.empty(m, n, dtype=torch.bfloat16, device="cuda")) for _ in range(nsets)]
        one = torch.ones((), device="cuda")

        def launch(i, h, sets=sets, one=one):
            a, b, o = sets[i % len(sets)]
            torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16, out=o)
        launch(0, None)  # the library's first call sets up state that graph capture does not allow
        torch.cuda.synchronize()
        ms = min(time_graph(torch, launch, 2 * nsets) for _ in range(3))
        res[f"{m}x{n}x{k}"] = {"us": round(ms * 1e3, 2), "tflops": round(2 * m * n * k / ms / 1e9, 1),
                               "rotating_sets": nsets}
        log(f"vendor yardstick {m}x{n}x{k}: {res[f'{m}x{n}x{k}']}")
        del sets
    return res


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def summarize(directory):
    """Markdown summary of a rocprofv3 run (--output-format csv): per-kernel
    statistics of a --kernel-trace --stats run and/or per-dispatch means of the
    counters of a --pmc run."""
    lines = []
    stats = _csv_rows(directory, "kernel_stats.csv")
    if stats:
        lines += ["| kernel | calls | average us | min us | max us | share % |", "|---|---:|---:|---:|---:|---:|"]
        for r in stats:
            lines.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f} |")
    counters = _csv_rows(directory, "counter_collection.csv")
    if counters:
        agg = {}
        for r in counters:
            key = (r["Kernel_Name"][:110], r["Counter_Name"])
            d = agg.setdefault(key, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        lines += ["", "| kernel | counter | dispatches | mean per dispatch |", "|---|---|---:|---:|"]
        for (k, c), d in sorted(agg.items()):
            lines.append(f"| `{k}` | {c} | {len(d)} | {sum(d.values()) / len(d):.1f} |")
    return "\n".join(lines)


def counter_mean(directory, counter, kernel_substr):
    """Mean per dispatch of `counter` over the dispatches whose kernel name
    contains `kernel_substr`."""
    per = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} under {directory}")
    return sum(per.values()) / len(per), len(per)


def write_traffic(name, kernel_substr, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """HBM bytes per launch of one kernel from FETCH_SIZE / WRITE_SIZE runs
    (KiB per dispatch), each scaled by what the same counter reads for the copy
    probe (COPY_PROBE_BYTES read and written per dispatch)."""
    fetch, nf = counter_mean(fetch_dir, "FETCH_SIZE", kernel_substr)
    write, nw = counter_mean(write_dir, "WRITE_SIZE", kernel_substr)
    cfetch, _ = counter_mean(copy_fetch_dir, "FETCH_SIZE", COPY_PROBE_KERNEL)
    cwrite, _ = counter_mean(copy_write_dir, "WRITE_SIZE", COPY_PROBE_KERNEL)
    f_read = COPY_PROBE_BYTES / (cfetch * 1024.0)
    f_write = COPY_PROBE_BYTES / (cwrite * 1024.0)
    read_b = fetch * 1024.0 * f_read
    write_b = write * 1024.0 * f_write
    out = {
        "kernel": kernel_substr,
        "source_hash": source_hash(),
        "fetch_kib_per_dispatch": round(fetch, 1), "fetch_dispatches": nf,
        "write_kib_per_dispatch": round(write, 1), "write_dispatches": nw,
        "copy_probe_fetch_kib": round(cfetch, 1), "copy_probe_write_kib": round(cwrite, 1),
        "read_scale": round(f_read, 5), "write_scale": round(f_write, 5),
        "read_bytes_per_launch": round(read_b), "write_bytes_per_launch": round(write_b),
        "bytes_per_launch": round(read_b + write_b),
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def trace_window(directory, kernel_substr, skip, count):
    """Mean / median duration (us) of dispatches skip .. skip+count-1, in
    dispatch order, of the kernels whose name contains `kernel_substr`, from a
    --kernel-trace run (selects one timing phase of this script)."""
    rows = [r for r in _csv_rows(directory, "kernel_trace.csv") if kernel_substr in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    sel = rows[skip:skip + count]
    if len(sel) < count:
        raise SystemExit(f"only {len(rows)} dispatches of {kernel_substr!r}")
    d = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel)
    return {"kernel": kernel_substr, "dispatches": f"{skip}..{skip + count - 1} of {len(rows)}",
            "mean_us": round(sum(d) / len(d), 3), "median_us": round(d[len(d) // 2], 3)}


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-window":
        print(json.dumps(trace_window(sys.argv[2], sys.argv[3], int(sys.argv[4]), int(sys.argv[5]))))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize":
        print(summarize(sys.argv[2]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--write-traffic":
        print(json.dumps(write_traffic(*sys.argv[2:8])))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The eager step settles after about 150 steps (10-step means from a fresh
    # process: 86, 88, 92, 94, 93, 92, 90, ... 84, 83 us), so the default warmup
    # runs past that before the timed steps.
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=8, help="input/output sets cycled to defeat the MALL")
    ap.add_argument("--kernel-reps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the decode / grouped / quantize-variant timings")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (PMC calibration) and exit")
    ap.add_argument("--grouped-only", action="store_true",
                    help="only run 10 launches of the grouped MoE GEMM (for the PMC traffic summary) and exit")
    ap.add_argument("--vendor-yardstick", action="store_true",
                    help="only time torch._scaled_mm (the vendor FP8 GEMM) on this library's GEMM shapes, as "
                         "context, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one MI355X; --gpus {args.gpus} is not supported (this library has no multi-GPU "
              "path; run it with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_dynamic_quantization_amd as hq
    import workloads

    if not os.path.exists(hq.LIB_PATH):
        from fp8_dynamic_quantization_amd import build as b
        b.build()
    lib = hq.load()
    torch.cuda.set_device(0)

    if args.copy_probe:
        # An elementwise kernel that reads 1 GiB and writes 1 GiB (a plain
        # memcpy may go to a DMA engine, which the shader counters miss).
        src = torch.zeros(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x bitwise_not over {COPY_PROBE_BYTES} bytes")
        return

    if args.grouped_only:
        moe = MoeSets(torch, hq, lib)
        h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(10):
            moe.launch(i, h)
        torch.cuda.synchronize()
        log("grouped MoE: 10 launches of hq_grouped_gemm_a8w8 over 5 rotating sets")
        return

    if args.vendor_yardstick:
        print(json.dumps(vendor_yardstick(torch)))
        return

    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    log("generating inputs ...")
    x_bits, w_bits = workloads.ptpc_square(1)
    pre_bytes = hq.hq_preshuffled_bytes(N, K)
    sets = [Buffers(torch, x_bits, w_bits, pre_bytes) for _ in range(args.rotate)]
    ops, two_launch = make_ops(hq, lib, stream)

    def same_traffic(b, h):  # h unused: inside the graph capture torch's current stream is h
        halves = b.x.view(torch.uint8).view(2, M * K)
        torch.bitwise_xor(halves[0], halves[1], out=b.xq.view(-1))

    def step(i):
        b = sets[i % len(sets)]
        for fn in ops.values():
            fn(b)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    log(f"step: {ms_step * 1e3:.1f} us")

    # Per-kernel durations: each kernel launched back to back over the rotating
    # sets inside a HIP graph on a side stream, bracketed by HIP events on that
    # stream (no host launch overhead, no event between launches).
    kms, warm_replays = {}, {}
    for name, fn in {**ops, **two_launch}.items():
        def launch(i, h, fn=fn):
            fn(sets[i % len(sets)], h)
        info = {}
        kms[name] = time_graph(torch, launch, 2 * len(sets), info=info)
        warm_replays[name] = info["untimed_replays"]
    for name, ms in kms.items():
        log(f"  {name}: {ms * 1e3:.2f} us")
    quant_bytes = M * K * 2 + M * K + M * 4 * 2      # bf16 in, codes out, scale + amax out
    pre_alg_bytes = N * K + pre_bytes
    qwp_bytes = N * K * 2 + pre_bytes + N * 4 * 2   # bf16 in, pre-shuffled codes out, scale + amax out
    gemm_tflops = flops / (kms["gemm"] * 1e-3) / 1e12
    quant_gbs = quant_bytes / (kms["quant_x"] * 1e-3) / 1e9

    # practical HBM ceiling: an elementwise read+write pass over 2 x 512 MiB
    src = torch.zeros(1 << 29, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = time_kernel(torch, lambda _: torch.bitwise_not(src, out=dst), [None], 5)
    copy_gbs = 2 * src.numel() / (copy_ms * 1e-3) / 1e9
    log(f"  copy probe: {copy_gbs:.0f} GB/s")
    del src, dst
    # the quantize's own traffic without its arithmetic: the 2 bytes of each
    # element read, one byte written (torch's vectorised elementwise xor of the
    # two halves of X's bytes into the code buffer), over the same rotating
    # sets; a practical ceiling for a pass of this size
    # The whole step (quantize X, quantize W into the pre-shuffled layout, GEMM)
    # as one graph of 16 steps over the rotating sets, timed like the kernels:
    # its device time per step beside the eager loop's and the kernels' sum.
    def step_launch(i, h):
        b = sets[i % len(sets)]
        for fn in ops.values():
            fn(b, h)
    step_graph_ms = time_graph(torch, step_launch, 2 * len(sets))
    log(f"  step as one graph: {step_graph_ms * 1e3:.2f} us")
    same_ms = time_graph(torch, lambda i, h: same_traffic(sets[i % len(sets)], h), 2 * len(sets))
    same_gbs = (M * K * 3) / (same_ms * 1e-3) / 1e9
    log(f"  same-traffic probe: {same_ms * 1e3:.2f} us = {same_gbs:.0f} GB/s")
    # the same bytes in the per-token kernel's own access pattern: the
    # hand-written row-streaming probe (one wavefront per row, 16-byte loads,
    # the next row's loads in flight, non-temporal 8-byte stores), at that
    # kernel's grid and at three others
    row_probe = {}
    for wpc in ROW_PROBE_WAVES_PER_CU:
        def plaunch(i, h, wpc=wpc):
            b = sets[i % len(sets)]
            st = lib.hq_stream_rows_probe(b.p["x"], M, 2 * K, wpc * NUM_CUS, b.p["xq"], h)
            assert st == 0, hq.hq_last_error()
        row_probe[wpc] = time_graph(torch, plaunch, 2 * len(sets))
    probe_ms = row_probe[QUANT_ROW_WAVES_PER_CU]
    log("  row-streaming probe: " + ", ".join(f"{w}/CU {v * 1e3:.2f} us" for w, v in row_probe.items()))
    other = None if args.no_other else other_workloads(torch, hq, lib, args.kernel_reps)
    if other:
        log(json.dumps(other))
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (E4M3 codes, fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {
            "workload": "PTPC square: X bf16 [4096,4096] N(0,1) with 0.1% of entries x50, W bf16 [4096,4096] "
                        "N(0,0.02^2); per-token X, per-output-channel W, E4M3; GEMM M=N=K=4096 -> bf16",
            "step": "quantize X per token + quantize W per output channel straight into the pre-shuffled "
                    "layout (hq_quantize_fp8_preshuffled: the codes and layout of per-token quantize + "
                    "pre-shuffle in one pass) + GEMM",
            "m": M, "n": N, "k": K, "rotating_sets": args.rotate,
        },
        "roofline": {
            "kernel": "gemm (hq_gemm_a8w8)",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
            "traffic": traffic_from_profile("gemm_ptpc4096"),
        },
        "kernels_us": {k: round(v * 1e3, 3) for k, v in kms.items()},
        "step_graph": {"us": round(step_graph_ms * 1e3, 3),
                       "tflops": round(flops / (step_graph_ms * 1e-3) / 1e12, 2),
                       "sum_of_step_kernels_us": round(sum(kms[k] for k in ops) * 1e3, 3),
                       "what": "the step's three launches captured as one HIP graph of 16 steps over the rotating "
                               "sets, timed like the kernels (device time per step, no host launch overhead)"},
        "kernel_timing": {"method": "HIP graph of launches over the rotating sets on torch's current stream, "
                                    "HIP events around the timed replays",
                          "launches_per_replay": 2 * args.rotate,
                          "untimed_replays": {"min_ms": GRAPH_WARM_MS, "count": warm_replays}, "timed_replays": 5,
                          "step_loop_launches_per_kernel": args.warmup + args.steps},
        "quantize": {
            "kernel": "per-token quantize of X (hq_quantize_fp8)",
            "bound": "hbm",
            "achieved": round(quant_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(quant_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": quant_bytes,
            "traffic": traffic_from_profile("quant_rows_ptpc4096"),
            "same_traffic_probe": {"us": round(same_ms * 1e3, 3), "gbs": round(same_gbs, 1),
                                   "what": "the 32 MiB of X read, 16 MiB written (torch elementwise xor of the "
                                           "two halves of X's bytes), same rotating sets",
                                   "quantize_frac_of_probe": round(same_ms / kms["quant_x"], 4)},
            "row_probe": {"us": round(probe_ms * 1e3, 3),
                          "gbs": round(M * K * 3 / (probe_ms * 1e-3) / 1e9, 1),
                          "waves_per_cu": QUANT_ROW_WAVES_PER_CU,
                          "what": "hq_stream_rows_probe: X's 32 MiB read and 16 MiB written with the per-token "
                                  "kernel's access pattern and grid, without its arithmetic",
                          "quantize_frac_of_probe": round(probe_ms / kms["quant_x"], 4),
                          "us_by_waves_per_cu": {str(w): round(v * 1e3, 3) for w, v in row_probe.items()}},
        },
        "quant_w_pre": {
            "kernel": "per-output-channel quantize of W into the pre-shuffled layout (hq_quantize_fp8_preshuffled)",
            "bound": "hbm",
            "achieved": round(qwp_bytes / (kms["quant_w_pre"] * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(qwp_bytes / (kms["quant_w_pre"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": qwp_bytes,
            "two_launch_us": round((kms["quant_w"] + kms["preshuffle"]) * 1e3, 3),
            "traffic": traffic_from_profile("quant_rows_pre_ptpc4096"),
        },
        "preshuffle_gbs": round(pre_alg_bytes / (kms["preshuffle"] * 1e-3) / 1e9, 1),
        "copy_probe_gbs": round(copy_gbs, 1),
        "other_workloads": other,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
