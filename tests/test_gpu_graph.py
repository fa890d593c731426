"""The hot path's entry points recorded once in a HIP graph and replayed.

Each replay must reproduce the oracle: the kernels keep no state outside the
caller's buffers except the workspace counters and barrier words, which every
call leaves ready for the next, and they record no memset. Between replays the
outputs are overwritten eagerly and the device synchronised, so a replay that
wrote nothing, or wrote stale values, fails. The delayed-scaling ring advances
once per replay, as the same call made eagerly would."""
import numpy as np
import pytest
import torch

import workloads
from oracle import fp8, preshuffle as P, quantize as Q
from tests.gpu_helpers import allowed_share, check_gemm, dev_bf16, host, require_gpu

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def hq():
    return require_gpu()


def _bf16(rng, shape, std=1.0):
    bits = workloads.random_bf16(rng, shape, std)
    return bits, dev_bf16(bits)


def test_quantize_and_gemm_graph_replays(hq):
    rng = np.random.default_rng(21)
    E4M3 = fp8.E4M3
    # per-token X and per-row W into the pre-shuffled layout, then the GEMM
    xb, x = _bf16(rng, (640, 1024))
    wb, w = _bf16(rng, (768, 1024), 0.02)
    # per-tensor and per-channel with their workspace (single-pass barrier kernels)
    tb, t = _bf16(rng, (512, 2048))
    cb, c = _bf16(rng, (1024, 512))
    # decode GEMM with a split-K workspace
    db, d = _bf16(rng, (8, 14336))
    vb, v = _bf16(rng, (1024, 14336), 0.02)
    # delayed scaling
    rb, rx = _bf16(rng, (256, 1024))

    lib = hq.load()
    dev = "cuda"
    qx = torch.empty((640, 1024), dtype=torch.uint8, device=dev)
    sx = torch.empty(640, dtype=torch.float32, device=dev)
    ax = torch.empty_like(sx)
    wpre = torch.empty(int(lib.hq_preshuffled_bytes(768, 1024)), dtype=torch.uint8, device=dev)
    sw = torch.empty(768, dtype=torch.float32, device=dev)
    aw = torch.empty_like(sw)
    out = torch.empty((640, 768), dtype=torch.bfloat16, device=dev)
    qt = torch.empty((512, 2048), dtype=torch.uint8, device=dev)
    st_ = torch.empty(1, dtype=torch.float32, device=dev)
    at_ = torch.empty_like(st_)
    ws_t = torch.zeros(int(lib.hq_quantize_workspace_bytes(Q.PER_TENSOR, 512, 2048)), dtype=torch.uint8, device=dev)
    qc = torch.empty((1024, 512), dtype=torch.uint8, device=dev)
    sc = torch.empty(512, dtype=torch.float32, device=dev)
    ac = torch.empty_like(sc)
    ws_c = torch.zeros(int(lib.hq_quantize_workspace_bytes(Q.PER_CHANNEL, 1024, 512)), dtype=torch.uint8, device=dev)
    # decode operands are quantized once, eagerly; the graph holds the decode GEMM
    qd, sd, _ = hq.hq_quantize_fp8(d, E4M3, Q.PER_TOKEN)
    vpre, sv, _, qv = hq.hq_quantize_fp8_preshuffled(v, E4M3, row_major=True)
    ws_g = torch.zeros(int(lib.hq_gemm_workspace_bytes(8, 1024, 14336)), dtype=torch.uint8, device=dev)
    assert ws_g.numel() > 0, "the decode shape is meant to run split"
    od = torch.empty((8, 1024), dtype=torch.bfloat16, device=dev)
    ring = hq.Ring(16)
    qr = torch.empty((256, 1024), dtype=torch.uint8, device=dev)
    sr = torch.empty(1, dtype=torch.float32, device=dev)
    ar = torch.empty_like(sr)
    torch.cuda.synchronize()

    def calls():
        hq.hq_quantize_fp8(x, E4M3, Q.PER_TOKEN, q=qx, scale_out=sx, amax_out=ax)
        hq.hq_quantize_fp8_preshuffled(w, E4M3, q_pre=wpre, scale_out=sw, amax_out=aw)
        hq.hq_gemm_a8w8(qx, E4M3, wpre, E4M3, sx, sw, 768, out=out)
        hq.hq_quantize_fp8(t, E4M3, Q.PER_TENSOR, q=qt, scale_out=st_, amax_out=at_, workspace=ws_t)
        hq.hq_quantize_fp8(c, E4M3, Q.PER_CHANNEL, q=qc, scale_out=sc, amax_out=ac, workspace=ws_c)
        hq.hq_gemm_a8w8(qd, E4M3, vpre, E4M3, sd, sv, 1024, out=od, workspace=ws_g)
        hq.hq_quantize_fp8(rx, E4M3, Q.PER_TENSOR, ring=ring, ring_idx=3, q=qr, scale_out=sr, amax_out=ar,
                           workspace=ws_t)

    # one eager pass first (on the capture stream, as before any capture), then the capture
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.synchronize()
    state0 = host(ring.state).copy()  # the ring after the eager pass; the replays continue from it
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            calls()
    torch.cuda.synchronize()

    # oracle
    qx_ref, sx_ref, _ = Q.quantize_dynamic(xb, Q.BF16, E4M3, Q.PER_TOKEN)
    qw_ref, sw_ref, _ = Q.quantize_dynamic(wb, Q.BF16, E4M3, Q.PER_TOKEN)
    qt_ref, st_ref, _ = Q.quantize_dynamic(tb, Q.BF16, E4M3, Q.PER_TENSOR)
    qc_ref, sc_ref, _ = Q.quantize_dynamic(cb, Q.BF16, E4M3, Q.PER_CHANNEL)
    assert np.array_equal(state0.view(np.uint32), host(ring.state).view(np.uint32)), "capture ran the ring"
    state = state0
    ring_refs = []
    for _ in range(REPLAYS):
        q_r, s_r, _, state, _ = Q.quantize_delayed(rb, Q.BF16, E4M3, state, 3, 0)
        ring_refs.append((q_r, s_r, state.copy()))
    pre_ref = P.preshuffle(qw_ref)
    qd_h, sd_h, qv_h, sv_h = host(qd), host(sd), host(qv), host(sv)
    prng = np.random.default_rng(5)
    pairs = np.stack([prng.integers(0, 640, 3000), prng.integers(0, 768, 3000)], axis=1)
    dpairs = np.stack([prng.integers(0, 8, 2000), prng.integers(0, 1024, 2000)], axis=1)

    first = None
    for rep in range(REPLAYS):
        for buf in (qx, wpre, qt, qc, qr):
            buf.fill_(0x5A)
        for buf in (out, od):
            buf.view(torch.int16).fill_(0x7FC1)
        for buf in (sx, sw, st_, sc, sr):
            buf.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(qx), qx_ref) and np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))
        assert np.array_equal(host(wpre), pre_ref) and np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
        assert np.array_equal(host(qt), qt_ref) and np.array_equal(host(st_).view(np.uint32), st_ref.view(np.uint32))
        assert np.array_equal(host(qc), qc_ref) and np.array_equal(host(sc).view(np.uint32), sc_ref.view(np.uint32))
        q_r, s_r, state_r = ring_refs[rep]
        assert np.array_equal(host(qr), q_r), f"replay {rep}: delayed codes"
        assert np.array_equal(host(sr).view(np.uint32), s_r.view(np.uint32)), f"replay {rep}: delayed scale"
        assert np.array_equal(host(ring.state).view(np.uint32), state_r.view(np.uint32)), f"replay {rep}: ring"
        ob, odb = host(out), host(od)
        check_gemm(ob, qx_ref, E4M3, qw_ref, E4M3, sx_ref, sw_ref, pairs=pairs,
                   max_strict_frac=allowed_share("graph gemm", len(pairs)), label="graph gemm")
        check_gemm(odb, qd_h, E4M3, qv_h, E4M3, sd_h, sv_h, pairs=dpairs,
                   max_strict_frac=allowed_share("graph decode", len(dpairs)), label="graph decode")
        if first is None:
            first = (ob.copy(), odb.copy())
        else:  # the GEMMs' sums are in a fixed order: replays agree bit for bit
            assert np.array_equal(ob, first[0]) and np.array_equal(odb, first[1])
    # the workspaces are left ready for eager calls after the replays
    q2, s2, _ = hq.hq_quantize_fp8(t, E4M3, Q.PER_TENSOR, workspace=ws_t)
    o2 = hq.hq_gemm_a8w8(qd, E4M3, vpre, E4M3, sd, sv, 1024, workspace=ws_g)
    torch.cuda.synchronize()
    assert np.array_equal(host(q2), qt_ref) and np.array_equal(host(o2), first[1])
