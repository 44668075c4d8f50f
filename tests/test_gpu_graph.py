"""The hot path captured in a HIP graph replays to the same bytes as eager calls.

One delayed-scaling step plus the 1x128 quantize and block-scaled GEMM is
captured once, then replayed several times with eager work between the
replays (the input is changed in place, so each replay sees a new amax and
scale).  After every replay the graph's outputs and scaler state must equal,
byte for byte, those of the same calls made eagerly on a second set of
buffers.  The library records no memset nodes: every reset is a kernel.
"""
import pytest
import torch

from block_scaled_precision_amax_amd import workloads as W

pytestmark = pytest.mark.gpu

E4, E5 = 0, 1


def test_graph_replay_matches_eager(fq, gpu):
    dev = gpu
    R, Cc = 1024, 1024
    M, N, K = 256, 384, 1024
    n = R * Cc
    x = W.delayed_step(R, Cc, 3.0, seed=901, device=dev)
    X = W.activation(M, K, seed=902, factor=1e3, dtype=torch.bfloat16, device=dev)
    w = W.weight(N, K, seed=903, device=dev)
    qW = torch.empty(N, K, dtype=torch.uint8, device=dev)
    sW = torch.empty(N // 128, K // 128, dtype=torch.float32, device=dev)
    fq.fp8q_quantize_128x128(w, N, K, K, E4, 1e-12, qW, K, sW, K // 128)

    def buffers():
        b = {
            "st": torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev),
            "am": torch.zeros(1, dtype=torch.float32, device=dev),
            "q": torch.empty(n, dtype=torch.uint8, device=dev),
            "qX": torch.empty(M, K, dtype=torch.uint8, device=dev),
            "sX": torch.empty(M, K // 128, dtype=torch.float32, device=dev),
            "C": torch.empty(M, N, dtype=torch.bfloat16, device=dev),
        }
        fq.fp8q_delayed_scaler_init(b["st"], 16, 448.0, 1e-12, 1.0)
        return b

    def step(b):
        sc = b["st"].data_ptr() + fq.SCALER_SCALE_OFFSET
        fq.fp8q_quantize_tensor(x, n, E4, sc, b["q"], b["am"])
        fq.fp8q_delayed_scaler_update(b["st"], b["am"])
        fq.fp8q_quantize_1x128(X, M, K, K, E4, 1e-12, b["qX"], K, b["sX"], K // 128)
        fq.fp8q_gemm_blockscaled(b["qX"], E4, K, b["sX"], K // 128, 1, qW, E4, K, sW, 2, K // 128, 1, b["C"], N,
                                 M, N, K)

    bg, be = buffers(), buffers()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        step(bg)
    for rep in range(4):
        gr.replay()
        torch.cuda.synchronize()
        step(be)
        torch.cuda.synchronize()
        for k in bg:
            a = bg[k].view(torch.uint8) if bg[k].dtype != torch.uint8 else bg[k]
            e = be[k].view(torch.uint8) if be[k].dtype != torch.uint8 else be[k]
            assert torch.equal(a, e), f"replay {rep}: {k} differs from the eager result"
        # eager work between replays: a new input magnitude for the next step
        x.mul_(1.75)
        X.mul_(-0.5)
        torch.cuda.synchronize()


def test_graph_replay_mx_and_fused_epilogue(fq, gpu):
    """MX quantize + MX GEMM, the GEMM with the 1x128 epilogue and an EMA
    scaler step, captured once and replayed against eager calls, with the
    inputs changed in place between replays."""
    dev = gpu
    M, N, K = 256, 384, 1024
    X = W.activation(M, K, seed=911, factor=1e3, dtype=torch.bfloat16, device=dev)
    w = W.weight(N, K, seed=912, device=dev)
    qW = torch.empty(N, K, dtype=torch.uint8, device=dev)
    sW = torch.empty(N // 128, K // 128, dtype=torch.float32, device=dev)
    fq.fp8q_quantize_128x128(w, N, K, K, E4, 1e-12, qW, K, sW, K // 128)
    qWm = torch.empty(N, K, dtype=torch.uint8, device=dev)
    sWm = torch.empty(N, K // 32, dtype=torch.uint8, device=dev)
    fq.fp8q_quantize_mx(w, N, K, K, E4, qWm, K, sWm, K // 32)
    x = W.delayed_step(512, 1024, 2.0, seed=913, device=dev)

    def buffers():
        b = {
            "qm": torch.empty(M, K, dtype=torch.uint8, device=dev),
            "sm": torch.empty(M, K // 32, dtype=torch.uint8, device=dev),
            "Cm": torch.empty(M, N, dtype=torch.bfloat16, device=dev),
            "qX": torch.empty(M, K, dtype=torch.uint8, device=dev),
            "sX": torch.empty(M, K // 128, dtype=torch.float32, device=dev),
            "qC": torch.empty(M, N, dtype=torch.uint8, device=dev),
            "sC": torch.empty(M, N // 128, dtype=torch.float32, device=dev),
            "st": torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev),
            "am": torch.zeros(1, dtype=torch.float32, device=dev),
            "q": torch.empty(x.numel(), dtype=torch.uint8, device=dev),
        }
        fq.fp8q_delayed_scaler_init_stat(b["st"], 4, 448.0, 1e-12, 1.0, fq.STAT_EMA, 0.25)
        return b

    def step(b):
        fq.fp8q_quantize_mx(X, M, K, K, E4, b["qm"], K, b["sm"], K // 32)
        fq.fp8q_gemm_mx(b["qm"], E4, K, b["sm"], K // 32, qWm, E4, K, sWm, K // 32, b["Cm"], N, M, N, K)
        fq.fp8q_quantize_1x128(X, M, K, K, E4, 1e-12, b["qX"], K, b["sX"], K // 128)
        fq.fp8q_gemm_blockscaled_q(b["qX"], E4, K, b["sX"], K // 128, 1, qW, E4, K, sW, 2, K // 128, 1, E4, 1e-12,
                                   b["qC"], N, b["sC"], N // 128, M, N, K)
        sc = b["st"].data_ptr() + fq.SCALER_SCALE_OFFSET
        fq.fp8q_quantize_tensor(x, x.numel(), E4, sc, b["q"], b["am"])
        fq.fp8q_delayed_scaler_update(b["st"], b["am"])

    bg, be = buffers(), buffers()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        step(bg)
    for rep in range(4):
        gr.replay()
        torch.cuda.synchronize()
        step(be)
        torch.cuda.synchronize()
        for k in bg:
            a = bg[k].view(torch.uint8) if bg[k].dtype != torch.uint8 else bg[k]
            e = be[k].view(torch.uint8) if be[k].dtype != torch.uint8 else be[k]
            assert torch.equal(a, e), f"replay {rep}: {k} differs from the eager result"
        X.mul_(-1.5)
        x.mul_(0.5)
        torch.cuda.synchronize()


def test_graph_replay_two_streams(fq, gpu):
    """The bench's step shape: the activation quantize, then a fork of the
    delayed-scaling kernels onto a second stream beside the GEMM, joined
    before the step ends; captured once and replayed against eager calls on
    one stream."""
    dev = gpu
    M, N, K = 256, 384, 1024
    X = W.activation(M, K, seed=921, factor=1e3, dtype=torch.bfloat16, device=dev)
    w = W.weight(N, K, seed=922, device=dev)
    qW = torch.empty(N, K, dtype=torch.uint8, device=dev)
    sW = torch.empty(N // 128, K // 128, dtype=torch.float32, device=dev)
    fq.fp8q_quantize_128x128(w, N, K, K, E4, 1e-12, qW, K, sW, K // 128)
    x = W.delayed_step(512, 1024, 3.0, seed=923, device=dev)
    g = W.gradient(512, 1024, seed=924, dtype=torch.bfloat16, device=dev)
    n = x.numel()

    def buffers():
        b = {
            "stx": torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev),
            "stg": torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev),
            "amx": torch.zeros(1, dtype=torch.float32, device=dev),
            "amg": torch.zeros(1, dtype=torch.float32, device=dev),
            "qx": torch.empty(n, dtype=torch.uint8, device=dev),
            "xh": torch.empty(n, dtype=torch.bfloat16, device=dev),
            "qg": torch.empty(n, dtype=torch.uint8, device=dev),
            "qX": torch.empty(M, K, dtype=torch.uint8, device=dev),
            "sX": torch.empty(M, K // 128, dtype=torch.float32, device=dev),
            "C": torch.empty(M, N, dtype=torch.bfloat16, device=dev),
        }
        fq.fp8q_delayed_scaler_init(b["stx"], 4, 448.0, 1e-12, 1.0)
        fq.fp8q_delayed_scaler_init(b["stg"], 4, 57344.0, 1e-12, 1.0)
        return b

    side = torch.cuda.Stream()

    def step(b, fork):
        fq.fp8q_quantize_1x128(X, M, K, K, E4, 1e-12, b["qX"], K, b["sX"], K // 128)
        join = None
        if fork:
            ev = torch.cuda.Event()
            ev.record()
            side.wait_event(ev)
        with torch.cuda.stream(side if fork else torch.cuda.current_stream()):
            scx = b["stx"].data_ptr() + fq.SCALER_SCALE_OFFSET
            scg = b["stg"].data_ptr() + fq.SCALER_SCALE_OFFSET
            fq.fp8q_quantize_tensor_dq(x, n, E4, scx, b["qx"], b["xh"], b["amx"])
            fq.fp8q_quantize_tensor(g, n, E5, scg, b["qg"], b["amg"])
            fq.fp8q_delayed_scaler_update(b["stx"], b["amx"])
            fq.fp8q_delayed_scaler_update(b["stg"], b["amg"])
            if fork:
                join = torch.cuda.Event()
                join.record()
        fq.fp8q_gemm_blockscaled(b["qX"], E4, K, b["sX"], K // 128, 1, qW, E4, K, sW, 2, K // 128, 1, b["C"], N,
                                 M, N, K)
        if fork:
            torch.cuda.current_stream().wait_event(join)

    bg, be = buffers(), buffers()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        step(bg, True)
    for rep in range(5):
        gr.replay()
        torch.cuda.synchronize()
        step(be, False)
        torch.cuda.synchronize()
        for k in bg:
            a = bg[k].view(torch.uint8) if bg[k].dtype != torch.uint8 else bg[k]
            e = be[k].view(torch.uint8) if be[k].dtype != torch.uint8 else be[k]
            assert torch.equal(a, e), f"replay {rep}: {k} differs from the eager result"
        x.mul_(1.5)
        g.mul_(0.25)
        X.mul_(-2.0)
        torch.cuda.synchronize()
