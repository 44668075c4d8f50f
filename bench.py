#!/usr/bin/env python3
"""Benchmark of the FP8 quantize + block-scaled GEMM hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
  1. a delayed-scaling step on bf16 8192x8192 tensors: the activation copy
     x_t (sigma_t * N(0,1), sigma_t log-uniform in [0.5, 50]) quantized to
     E4M3FN and the gradient copy g_t (|g| log-uniform in [1e-6, 1e-2])
     quantized to E5M2, each with the scale of the previous steps (window
     16) and the amax fused into the same pass, the x_t codes dequantized
     back to bf16, then both scalers updated;
  2. the LLM-layer fused path: bf16 activations 16384x7168 (N(0,1), four
     outlier columns x1e3) quantized 1x128 to E4M3FN, times the E4M3FN
     weight 18432x7168 with 128x128 scales (quantized once, untimed), fp32
     accumulation promoted every 128 K, bf16 output.
Inputs rotate over several buffers so repeated reads are not served from
the 256 MB last-level cache.

`value` is the step's throughput in TFLOP/s: the layer GEMM's 2*M*N*K per
step over the step time.  All launches are captured into HIP graphs and
replayed (one graph per input rotation), so host launch costs stay out of
the timings; per-kernel figures (GB/s for the quantizers, TFLOP/s for the
GEMM, each with its roofline fraction) come from graphs of repeated
launches of one kernel, timed with events on the replay stream.
`cpu_baseline` times the CPU oracle on a bounded sample of the same step
and extrapolates per unit.
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (the exact GEMM path's matrix instructions)

# workload sizes
DS_ROWS = DS_COLS = 8192        # delayed-scaling tensors
LM, LN, LK = 16384, 18432, 7168  # LLM layer: X [M,K] bf16, W [N,K], C [M,N] bf16
WINDOW = 16
N_ROT = 8                        # rotating delayed-scaling buffers per tensor
X_ROT = 2
COPY_ELEMS = 1 << 28             # fp32 copy reference: 1 GiB read + 1 GiB written

# HBM bytes per GEMM launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE counter
# passes over this same command, scaled by what the counters read for the
# copy reference; valid only for the kernel source the counters were taken on.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_blockscaled_16384x18432x7168_hbm_traffic.md")
# MFMA-pipe busy fraction of the same kernel from one rocprofv3 counter pass
# (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE cycles x 1024 SIMDs), with the
# same validity rule.
MFMA_SUMMARY = os.path.join(ROOT, "profiles", "gemm_blockscaled_16384x18432x7168_mfma_counters.md")
GEMM_SOURCES = ("block_scaled_precision_amax_amd/csrc/fp8q_gemm.hip",
                "block_scaled_precision_amax_amd/csrc/fp8q_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic():
    n = DS_ROWS * DS_COLS
    nx = LM * LK
    return {
        "quantize_tensor_bytes": n * 2 + n + 4,            # bf16 read, codes written, amax
        "dequantize_bytes": n + 2 * n + 4,                  # codes read, bf16 written, scale
        "quantize_dq_bytes": 2 * n + n + 2 * n + 4,         # bf16 read, codes and bf16 round trip written
        "quantize_1x128_bytes": nx * 2 + nx + 4 * nx // 128,  # bf16 read, codes + scales written
        "quantize_mx_bytes": nx * 2 + nx + nx // 32,     # bf16 in, codes + E8M0 bytes (same for dequantize)
        "gemm_flop": 2 * LM * LN * LK,
        # codes of A and B, their scales, bf16 C
        "gemm_bytes": LM * LK + LN * LK + 4 * (LM * (LK // 128) + (LN // 128) * (LK // 128)) + 2 * LM * LN,
    }


def gemm_source_sha256() -> str:
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_field(path, name, kind):
    """A field of a committed counter summary, or None when the summary is
    missing or was taken on different GEMM source."""
    try:
        with open(path) as f:
            fields = dict(re.findall(r"^- (\w+): (\S+)\s*$", f.read(), re.M))
    except OSError:
        return None
    if fields.get("source_sha256") != gemm_source_sha256() or name not in fields:
        return None
    return kind(fields[name])


def measured_traffic():
    """Counter-measured HBM bytes per GEMM launch (or None)."""
    return counter_field(TRAFFIC_SUMMARY, "traffic_bytes_per_launch", int)


def run_gpu(steps: int, warmup: int):
    import torch

    import block_scaled_precision_amax_amd as fq
    from block_scaled_precision_amax_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = DS_ROWS * DS_COLS
    log("building inputs ...")
    sig = W.sigma_schedule(64, seed=2)
    xs = [W.delayed_step(DS_ROWS, DS_COLS, sig[i], seed=200 + i, device=dev) for i in range(N_ROT)]
    gs = [W.gradient(DS_ROWS, DS_COLS, seed=300 + i, device=dev, dtype=torch.bfloat16) for i in range(N_ROT)]
    Xs = [W.activation(LM, LK, seed=4 + 10 * i, factor=1e3, dtype=torch.bfloat16, device=dev) for i in range(X_ROT)]
    w32 = W.weight(LN, LK, seed=40, device=dev)
    qW = torch.empty(LN, LK, dtype=torch.uint8, device=dev)
    sW = torch.empty(LN // 128, LK // 128, dtype=torch.float32, device=dev)
    fq.fp8q_quantize_128x128(w32, LN, LK, LK, fq.E4M3FN, 1e-12, qW, LK, sW, LK // 128)
    del w32
    qx = torch.empty(n, dtype=torch.uint8, device=dev)
    qg = torch.empty(n, dtype=torch.uint8, device=dev)
    xhat = torch.empty(n, dtype=torch.bfloat16, device=dev)
    qX = torch.empty(LM, LK, dtype=torch.uint8, device=dev)
    sX = torch.empty(LM, LK // 128, dtype=torch.float32, device=dev)
    C = torch.empty(LM, LN, dtype=torch.bfloat16, device=dev)
    st_x = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev)
    st_g = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev)
    fq.fp8q_delayed_scaler_init(st_x, WINDOW, 448.0, 1e-12, 1.0)
    fq.fp8q_delayed_scaler_init(st_g, WINDOW, 57344.0, 1e-12, 1.0)
    sc_x = st_x.data_ptr() + fq.SCALER_SCALE_OFFSET
    sc_g = st_g.data_ptr() + fq.SCALER_SCALE_OFFSET
    torch.cuda.synchronize()

    # The delayed-scaling kernels (HBM-bound) and the layer's quantize + GEMM
    # (MFMA-bound) share no buffer, so the step forks the former onto a
    # second stream (default priority) and joins it before the step ends.
    side = torch.cuda.Stream()

    def step(t: int):
        x, g, X = xs[t % N_ROT], gs[t % N_ROT], Xs[t % X_ROT]
        fq.fp8q_quantize_1x128(X, LM, LK, LK, fq.E4M3FN, 1e-12, qX, LK, sX, LK // 128)
        # fork after the (HBM-bound) activation quantize, so that the
        # delayed-scaling kernels overlap the GEMM rather than compete with it
        fork = torch.cuda.Event()
        fork.record()
        side.wait_event(fork)
        with torch.cuda.stream(side):
            # x's codes and their bf16 round trip in one pass, g's codes, each
            # with its scaler's scale and its amax folded into the scaler
            fq.fp8q_quantize_tensor_delayed(x, n, fq.E4M3FN, st_x, qx, xhat)
            fq.fp8q_quantize_tensor_delayed(g, n, fq.E5M2, st_g, qg)
            fq.fp8q_delayed_scaler_update(st_x)
            fq.fp8q_delayed_scaler_update(st_g)
            join = torch.cuda.Event()
            join.record()
        fq.fp8q_gemm_blockscaled(qX, fq.E4M3FN, LK, sX, LK // 128, 1, qW, fq.E4M3FN, LK, sW, fq.GRAN_128x128,
                                 LK // 128, 1, C, LN, LM, LN, LK)
        torch.cuda.current_stream().wait_event(join)

    # Every launch is captured into HIP graphs and replayed: a Python launch
    # costs about as much host time as one of the quantizer kernels runs, so
    # eager launches would measure the host.  One graph per input rotation.
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        step(0)  # one eager pass before capture
    torch.cuda.synchronize()
    period = N_ROT  # multiple of X_ROT
    graphs = []
    for t in range(period):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap):
            step(t)
        graphs.append(gr)

    def E():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    log(f"warmup {warmup} steps ...")
    for t in range(warmup):
        graphs[t % period].replay()
    torch.cuda.synchronize()
    log(f"timing {steps} steps ...")
    t0 = time.perf_counter()
    e0 = E()
    for t in range(warmup, warmup + steps):
        graphs[t % period].replay()
    e1 = E()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1) / steps

    # per-kernel averages: a graph of `reps` launches of one kernel, replayed
    def per_launch(launch, reps):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap):
            for r in range(reps):
                launch(r)
        gr.replay()
        torch.cuda.synchronize()
        a = E()
        gr.replay()
        b = E()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    log("per-kernel timing ...")
    am_tmp = torch.zeros(1, dtype=torch.float32, device=dev)
    st_tmp = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev)
    fq.fp8q_delayed_scaler_init(st_tmp, WINDOW, 448.0, 1e-12, 1.0)
    # the other window statistics, at the longest window
    st_mean = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev)
    fq.fp8q_delayed_scaler_init_stat(st_mean, 1024, 448.0, 1e-12, 1.0, fq.STAT_MEAN)
    st_ema = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev)
    fq.fp8q_delayed_scaler_init_stat(st_ema, 1024, 448.0, 1e-12, 1.0, fq.STAT_EMA, 0.01)
    # dequantizer inputs and outputs rotate over N_ROT sets (1.5 GiB in all),
    # so that no launch finds its codes in the 256 MB last-level cache
    qxs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(N_ROT)]
    xhats = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(N_ROT)]
    for i in range(N_ROT):
        fq.fp8q_quantize_tensor(xs[i], n, fq.E4M3FN, sc_x, qxs[i])
    # the quantizer rows write their codes (and round trips) to rotating
    # outputs as well, so that no launch writes into lines a previous launch
    # left in the last-level cache
    qos = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(N_ROT)]
    X_OUT = 3
    qXos = [torch.empty(LM, LK, dtype=torch.uint8, device=dev) for _ in range(X_OUT)]
    per = {
        # the step's per-tensor quantizers: scale and amax accumulator in the scaler
        "quantize_tensor_x": per_launch(lambda r: fq.fp8q_quantize_tensor_delayed(xs[r % N_ROT], n, fq.E4M3FN, st_tmp,
                                                                                  qos[r % N_ROT]), 16),
        "quantize_tensor_g": per_launch(lambda r: fq.fp8q_quantize_tensor_delayed(gs[r % N_ROT], n, fq.E5M2, st_tmp,
                                                                                  qos[r % N_ROT]), 16),
        "quantize_tensor_dq_x": per_launch(lambda r: fq.fp8q_quantize_tensor_delayed(xs[r % N_ROT], n, fq.E4M3FN,
                                                                                     st_tmp, qos[r % N_ROT],
                                                                                     xhats[r % N_ROT]), 16),
        # the per-tensor quantizer with a caller's amax output, overwritten
        # (a one-thread reset launch, then the pass)
        "quantize_tensor_amax_out_x": per_launch(lambda r: fq.fp8q_quantize_tensor(xs[r % N_ROT], n, fq.E4M3FN, sc_x,
                                                                                   qos[r % N_ROT], am_tmp), 16),
        "dequantize_x": per_launch(lambda r: fq.fp8q_dequantize(qxs[r % N_ROT], fq.E4M3FN, 1, n, n, sc_x, fq.GRAN_TENSOR,
                                                                1, xhats[r % N_ROT], n), 16),
        "scaler_update": per_launch(lambda r: fq.fp8q_delayed_scaler_update(st_tmp, am_tmp), 16),
        "scaler_update_mean_1024": per_launch(lambda r: fq.fp8q_delayed_scaler_update(st_mean, am_tmp), 16),
        "scaler_update_ema_1024": per_launch(lambda r: fq.fp8q_delayed_scaler_update(st_ema, am_tmp), 16),
        "quantize_1x128": per_launch(lambda r: fq.fp8q_quantize_1x128(Xs[r % X_ROT], LM, LK, LK, fq.E4M3FN, 1e-12,
                                                                       qXos[r % X_OUT], LK, sX, LK // 128), 6),
        "gemm": per_launch(lambda r: fq.fp8q_gemm_blockscaled(qX, fq.E4M3FN, LK, sX, LK // 128, 1, qW, fq.E4M3FN, LK, sW,
                                                              fq.GRAN_128x128, LK // 128, 1, C, LN, LM, LN, LK), 4),
        "gemm_fast": per_launch(lambda r: fq.fp8q_gemm_blockscaled_fast(qX, fq.E4M3FN, LK, sX, LK // 128, 1, qW, fq.E4M3FN,
                                                                        LK, sW, fq.GRAN_128x128, LK // 128, 1, C, LN, LM,
                                                                        LN, LK), 4),
    }
    # the remaining quantizer rows: 128x128 blocks of the activation, amax
    # alone, and current scaling (amax, the scale from it, the quantize: two
    # reads and one write of the tensor)
    sX128 = torch.empty(LM // 128, LK // 128, dtype=torch.float32, device=dev)
    per["quantize_128x128"] = per_launch(lambda r: fq.fp8q_quantize_128x128(Xs[r % X_ROT], LM, LK, LK, fq.E4M3FN, 1e-12,
                                                                             qXos[r % X_OUT], LK, sX128, LK // 128), 6)
    per["amax_x"] = per_launch(lambda r: fq.fp8q_amax(xs[r % N_ROT], n, am_tmp), 16)
    st_w1 = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=dev)
    fq.fp8q_delayed_scaler_init(st_w1, 1, 448.0, 1e-12, 1.0)

    def current_scaling(r):
        fq.fp8q_amax(xs[r % N_ROT], n, am_tmp)
        fq.fp8q_delayed_scaler_update(st_w1, am_tmp)  # window 1: s = amax / 448
        fq.fp8q_quantize_tensor_delayed(xs[r % N_ROT], n, fq.E4M3FN, st_w1, qos[r % N_ROT])
    per["current_scaling_x"] = per_launch(current_scaling, 8)
    # the same GEMM with its output quantized 1x128 (E4M3FN) in the epilogue
    qC = torch.empty(LM, LN, dtype=torch.uint8, device=dev)
    sC = torch.empty(LM, LN // 128, dtype=torch.float32, device=dev)
    per["gemm_q"] = per_launch(lambda r: fq.fp8q_gemm_blockscaled_q(qX, fq.E4M3FN, LK, sX, LK // 128, 1, qW, fq.E4M3FN,
                                                                    LK, sW, fq.GRAN_128x128, LK // 128, 1, fq.E4M3FN,
                                                                    1e-12, qC, LN, sC, LN // 128, LM, LN, LK), 4)
    del qC, sC
    # The other GEMM shapes (per-kernel figures only, not part of the step):
    # 4096^3 with 1x128 A and 128x128 B scales, bf16 out; and the backward
    # GEMMs of a 4096-wide layer over 16384 tokens, fp32 out: dgrad (E5M2
    # gradients x E4M3 transposed weight, 128x128 B scales) and wgrad (both
    # operands 1x128 along the tokens).  Inputs are quantized by the library
    # once, untimed.
    inputs = {"ds": (xs[0], gs[0]), "X": Xs[0], "qW": qW, "sW": sW}
    log("other GEMM shapes ...")
    del xs, gs, qxs, xhats, qos
    torch.cuda.empty_cache()

    def q1x128(x, fmt):
        r, c = x.shape
        q = torch.empty(r, c, dtype=torch.uint8, device=dev)
        sc = torch.empty(r, c // 128, dtype=torch.float32, device=dev)
        fq.fp8q_quantize_1x128(x, r, c, c, fmt, 1e-12, q, c, sc, c // 128)
        return q, sc

    def q128(x, fmt):
        r, c = x.shape
        q = torch.empty(r, c, dtype=torch.uint8, device=dev)
        sc = torch.empty(r // 128, c // 128, dtype=torch.float32, device=dev)
        fq.fp8q_quantize_128x128(x, r, c, c, fmt, 1e-12, q, c, sc, c // 128)
        return q, sc

    def gemm_ms(qa, fa, sa, qb, fb, sb, gb, out_dtype):
        Mg, Kg = qa.shape
        Ng = qb.shape[0]
        Cg = torch.empty(Mg, Ng, dtype=out_dtype, device=dev)
        return per_launch(lambda r: fq.fp8q_gemm_blockscaled(qa, fa, Kg, sa, sa.shape[1], 1, qb, fb, Kg, sb, gb,
                                                             sb.shape[1], 1, Cg, Ng, Mg, Ng, Kg), 8)

    a3, sa3 = q1x128(W.activation(4096, 4096, seed=3, factor=100.0, device=dev), fq.E4M3FN)
    b3, sb3 = q128(W.weight(4096, 4096, seed=30, device=dev), fq.E4M3FN)
    per["gemm_4096"] = gemm_ms(a3, fq.E4M3FN, sa3, b3, fq.E4M3FN, sb3, fq.GRAN_128x128, torch.bfloat16)
    del a3, sa3, b3, sb3
    dy, sdy = q1x128(W.gradient(16384, 4096, seed=5, device=dev), fq.E5M2)
    wt, swt = q128(W.weight(4096, 4096, seed=50, device=dev), fq.E4M3FN)
    per["gemm_dgrad"] = gemm_ms(dy, fq.E5M2, sdy, wt, fq.E4M3FN, swt, fq.GRAN_128x128, torch.float32)
    # the dgrad's output is the previous layer's gradient: quantized to E5M2
    # in both layouts that layer needs (1x128 along features for its dgrad,
    # along tokens for its wgrad) in the epilogue, against the unfused chain
    # (fp32 C written, then read by the two quantizers)
    DM, DN, DK = 16384, 4096, 4096
    gq = torch.empty(DM, DN, dtype=torch.uint8, device=dev)
    gs_ = torch.empty(DM, DN // 128, dtype=torch.float32, device=dev)
    gqt = torch.empty(DN, DM, dtype=torch.uint8, device=dev)
    gst = torch.empty(DN, DM // 128, dtype=torch.float32, device=dev)
    per["gemm_dgrad_qt"] = per_launch(lambda r: fq.fp8q_gemm_blockscaled_qt(
        dy, fq.E5M2, DK, sdy, DK // 128, 1, wt, fq.E4M3FN, DK, swt, fq.GRAN_128x128, DK // 128, 1, fq.E5M2, 1e-12,
        gqt, DM, gst, DM // 128, gq, DN, gs_, DN // 128, DM, DN, DK), 8)
    Cd = torch.empty(DM, DN, dtype=torch.float32, device=dev)

    def unfused(r):
        fq.fp8q_gemm_blockscaled(dy, fq.E5M2, DK, sdy, DK // 128, 1, wt, fq.E4M3FN, DK, swt, fq.GRAN_128x128,
                                 DK // 128, 1, Cd, DN, DM, DN, DK)
        fq.fp8q_quantize_1x128(Cd, DM, DN, DN, fq.E5M2, 1e-12, gq, DN, gs_, DN // 128)
        fq.fp8q_quantize_1x128_t(Cd, DM, DN, DN, fq.E5M2, 1e-12, gqt, DM, gst, DM // 128)
    per["gemm_dgrad_unfused_chain"] = per_launch(unfused, 8)
    del dy, sdy, wt, swt, gq, gs_, gqt, gst, Cd
    dyt, sdyt = q1x128(W.gradient(4096, 16384, seed=51, device=dev), fq.E5M2)
    # the activations' operand comes from bf16 X [tokens, features] through
    # the transposed 1x128 quantizer (timed here as well)
    # (six input / output sets, 1.2 GB in all, rotated past the last-level cache)
    T_ROT = 6
    Xas = [W.normal((16384, 4096), seed=52 + i, device=dev, dtype=torch.bfloat16) for i in range(T_ROT)]
    xts = [torch.empty(4096, 16384, dtype=torch.uint8, device=dev) for _ in range(T_ROT)]
    sxts = [torch.empty(4096, 128, dtype=torch.float32, device=dev) for _ in range(T_ROT)]
    per["quantize_1x128_t"] = per_launch(lambda r: fq.fp8q_quantize_1x128_t(Xas[r % T_ROT], 16384, 4096, 4096,
                                                                            fq.E4M3FN, 1e-12, xts[r % T_ROT], 16384,
                                                                            sxts[r % T_ROT], 128), 18)
    xt, sxt = xts[0], sxts[0]
    per["gemm_wgrad"] = gemm_ms(dyt, fq.E5M2, sdyt, xt, fq.E4M3FN, sxt, fq.GRAN_1x128, torch.float32)
    del dyt, sdyt, xt, sxt, Xas, xts, sxts
    torch.cuda.empty_cache()

    # MX FP8 (32-element blocks, E8M0 scales) on the layer's shapes: the bf16
    # activation quantized, dequantized, and the MX GEMM against the weight
    Xm = inputs["X"]
    qm = torch.empty(LM, LK, dtype=torch.uint8, device=dev)
    sm = torch.empty(LM, LK // 32, dtype=torch.uint8, device=dev)
    per["quantize_mx"] = per_launch(lambda r: fq.fp8q_quantize_mx(Xs[r % X_ROT], LM, LK, LK, fq.E4M3FN,
                                                                  qXos[r % X_OUT], LK, sm, LK // 32), 12)
    # MX dequantize over four code / output sets (1.3 GB), past the last-level cache
    D_ROT = 4
    qms = [torch.empty(LM, LK, dtype=torch.uint8, device=dev) for _ in range(D_ROT)]
    sms = [torch.empty(LM, LK // 32, dtype=torch.uint8, device=dev) for _ in range(D_ROT)]
    yms = [torch.empty(LM, LK, dtype=torch.bfloat16, device=dev) for _ in range(D_ROT)]
    for i in range(D_ROT):
        fq.fp8q_quantize_mx(Xs[i % X_ROT], LM, LK, LK, fq.E4M3FN, qms[i], LK, sms[i], LK // 32)
    per["dequantize_mx"] = per_launch(lambda r: fq.fp8q_dequantize_mx(qms[r % D_ROT], fq.E4M3FN, LM, LK, LK,
                                                                      sms[r % D_ROT], LK // 32, yms[r % D_ROT], LK), 16)
    del qms, sms, yms, qXos
    wm = W.weight(LN, LK, seed=40, device=dev)
    qwm = torch.empty(LN, LK, dtype=torch.uint8, device=dev)
    swm = torch.empty(LN, LK // 32, dtype=torch.uint8, device=dev)
    fq.fp8q_quantize_mx(wm, LN, LK, LK, fq.E4M3FN, qwm, LK, swm, LK // 32)
    del wm
    fq.fp8q_quantize_mx(Xm, LM, LK, LK, fq.E4M3FN, qm, LK, sm, LK // 32)
    Cm = torch.empty(LM, LN, dtype=torch.bfloat16, device=dev)
    per["gemm_mx"] = per_launch(lambda r: fq.fp8q_gemm_mx(qm, fq.E4M3FN, LK, sm, LK // 32, qwm, fq.E4M3FN, LK, swm,
                                                          LK // 32, Cm, LN, LM, LN, LK), 8)
    del qm, sm, qwm, swm, Cm
    torch.cuda.empty_cache()

    per["stream"] = stream_ceiling(dev, per_launch)
    # Copy reference: a plain elementwise pass (fp32 negation) over 1 GiB,
    # the yardstick for the streaming kernels and the calibration of the
    # HBM byte counters.
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    per["copy_reference"] = per_launch(lambda r: torch.neg(src, out=dst), 8)
    del src, dst
    return per, gpu_ms, wall * 1e3 / steps, inputs


# Read / write bytes per item of the streaming reference (libfp8q_stream.so):
# a copy, a bf16 quantizer's 2:1, an fp32 quantizer's 4:1, a bf16
# dequantizer's 1:2 (8-byte reads, or 16-byte reads and two 16-byte writes),
# and a bf16 quantizer that also writes the bf16 round trip, 2:3 (codes and
# values to two regions), each over about 1 GiB read.
STREAM_KINDS = {"copy": (16, 16), "bf16_to_codes": (16, 8), "fp32_to_codes": (16, 4), "codes_to_bf16": (8, 16),
                "codes_to_bf16_wide": (16, 32), "bf16_to_codes_and_bf16": (16, 24)}
STREAM_READ_BYTES = 1 << 30


def stream_ceiling(dev, per_launch):
    """The fastest hand-written stream of each read:write proportion over
    a sweep of chunk depths and persistent-grid sizes: the attainable HBM
    rate the quantizers are set against."""
    import ctypes

    import torch

    from block_scaled_precision_amax_amd import build as B

    L = ctypes.CDLL(B.STREAM_LIB)
    L.fp8q_stream_ref.restype = ctypes.c_int
    L.fp8q_stream_ref.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    src = torch.ones(STREAM_READ_BYTES // 4 + 1024, dtype=torch.float32, device=dev)
    dst = torch.empty(2 * STREAM_READ_BYTES // 4 + 1024, dtype=torch.float32, device=dev)
    out = {}
    for kind, (rd, wr) in STREAM_KINDS.items():
        items = STREAM_READ_BYTES // rd
        best = None
        # 256-thread workgroups (the quantizers' size) and 1024-thread ones,
        # from a few long-lived workgroups per CU to many short ones
        sweep = [(256, u, g) for u in (1, 2, 4, 8) for g in (4, 8, 16, 32, 64, 128)] + \
                [(1024, u, g) for u in (1, 2) for g in (1, 2, 4, 8)]
        for th, u, g in sweep:
            def launch(r, u=u, g=g, th=th):
                rc = L.fp8q_stream_ref(src.data_ptr(), dst.data_ptr(), items, rd, wr, u, g, cus, th,
                                       torch.cuda.current_stream().cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"fp8q_stream_ref failed: {rc}")
            ms = per_launch(launch, 8)
            gbs = items * (rd + wr) / (ms * 1e-3) / 1e9
            if best is None or gbs > best["GB/s"]:
                best = {"GB/s": round(gbs, 1), "ms": round(ms, 4), "threads": th, "vectors_per_lane": u,
                        "wg_per_cu": g, "read_bytes": items * rd, "write_bytes": items * wr}
        best["frac_hbm"] = round(best["GB/s"] / HBM_PEAK_GBPS, 4)
        out[kind] = best
    del src, dst
    return out


def cpu_baseline(inputs, budget_s: float = 20.0):
    """The CPU oracle (as it stands) on a bounded sample of the step, rates
    extrapolated per element / per MAC to the full step."""
    import numpy as np
    import torch

    import oracle as orc
    from block_scaled_precision_amax_amd import workloads as W

    orc.build(force=False)
    alg = algorithmic()
    n = DS_ROWS * DS_COLS
    x, g = inputs["ds"]
    rows_ds = 2048
    xs = W.to_numpy_input(x[:rows_ds])
    gs = W.to_numpy_input(g[:rows_ds])
    m_ds = rows_ds * DS_COLS
    t0 = time.perf_counter()
    qx = orc.quantize_tensor(xs, orc.E4M3FN, 0.05)
    orc.quantize_tensor(gs, orc.E5M2, 1e-6)
    orc.amax(xs)
    orc.amax(gs)
    orc.dequantize(qx.reshape(1, -1), orc.E4M3FN, np.array([0.05], np.float32), orc.GRAN_TENSOR, out_bf16=True)
    t_ds = time.perf_counter() - t0
    rows_x = 2048
    Xs = W.to_numpy_input(inputs["X"][:rows_x])
    t0 = time.perf_counter()
    qa, sa = orc.quantize_1x128(Xs, orc.E4M3FN)
    t_q = time.perf_counter() - t0
    qW = inputs["qW"].cpu().numpy()
    sW = inputs["sW"].cpu().numpy()
    # GEMM rows in growing chunks until about `budget_s` of oracle time is spent
    t_g, rows_g, chunk = 0.0, 0, 8
    t_start = time.perf_counter()
    while rows_g < rows_x and time.perf_counter() - t_start < budget_s - (t_ds + t_q):
        hi = min(rows_g + chunk, rows_x)
        t0 = time.perf_counter()
        orc.gemm_blockscaled(qa[rows_g:hi], orc.E4M3FN, sa[rows_g:hi], qW, orc.E4M3FN, sW, orc.GRAN_128x128)
        t_g += time.perf_counter() - t0
        rows_g = hi
        chunk *= 2
    est = (t_ds * n / m_ds + t_q * LM / rows_x + t_g * LM / rows_g)
    cores = orc.max_threads()
    # the same on one thread, on a smaller sample (a few seconds)
    orc.set_threads(1)
    try:
        r1 = 128
        t0 = time.perf_counter()
        q1 = orc.quantize_tensor(xs[:r1], orc.E4M3FN, 0.05)
        orc.quantize_tensor(gs[:r1], orc.E5M2, 1e-6)
        orc.amax(xs[:r1])
        orc.amax(gs[:r1])
        orc.dequantize(q1.reshape(1, -1), orc.E4M3FN, np.array([0.05], np.float32), orc.GRAN_TENSOR, out_bf16=True)
        t1_ds = time.perf_counter() - t0
        t0 = time.perf_counter()
        qa1, sa1 = orc.quantize_1x128(Xs[:r1], orc.E4M3FN)
        t1_q = time.perf_counter() - t0
        g1 = 4
        t0 = time.perf_counter()
        orc.gemm_blockscaled(qa1[:g1], orc.E4M3FN, sa1[:g1], qW, orc.E4M3FN, sW, orc.GRAN_128x128)
        t1_g = time.perf_counter() - t0
    finally:
        orc.set_threads(cores)
    est1 = t1_ds * n / (r1 * DS_COLS) + t1_q * LM / r1 + t1_g * LM / g1
    return {
        "value": alg["gemm_flop"] / est / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"oracle on {rows_ds} of {DS_ROWS} rows of both delayed-scaling tensors (quantize, amax, "
                   f"dequantize), {rows_x} of {LM} activation rows (1x128 quantize) and {rows_g} of {LM} "
                   f"GEMM rows; measured {t_ds + t_q + t_g:.1f} s, extrapolated per element / per row "
                   f"to a full step of {est:.1f} s"),
        "single_thread": {"value": alg["gemm_flop"] / est1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                          "sample": (f"{r1} rows of each delayed-scaling tensor, {r1} activation rows and "
                                     f"{g1} GEMM rows on one thread; measured {t1_ds + t1_q + t1_g:.1f} s, "
                                     f"extrapolated to a full step of {est1:.0f} s")},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    per, gpu_ms, wall_ms, inputs = run_gpu(args.steps, args.warmup)
    alg = algorithmic()
    step_ms = max(gpu_ms, wall_ms)
    value = alg["gemm_flop"] / (step_ms * 1e-3) / 1e12

    def gbps(bytes_, ms):
        return bytes_ / (ms * 1e-3) / 1e9

    def gemm_entry(ms, m, n, k, what):
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "TFLOP/s": round(tf, 2), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
                "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4), "operands": what}

    gemm_tflops = alg["gemm_flop"] / (per["gemm"] * 1e-3) / 1e12
    fast_tflops = alg["gemm_flop"] / (per["gemm_fast"] * 1e-3) / 1e12
    q_tflops = alg["gemm_flop"] / (per["gemm_q"] * 1e-3) / 1e12
    q_t = gbps(alg["quantize_tensor_bytes"], per["quantize_tensor_x"])
    q_g = gbps(alg["quantize_tensor_bytes"], per["quantize_tensor_g"])
    q_1 = gbps(alg["quantize_1x128_bytes"], per["quantize_1x128"])
    dq = gbps(alg["dequantize_bytes"], per["dequantize_x"])
    q_dq = gbps(alg["quantize_dq_bytes"], per["quantize_tensor_dq_x"])
    cp = gbps(8 * COPY_ELEMS, per["copy_reference"])
    q_mx = gbps(alg["quantize_mx_bytes"], per["quantize_mx"])
    dq_mx = gbps(alg["quantize_mx_bytes"], per["dequantize_mx"])
    mx_tflops = alg["gemm_flop"] / (per["gemm_mx"] * 1e-3) / 1e12
    traffic = measured_traffic()

    def fs(gbs, *kinds):
        """Fraction of the measured stream ceiling of the same read:write
        proportion (the fastest of the streams given)."""
        return round(gbs / max(per["stream"][k]["GB/s"] for k in kinds), 4)

    out = {
        "metric": "quantize GB/s + block-scaled FP8 GEMM TFLOPS, % of HBM / FP8-MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3fn/e5m2 codes, fp32 accumulate",
        "data": "synthetic (seeded torch generators)",
        "config": {
            "workload": ("fp8 hot path step: delayed-scaling quantize of bf16 8192x8192 x (E4M3FN) and g (E5M2) "
                         "with fused amax, window 16, x round-tripped to bf16 in the same pass (on a second stream beside the layer); LLM layer bf16 X 16384x7168 1x128 "
                         "E4M3FN quantize + block-scaled GEMM vs E4M3FN W 18432x7168 (128x128 scales), bf16 out"),
            "M": LM, "N": LN, "K": LK, "delayed_shape": [DS_ROWS, DS_COLS], "window": WINDOW,
        },
        # The block-scaled FP8 GEMM is judged against the FP8 MFMA peak.  The
        # exact path runs its products on the bf16 MFMA (FP8 codes decoded
        # losslessly), whose own peak is half of that, so it cannot pass 0.50
        # of the FP8 peak; its fraction of the bf16 peak is kept beside it.
        "roofline": {
            "bound": "mfma", "kernel": "gemm_blockscaled", "mfma_dtype": "bf16 (FP8 codes decoded exactly)",
            "achieved": round(gemm_tflops, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
            "frac_bf16_peak": round(gemm_tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "traffic_unit": "bytes per launch", "algorithmic_bytes": alg["gemm_bytes"],
            "mfma_busy": counter_field(MFMA_SUMMARY, "mfma_busy", float),
            "mfma_busy_clock_ghz": counter_field(MFMA_SUMMARY, "clock_ghz", float),
        },
        "kernels": {
            "gemm_blockscaled": {"ms": round(per["gemm"], 4), "TFLOP/s": round(gemm_tflops, 2),
                                 "frac_bf16_peak": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
                                 "frac_fp8_peak": round(gemm_tflops / FP8_PEAK_TFLOPS, 4)},
            "gemm_blockscaled_fast": {"ms": round(per["gemm_fast"], 4), "TFLOP/s": round(fast_tflops, 2),
                                      "frac_fp8_peak": round(fast_tflops / FP8_PEAK_TFLOPS, 4),
                                      "note": "FP8 MFMA path, measured outside the step"},
            "gemm_blockscaled_q": {"ms": round(per["gemm_q"], 4), "TFLOP/s": round(q_tflops, 2),
                                   "frac_fp8_peak": round(q_tflops / FP8_PEAK_TFLOPS, 4),
                                   "frac_bf16_peak": round(q_tflops / BF16_PEAK_TFLOPS, 4),
                                   "note": "exact path, output quantized 1x128 to E4M3FN in the epilogue"},
            "quantize_1x128_bf16": {"ms": round(per["quantize_1x128"], 4), "GB/s": round(q_1, 1),
                                    "frac_hbm": round(q_1 / HBM_PEAK_GBPS, 4),
                                    "frac_stream": fs(q_1, "bf16_to_codes")},
            "quantize_tensor_bf16_e4m3": {"ms": round(per["quantize_tensor_x"], 4), "GB/s": round(q_t, 1),
                                          "note": "fp8q_quantize_tensor_delayed (the step's x, without the round trip)",
                                          "frac_hbm": round(q_t / HBM_PEAK_GBPS, 4),
                                          "frac_stream": fs(q_t, "bf16_to_codes")},
            "quantize_tensor_bf16_e5m2": {"ms": round(per["quantize_tensor_g"], 4), "GB/s": round(q_g, 1),
                                          "frac_hbm": round(q_g / HBM_PEAK_GBPS, 4),
                                          "frac_stream": fs(q_g, "bf16_to_codes")},
            "quantize_tensor_amax_out_bf16_e4m3": {
                "ms": round(per["quantize_tensor_amax_out_x"], 4),
                "GB/s": round(gbps(alg["quantize_tensor_bytes"], per["quantize_tensor_amax_out_x"]), 1),
                "frac_hbm": round(gbps(alg["quantize_tensor_bytes"], per["quantize_tensor_amax_out_x"]) / HBM_PEAK_GBPS, 4),
                "note": "fp8q_quantize_tensor with its amax output overwritten: a one-thread reset launch, then the pass"},
            "quantize_tensor_dq_bf16_e4m3": {"ms": round(per["quantize_tensor_dq_x"], 4), "GB/s": round(q_dq, 1),
                                             "frac_hbm": round(q_dq / HBM_PEAK_GBPS, 4), "frac_stream": fs(q_dq, "bf16_to_codes_and_bf16"),
                                             "note": "codes and their bf16 round trip in one pass (the step's x)"},
            "quantize_128x128_bf16": {
                "ms": round(per["quantize_128x128"], 4),
                "GB/s": round(gbps(LM * LK * (3 + 4 / 16384), per["quantize_128x128"]), 1),
                "frac_hbm": round(gbps(LM * LK * (3 + 4 / 16384), per["quantize_128x128"]) / HBM_PEAK_GBPS, 4),
                "frac_stream": fs(gbps(LM * LK * (3 + 4 / 16384), per["quantize_128x128"]), "bf16_to_codes"),
                "note": "128x128 blocks of the layer's activation 16384x7168"},
            "amax_bf16": {"ms": round(per["amax_x"], 4), "GB/s": round(gbps(2 * DS_ROWS * DS_COLS, per["amax_x"]), 1),
                          "frac_hbm": round(gbps(2 * DS_ROWS * DS_COLS, per["amax_x"]) / HBM_PEAK_GBPS, 4),
                          "note": "fp8q_amax alone over the 8192x8192 bf16 tensor (one read)"},
            "current_scaling_bf16_e4m3": {
                "ms": round(per["current_scaling_x"], 4), "GB/s": round(gbps(5 * DS_ROWS * DS_COLS, per["current_scaling_x"]), 1),
                "frac_hbm": round(gbps(5 * DS_ROWS * DS_COLS, per["current_scaling_x"]) / HBM_PEAK_GBPS, 4),
                "note": "current scaling: amax, the scale from it, then the quantize (two reads + one write)"},
            "dequantize_bf16": {"ms": round(per["dequantize_x"], 4), "GB/s": round(dq, 1),
                                "frac_hbm": round(dq / HBM_PEAK_GBPS, 4),
                                "frac_stream": fs(dq, "codes_to_bf16", "codes_to_bf16_wide")},
            "scaler_update": {"ms": round(per["scaler_update"], 4)},
            "scaler_update_mean_1024": {"ms": round(per["scaler_update_mean_1024"], 4),
                                        "note": "window mean over 1024 slots (fp64 pairwise)"},
            "scaler_update_ema_1024": {"ms": round(per["scaler_update_ema_1024"], 4), "note": "EMA, alpha 0.01"},
            "quantize_1x128_t_bf16_16384x4096": {
                "ms": round(per["quantize_1x128_t"], 4),
                "GB/s": round(gbps(16384 * 4096 * (3 + 4 / 128), per["quantize_1x128_t"]), 1),
                "frac_hbm": round(gbps(16384 * 4096 * (3 + 4 / 128), per["quantize_1x128_t"]) / HBM_PEAK_GBPS, 4),
                "frac_stream": fs(gbps(16384 * 4096 * (3 + 4 / 128), per["quantize_1x128_t"]), "bf16_to_codes"),
                "note": "codes of the transpose, 1x128 along tokens (weight-gradient operand)"},
            "gemm_blockscaled_4096x4096x4096": gemm_entry(per["gemm_4096"], 4096, 4096, 4096,
                                                          "E4M3FN x E4M3FN, 1x128 A / 128x128 B scales, bf16 out"),
            "gemm_blockscaled_dgrad_16384x4096x4096": gemm_entry(per["gemm_dgrad"], 16384, 4096, 4096,
                                                                 "E5M2 x E4M3FN, 1x128 A / 128x128 B scales, fp32 out"),
            "gemm_blockscaled_qt_dgrad_16384x4096x4096": {
                **gemm_entry(per["gemm_dgrad_qt"], 16384, 4096, 4096,
                             "E5M2 x E4M3FN, output quantized to E5M2 in the epilogue, 1x128 along N and along M"),
                "unfused_chain_ms": round(per["gemm_dgrad_unfused_chain"], 4),
                "note": ("unfused chain: the fp32-out dgrad, then fp8q_quantize_1x128 and fp8q_quantize_1x128_t of "
                         "its 256 MB output")},
            "gemm_blockscaled_wgrad_4096x4096x16384": gemm_entry(per["gemm_wgrad"], 4096, 4096, 16384,
                                                                 "E5M2 x E4M3FN, 1x128 A and B scales, fp32 out"),
            "quantize_mx_bf16": {"ms": round(per["quantize_mx"], 4), "GB/s": round(q_mx, 1),
                                 "frac_hbm": round(q_mx / HBM_PEAK_GBPS, 4), "frac_stream": fs(q_mx, "bf16_to_codes"),
                                 "note": "MX E4M3FN, 32-element blocks, E8M0 scales; the layer's activation"},
            "dequantize_mx_bf16": {"ms": round(per["dequantize_mx"], 4), "GB/s": round(dq_mx, 1),
                                   "frac_hbm": round(dq_mx / HBM_PEAK_GBPS, 4),
                                   "frac_stream": fs(dq_mx, "codes_to_bf16", "codes_to_bf16_wide")},
            "gemm_mx": {"ms": round(per["gemm_mx"], 4), "TFLOP/s": round(mx_tflops, 2),
                        "frac_fp8_peak": round(mx_tflops / FP8_PEAK_TFLOPS, 4),
                        "operands": "MX E4M3FN x MX E4M3FN, scaled FP8 MFMA, bf16 out, the layer's shape"},
            "stream_ceiling": {**per["stream"],
                               "note": ("hand-written 16-B-per-lane streams (libfp8q_stream.so), best of a sweep of "
                                        "chunk depth, grid size and workgroup size (256 or 1024 threads), about "
                                        "1 GiB read each: the attainable HBM rate for each read:write proportion")},
            "copy_reference_fp32": {"ms": round(per["copy_reference"], 4), "GB/s": round(cp, 1),
                                    "frac_hbm": round(cp / HBM_PEAK_GBPS, 4),
                                    "note": "torch elementwise pass, 1 GiB in + 1 GiB out: attainable streaming rate"},
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
