"""GPU parity of the quantizers against the CPU oracle, bit for bit.

Every call goes through the C ABI (the ctypes binding); inputs come from
the seeded generators and reach both sides as the same bytes.  Codes,
scales, amax values and scaler states must be identical; NaN results are
compared as the canonical quiet NaN both sides produce.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

from block_scaled_precision_amax_amd import workloads as W

pytestmark = pytest.mark.gpu

E4, E5 = 0, 1
MAXF = {E4: 448.0, E5: 57344.0}
EPS = 1e-12


def f32bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_codes_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {bad[0]}: {got.reshape(-1)[bad[0]]:#x} vs {want.reshape(-1)[bad[0]]:#x}"


# ------------------------------------------------------------------ helpers
def run_block(fq, x_dev, rows, cols, ldx, fmt, br, eps=EPS, pad_q=0, pad_s=0):
    """Quantize the rows x cols view of x_dev (leading dimension ldx) on the GPU."""
    ldq, ld_s = cols + pad_q, cols // 128 + pad_s
    q = torch.full((rows, ldq), 0xAA, dtype=torch.uint8, device=x_dev.device)
    s = torch.full(((rows // br), ld_s), -7.0, dtype=torch.float32, device=x_dev.device)
    fn = fq.fp8q_quantize_1x128 if br == 1 else fq.fp8q_quantize_128x128
    fn(x_dev, rows, cols, ldx, fmt, eps, q, ldq, s, ld_s)
    torch.cuda.synchronize()
    qn, sn = q.cpu().numpy(), s.cpu().numpy()
    if pad_q:
        assert np.all(qn[:, cols:] == 0xAA), "wrote past the row"
    if pad_s:
        assert np.all(sn[:, cols // 128:] == -7.0), "wrote past the scale row"
    return qn[:, :cols], sn[:, :cols // 128]


def oracle_block(orc, x_np, br, fmt, eps=EPS):
    return orc.quantize_blocks(x_np, br, 128, fmt, eps)


def special_blocks_fp32(rng, rows):
    """rows x 1024 fp32 whose 128-wide blocks exercise every branch: zeros,
    signed zeros, NaN, +-Inf, fp32 denormals, values below eps, huge values
    (the IEEE-division path), exact FP8 rounding midpoints and their fp32
    neighbours, and ordinary N(0,1) data."""
    x = rng.standard_normal((rows, 1024)).astype(np.float32)
    x[:, 0:128] = 0.0
    x[::2, 0:128] = -0.0
    x[1::3, 5] = -0.0
    x[:, 128:256] *= np.float32(3.0)
    x[0, 130] = np.nan
    x[1, 131] = np.inf
    x[2, 132] = -np.inf
    x[3, 133] = -np.nan
    x[:, 256:384] = (rng.standard_normal((rows, 128)) * 1e-41).astype(np.float32)  # fp32 denormals
    x[:, 384:512] = (rng.standard_normal((rows, 128)) * 1e-13).astype(np.float32)  # below eps
    x[:, 512:640] = (rng.standard_normal((rows, 128)) * 1e37).astype(np.float32)   # s > 2^80
    x[::2, 512:640] = np.float32(3.4e38)
    # exact rounding midpoints of E4M3/E5M2 in [1, 448) with the block
    # amax 448 (so s = 1, x / s = x) and their fp32 neighbours
    mids = []
    for e in range(-9, 9):
        for m in range(16):
            v = (1 + (m + 0.5) / 8) * 2.0 ** e
            if v < 448:
                mids.append(v)
    mids = np.array(mids, dtype=np.float32)
    k = rng.integers(0, mids.size, size=(rows, 127))
    ulp = rng.integers(-2, 3, size=(rows, 127)).astype(np.int32)
    v = (mids[k].view(np.int32) + ulp).view(np.float32) * np.where(rng.random((rows, 127)) < 0.5, -1, 1)
    x[:, 640:767] = v.astype(np.float32)
    x[:, 767] = np.float32(448.0)
    # the same midpoints against a non power-of-two scale: amax 300 -> s = 300/448
    s = np.float32(300.0) / np.float32(448.0)
    w = (mids[k] * s).astype(np.float32)
    w = (w.view(np.int32) + ulp).view(np.float32)
    x[:, 768:895] = np.minimum(np.abs(w), np.float32(299.0)) * np.sign(w)
    x[:, 895] = np.float32(300.0)
    return x


# ------------------------------------------------------------------ the hardware cast, exhaustively
@pytest.mark.parametrize("fmt", [E4, E5])
def test_cast_every_fp32_pattern(fq, orc, gpu, fmt):
    """All 2^32 fp32 bit patterns through fp8q_quantize_tensor with s = 1
    (so x / s = x): every code equals the oracle's encoder."""
    one = torch.ones(1, dtype=torch.float32, device=gpu)
    chunk = 1 << 28
    q = torch.empty(chunk, dtype=torch.uint8, device=gpu)
    for start in range(0, 1 << 32, chunk):
        # int64 -> int32 keeps the low 32 bits: the patterns start .. start+chunk-1
        bits = torch.arange(start, start + chunk, dtype=torch.int64, device=gpu).to(torch.int32)
        x = bits.view(torch.float32)
        fq.fp8q_quantize_tensor(x, chunk, fmt, one, q)
        torch.cuda.synchronize()
        want = orc.encode_bits_range(start, chunk, fmt)
        assert_codes_equal(q.cpu().numpy(), want, f"patterns {start:#x}+")
        del bits, x


@pytest.mark.parametrize("fmt", [E4, E5])
def test_cast_every_bf16_pattern(fq, orc, gpu, fmt):
    """All 2^16 bf16 bit patterns, s = 1."""
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).to(gpu)
    one = torch.ones(1, dtype=torch.float32, device=gpu)
    q = torch.empty(1 << 16, dtype=torch.uint8, device=gpu)
    fq.fp8q_quantize_tensor(x, 1 << 16, fmt, one, q)
    torch.cuda.synchronize()
    want = orc.quantize_tensor(bits.numpy().view(np.uint16), fmt, 1.0)
    assert_codes_equal(q.cpu().numpy(), want)


# ------------------------------------------------------------------ amax
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [1, 7, 8, 1000, (1 << 20) + 3, 5_000_011])
def test_amax(fq, orc, gpu, dtype, n):
    x = W.normal((n,), seed=n, device="cpu", std=3.0, dtype=dtype)
    if n > 10:
        x[n // 3] = -1e4
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=gpu)
    fq.fp8q_amax(x.to(gpu), n, amax)
    torch.cuda.synchronize()
    want = orc.amax(W.to_numpy_input(x))
    assert f32bits(amax.cpu().numpy())[0] == f32bits([want])[0]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_amax_special(fq, orc, gpu, dtype):
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    for vals in ([0.0, -0.0], [1.0, -math.inf, 2.0], [1.0, float("nan"), 5.0], [-float("nan")] * 9):
        x = torch.tensor(vals * 37, dtype=dtype)
        fq.fp8q_amax(x.to(gpu), x.numel(), amax)
        torch.cuda.synchronize()
        want = orc.amax(W.to_numpy_input(x))
        assert f32bits(amax.cpu().numpy())[0] == f32bits([want])[0], vals


# ------------------------------------------------------------------ per-tensor
SCALES = [1.0, 0.37, 1e-3, 12345.0, 2.0 ** -79, 2.0 ** -81, 2.0 ** 81, 0.0, math.inf, float("nan"), 1e-30,
          1e-40, 3.0e38, -2.0]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", [E4, E5])
def test_quantize_tensor(fq, orc, gpu, dtype, fmt):
    n = 100_003
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(n) * np.exp(rng.standard_normal(n) * 4)).astype(np.float32)
    x[::97] = 0.0
    x[1::97] = -0.0
    x[5] = np.nan
    x[6] = np.inf
    x[n - 1] = -np.inf
    x[n - 2] = np.nan
    xt = torch.from_numpy(x).to(dtype)
    xd = xt.to(gpu)
    xn = W.to_numpy_input(xt)
    q = torch.empty(n, dtype=torch.uint8, device=gpu)
    for s in SCALES:
        sd = torch.tensor([s], dtype=torch.float32, device=gpu)
        fq.fp8q_quantize_tensor(xd, n, fmt, sd, q)
        torch.cuda.synchronize()
        assert_codes_equal(q.cpu().numpy(), orc.quantize_tensor(xn, fmt, float(np.float32(s))), f"s={s}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_quantize_tensor_round_trip(fq, orc, gpu, dtype, fmt, out):
    """fp8q_quantize_tensor_dq: codes as fp8q_quantize_tensor, the round
    trip as the oracle's dequantize of those codes (fp32 bit for bit; bf16
    as its RNE, NaN as 0x7FC0), a ragged length (tail elements), NaN / Inf /
    signed zeros, every scale regime, and the fused amax."""
    n = 100_003
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(n) * np.exp(rng.standard_normal(n) * 4)).astype(np.float32)
    x[::97] = 0.0
    x[1::97] = -0.0
    x[5] = np.nan
    x[6] = np.inf
    x[n - 1] = -np.inf
    x[n - 2] = np.nan
    xt = torch.from_numpy(x).to(dtype)
    xd = xt.to(gpu)
    xn = W.to_numpy_input(xt)
    q = torch.empty(n, dtype=torch.uint8, device=gpu)
    y = torch.empty(n, dtype=out, device=gpu)
    acc = torch.zeros(1, dtype=torch.float32, device=gpu)
    for s in SCALES:
        sd = torch.tensor([s], dtype=torch.float32, device=gpu)
        fq.fp8q_quantize_tensor_dq(xd, n, fmt, sd, q, y, acc)
        torch.cuda.synchronize()
        wq = orc.quantize_tensor(xn, fmt, float(np.float32(s))).reshape(-1)
        assert_codes_equal(q.cpu().numpy(), wq, f"s={s}")
        sc = np.array([s], np.float32)
        if out == torch.float32:
            wy = orc.dequantize(wq.reshape(1, -1), fmt, sc, orc.GRAN_TENSOR).reshape(-1)
            assert np.array_equal(f32bits(y.cpu().numpy()), f32bits(wy)), f"s={s}"
        else:
            wy = orc.dequantize(wq.reshape(1, -1), fmt, sc, orc.GRAN_TENSOR, out_bf16=True).reshape(-1)
            assert np.array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), wy), f"s={s}"
    assert f32bits(acc.cpu().numpy())[0] == 0x7FC00000  # x holds NaN


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_tensor_amax_overwrites(fq, orc, gpu, dtype):
    """The fused amax is written, not accumulated: a caller that hands in
    whatever buffer it has (a stale larger value, a stale NaN, garbage) gets
    this call's amax(x); a NaN in x gives the quiet NaN; back-to-back calls
    on different tensors with no reset in between each get their own."""
    x = W.normal((77_777,), seed=3, std=5.0, dtype=dtype)
    xd = x.to(gpu)
    q = torch.empty(x.numel(), dtype=torch.uint8, device=gpu)
    sd = torch.tensor([0.5], dtype=torch.float32, device=gpu)
    want = f32bits([orc.amax(W.to_numpy_input(x))])[0]
    for stale in (0.0, 1e9, float("nan"), float("inf"), -3.0):
        out = torch.tensor([stale], dtype=torch.float32, device=gpu)
        fq.fp8q_quantize_tensor(xd, x.numel(), E4, sd, q, out)
        torch.cuda.synchronize()
        assert f32bits(out.cpu().numpy())[0] == want, stale
    xn = x.clone()
    xn[123] = float("nan")
    out = torch.zeros(1, dtype=torch.float32, device=gpu)
    fq.fp8q_quantize_tensor(xn.to(gpu), x.numel(), E4, sd, q, out)
    torch.cuda.synchronize()
    assert f32bits(out.cpu().numpy())[0] == 0x7FC00000
    # the same buffer again, no reset by the caller: the NaN does not stick
    small = W.normal((4096,), seed=4, std=0.01, dtype=dtype)
    fq.fp8q_quantize_tensor(small.to(gpu), small.numel(), E4, sd, q, out)
    torch.cuda.synchronize()
    assert f32bits(out.cpu().numpy())[0] == f32bits([orc.amax(W.to_numpy_input(small))])[0]
    # and the round-trip variant
    y = torch.empty(x.numel(), dtype=torch.float32, device=gpu)
    fq.fp8q_quantize_tensor_dq(xd, x.numel(), E4, sd, q, y, out)
    torch.cuda.synchronize()
    assert f32bits(out.cpu().numpy())[0] == want


def test_fused_amax_concurrent_calls(fq, orc, gpu):
    """Per-tensor quantizations and fp8q_amax calls in flight at the same time
    on eight streams (default priority), each with its own amax output: the
    one-launch reduction keys its device-side slot by the output, so every
    output gets its own tensor's amax, over three rounds with no reset."""
    streams = [torch.cuda.Stream() for _ in range(8)]
    xs = [W.normal(((1 << 20) + 37 * i,), seed=60 + i, std=float(2 ** i), dtype=torch.bfloat16).to(gpu)
          for i in range(8)]
    want = [f32bits([orc.amax(W.to_numpy_input(x.cpu()))])[0] for x in xs]
    outs = [torch.full((1,), float("nan"), dtype=torch.float32, device=gpu) for _ in range(8)]
    qs = [torch.empty(x.numel(), dtype=torch.uint8, device=gpu) for x in xs]
    sd = torch.tensor([0.25], dtype=torch.float32, device=gpu)
    torch.cuda.synchronize()
    for rnd in range(3):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                if (i + rnd) % 2:
                    fq.fp8q_quantize_tensor(xs[i], xs[i].numel(), E4, sd, qs[i], outs[i])
                else:
                    fq.fp8q_amax(xs[i], xs[i].numel(), outs[i])
        torch.cuda.synchronize()
        for i in range(8):
            assert f32bits(outs[i].cpu().numpy())[0] == want[i], (rnd, i)


# ------------------------------------------------------------------ block quantizers
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("factor", [1e2, 1e4, 3e4])
def test_1x128_outlier_experiment(fq, orc, gpu, fmt, factor):
    """The handbook's 256x1024 outlier activation (columns 0-3 scaled)."""
    x = W.activation(256, 1024, seed=0, factor=factor)
    q, s = run_block(fq, x.to(gpu), 256, 1024, 1024, fmt, 1)
    wq, ws = oracle_block(orc, x.numpy(), 1, fmt)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_special_values(fq, orc, gpu, br, fmt, dtype):
    rng = np.random.default_rng(12 + br)
    x = special_blocks_fp32(rng, 256)
    xt = torch.from_numpy(x).to(dtype)
    q, s = run_block(fq, xt.to(gpu), 256, 1024, 1024, fmt, br)
    wq, ws = oracle_block(orc, W.to_numpy_input(xt), br, fmt)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_random_bit_patterns(fq, orc, gpu, br, dtype):
    """Uniformly random bit patterns (every exponent, NaN and Inf included)."""
    g = torch.Generator().manual_seed(99)
    if dtype == torch.float32:
        bits = torch.randint(-(1 << 31), 1 << 31, (384, 640), generator=g, dtype=torch.int64).to(torch.int32)
        xt = bits.view(torch.float32)
    else:
        bits = torch.randint(-(1 << 15), 1 << 15, (384, 640), generator=g, dtype=torch.int32).to(torch.int16)
        xt = bits.view(torch.bfloat16)
    for fmt in (E4, E5):
        q, s = run_block(fq, xt.to(gpu), 384, 640, 640, fmt, br)
        wq, ws = oracle_block(orc, W.to_numpy_input(xt), br, fmt)
        assert_codes_equal(q, wq)
        assert np.array_equal(f32bits(s), f32bits(ws))


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_strided_and_ragged(fq, orc, gpu, br, dtype):
    """A strided view (ldx > cols), padded q / scale rows that must stay
    untouched, a row count that leaves a partial wavefront group, eps != 1e-12."""
    rows = 37 * 128 if br == 128 else 1237
    cols, ldx = 384, 512
    full = W.activation(rows, ldx, seed=21, outlier_cols=3, factor=300.0, dtype=dtype)
    for fmt in (E4, E5):
        q, s = run_block(fq, full.to(gpu), rows, cols, ldx, fmt, br, eps=1e-3, pad_q=16, pad_s=3)
        wq, ws = oracle_block(orc, W.to_numpy_input(full[:, :cols].contiguous()), br, fmt, eps=1e-3)
        assert_codes_equal(q, wq)
        assert np.array_equal(f32bits(s), f32bits(ws))


@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 128), (5, 256), (63, 384), (65, 128)])
def test_1x128_small_shapes(fq, orc, gpu, rows, cols):
    x = W.normal((rows, cols), seed=rows * cols, std=2.0)
    for fmt in (E4, E5):
        q, s = run_block(fq, x.to(gpu), rows, cols, cols, fmt, 1)
        wq, ws = oracle_block(orc, x.numpy(), 1, fmt)
        assert_codes_equal(q, wq)
        assert np.array_equal(f32bits(s), f32bits(ws))


# ------------------------------------------------------------------ full-size workloads
def test_full_size_activation_1x128_bf16(fq, orc, gpu):
    """The LLM-layer activation at its real shape: bf16 16384x7168 N(0,1),
    columns 0-3 x1e3, 1x128 E4M3FN, compared in full."""
    x = W.activation(16384, 7168, seed=4, factor=1e3, dtype=torch.bfloat16, device=gpu)
    q, s = run_block(fq, x, 16384, 7168, 7168, E4, 1)
    wq, ws = oracle_block(orc, W.to_numpy_input(x), 1, E4)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))


def test_full_size_delayed_step_tensor_bf16(fq, orc, gpu):
    """One delayed-scaling step at its real shape: bf16 8192x8192, sigma 37."""
    x = W.delayed_step(8192, 8192, 37.0, seed=2, device=gpu)
    n = x.numel()
    q = torch.empty(n, dtype=torch.uint8, device=gpu)
    acc = torch.zeros(1, dtype=torch.float32, device=gpu)
    s = torch.tensor([0.3], dtype=torch.float32, device=gpu)
    fq.fp8q_quantize_tensor(x, n, E4, s, q, acc)
    torch.cuda.synchronize()
    xn = W.to_numpy_input(x)
    assert_codes_equal(q.cpu().numpy(), orc.quantize_tensor(xn, E4, float(np.float32(0.3))))
    assert f32bits(acc.cpu().numpy())[0] == f32bits([orc.amax(xn)])[0]


def test_full_size_gemm_operands(fq, orc, gpu):
    """The 4096^3 GEMM's operands: A fp32 N(0,1) with 4 outlier columns x100
    (1x128), B fp32 0.02*N(0,1) (128x128), both E4M3FN, compared in full."""
    a = W.activation(4096, 4096, seed=3, factor=100.0, device=gpu)
    q, s = run_block(fq, a, 4096, 4096, 4096, E4, 1)
    wq, ws = oracle_block(orc, a.cpu().numpy(), 1, E4)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))
    b = W.weight(4096, 4096, seed=30, device=gpu)
    q, s = run_block(fq, b, 4096, 4096, 4096, E4, 128)
    wq, ws = oracle_block(orc, b.cpu().numpy(), 128, E4)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))


def test_full_size_weight_128x128_fp32(fq, orc, gpu):
    """The LLM-layer weight: fp32 0.02*N(0,1) [18432, 7168], 128x128 E4M3FN."""
    w = W.weight(18432, 7168, seed=4, device=gpu)
    q, s = run_block(fq, w, 18432, 7168, 7168, E4, 128)
    wq, ws = oracle_block(orc, w.cpu().numpy(), 128, E4)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))


# ------------------------------------------------------------------ 1x128 of the transpose
def run_block_t(fq, x_dev, rows, cols, ldx, fmt, pad_q=0, pad_s=0):
    """fp8q_quantize_1x128_t of the rows x cols view of x_dev: codes [cols, rows]."""
    ldq, ld_s = rows + pad_q, rows // 128 + pad_s
    q = torch.full((cols, ldq), 0xAA, dtype=torch.uint8, device=x_dev.device)
    s = torch.full((cols, ld_s), -7.0, dtype=torch.float32, device=x_dev.device)
    fq.fp8q_quantize_1x128_t(x_dev, rows, cols, ldx, fmt, EPS, q, ldq, s, ld_s)
    torch.cuda.synchronize()
    qn, sn = q.cpu().numpy(), s.cpu().numpy()
    assert np.all(qn[:, rows:] == 0xAA), "wrote past the row"
    assert np.all(sn[:, rows // 128:] == -7.0), "wrote past the scale row"
    return qn[:, :rows], sn[:, :rows // 128]


def oracle_t(orc, x_np, fmt):
    """The definition: 1x128 quantization of the transpose."""
    return orc.quantize_1x128(np.ascontiguousarray(x_np.T), fmt, EPS)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("rows,cols,ldx,pad_q", [(128, 64, 64, 0), (256, 192, 200, 32), (384, 128, 136, 16),
                                                 (128, 1024, 1024, 0), (384, 512, 520, 16), (640, 768, 768, 0),
                                                 (1280, 256, 264, 16), (1152, 320, 320, 0)])
def test_quantize_1x128_t(fq, orc, gpu, dt, fmt, rows, cols, ldx, pad_q):
    """Padded rows; one or an odd number of 64-column slabs (64-column
    workgroups) and pairs of them (128-column workgroups); several 128-row
    blocks per workgroup, and a last workgroup with fewer row blocks."""
    rng = np.random.default_rng(rows + cols + fmt)
    x = (rng.standard_normal((rows, ldx)) * np.exp(rng.standard_normal((1, ldx)) * 3)).astype(np.float32)
    xd = torch.from_numpy(x).to(dt).to(gpu)
    xv = W.to_numpy_input(xd.cpu())[:, :cols]
    q, s = run_block_t(fq, xd, rows, cols, ldx, fmt, pad_q=pad_q, pad_s=1)
    wq, ws = oracle_t(orc, xv, fmt)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("ncols", [64, 256])
def test_quantize_1x128_t_special_values(fq, orc, gpu, dt, fmt, ncols):
    """Every special block (zeros, NaN, Inf, denormals, below eps, huge,
    rounding midpoints) as 128-row column segments, one and four slabs."""
    x = np.ascontiguousarray(special_blocks_fp32(np.random.default_rng(11), ncols).T)  # 1024 x ncols
    xd = torch.from_numpy(x).to(dt).to(gpu)
    xv = W.to_numpy_input(xd.cpu())
    q, s = run_block_t(fq, xd, 1024, ncols, ncols, fmt)
    wq, ws = oracle_t(orc, xv, fmt)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))


def test_quantize_1x128_t_full_wgrad_operand(fq, orc, gpu):
    """The weight-gradient operand: bf16 activations [16384 tokens, 4096]
    N(0,1), quantized to E4M3FN codes [4096, 16384] with scales per 128 tokens."""
    x = W.normal((16384, 4096), seed=52, device=gpu, dtype=torch.bfloat16)
    q, s = run_block_t(fq, x, 16384, 4096, 4096, E4)
    wq, ws = oracle_t(orc, W.to_numpy_input(x.cpu()), E4)
    assert_codes_equal(q, wq)
    assert np.array_equal(f32bits(s), f32bits(ws))


# ------------------------------------------------------------------ dequantize
@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("gran", [0, 1, 2])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_dequantize(fq, orc, gpu, fmt, gran, out):
    rows, cols = 256, 640
    q = torch.randint(0, 256, (rows, cols), generator=torch.Generator().manual_seed(5), dtype=torch.int32)
    q = q.to(torch.uint8)
    rng = np.random.default_rng(6)
    shape = {0: (1, 1), 1: (rows, cols // 128), 2: ((rows + 127) // 128, cols // 128)}[gran]
    s = np.exp(rng.standard_normal(shape) * 5).astype(np.float32)
    s.reshape(-1)[0] = np.float32(1e-40)
    y = torch.empty(rows, cols, dtype=out, device=gpu)
    fq.fp8q_dequantize(q.to(gpu), fmt, rows, cols, cols, torch.from_numpy(s).to(gpu), gran, shape[1], y, cols)
    torch.cuda.synchronize()
    want = orc.dequantize(q.numpy(), fmt, s, gran, out_bf16=out == torch.bfloat16)
    got = y.cpu().view(torch.int32 if out == torch.float32 else torch.int16).numpy()
    # bit patterns (NaN results are the canonical quiet NaN on both sides)
    assert np.array_equal(got.view(np.uint32 if out == torch.float32 else np.uint16),
                          want.view(np.uint32 if out == torch.float32 else np.uint16))


@pytest.mark.parametrize("gran,rows,cols,ld", [(0, 100, 1000, 1004), (1, 100, 384, 388), (2, 300, 384, 388),
                                                 (0, 3, 4096, 4100), (1, 129, 512, 528)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_dequantize_strided(fq, orc, gpu, gran, rows, cols, ld, out):
    """Leading dimensions that are not 16-byte row strides (the dword path) or
    are (ld 528), rows whose length is not a multiple of 16 codes, and a
    subnormal scale."""
    q = W.fp8_codes((rows, ld), E4, seed=rows + cols)
    rng = np.random.default_rng(ld)
    shape = {0: (1, 1), 1: (rows, cols // 128), 2: ((rows + 127) // 128, cols // 128)}[gran]
    s = np.exp(rng.standard_normal(shape) * 5).astype(np.float32)
    s.reshape(-1)[-1] = np.float32(3e-41)
    y = torch.full((rows, ld), 7.0, dtype=out, device=gpu)
    fq.fp8q_dequantize(q.to(gpu), E4, rows, cols, ld, torch.from_numpy(s).to(gpu), gran, shape[1], y, ld)
    torch.cuda.synchronize()
    want = orc.dequantize(np.ascontiguousarray(q.numpy()[:, :cols]), E4, s, gran, out_bf16=out == torch.bfloat16)
    bits = np.uint32 if out == torch.float32 else np.uint16
    got = y.cpu().view(torch.int32 if out == torch.float32 else torch.int16).numpy().view(bits)
    assert np.array_equal(got[:, :cols], want.view(bits))
    pad = np.float32(7.0).view(np.uint32) if out == torch.float32 else np.uint16(0x40E0)
    assert np.all(got[:, cols:] == pad), "dequantize wrote past the row"


@pytest.mark.parametrize("gran,rows,cols", [(0, 1, 70_000_000), (1, 40_000, 128), (2, 40_100, 256)])
def test_dequantize_many_passes(fq, orc, gpu, gran, rows, cols):
    """More work units (a row's chunk of 4096 codes) than the grid has
    workgroups, so every workgroup walks several units: bf16 bit-exact
    against the oracle over the whole tensor."""
    q = W.fp8_codes((rows, cols), E4, seed=rows + cols)
    rng = np.random.default_rng(rows)
    shape = {0: (1, 1), 1: (rows, cols // 128), 2: ((rows + 127) // 128, cols // 128)}[gran]
    s = np.exp(rng.standard_normal(shape) * 3).astype(np.float32)
    y = torch.empty(rows, cols, dtype=torch.bfloat16, device=gpu)
    fq.fp8q_dequantize(q.to(gpu), E4, rows, cols, cols, torch.from_numpy(s).to(gpu), gran, shape[1], y, cols)
    torch.cuda.synchronize()
    want = orc.dequantize(q.numpy(), E4, s, gran, out_bf16=True)
    assert np.array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), want.view(np.uint16))


def test_dequantize_flat_ragged(fq, orc, gpu):
    n = 10_007
    q = W.fp8_codes((n,), E4, seed=8)
    s = np.array([0.123], np.float32)
    y = torch.empty(n, dtype=torch.float32, device=gpu)
    fq.fp8q_dequantize(q.to(gpu), E4, 1, n, n, torch.from_numpy(s).to(gpu), 0, 1, y, n)
    torch.cuda.synchronize()
    want = orc.dequantize(q.numpy().reshape(1, n), E4, s, 0)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), want.reshape(-1).view(np.uint32))


# ------------------------------------------------------------------ delayed scaler
def read_scaler(fq, st_dev):
    raw = st_dev.cpu().numpy().tobytes()
    return fq.Scaler.from_buffer_copy(raw)


def assert_scaler_equal(g, o):
    assert g.window == o.window and g.count == o.count and g.pos == o.pos and g.stat == o.stat
    assert np.array_equal(f32bits(np.array(g.ring[:g.window])), f32bits(np.array(o.ring[:o.window])))
    assert f32bits([g.scale])[0] == f32bits([o.scale])[0], (g.scale, o.scale)
    for f in ("max_val", "eps", "margin", "alpha"):
        assert f32bits([getattr(g, f)])[0] == f32bits([getattr(o, f)])[0]
    ge, oe = np.array([g.ema], np.float64).view(np.uint64)[0], np.array([o.ema], np.float64).view(np.uint64)[0]
    assert ge == oe or (np.isnan(g.ema) and np.isnan(o.ema)), (g.ema, o.ema)


@pytest.mark.parametrize("window,fmt,margin", [(16, E4, 1.0), (1, E4, 1.0), (5, E5, 1.1), (1024, E5, 1.0)])
def test_scaler_sequence(fq, orc, gpu, window, fmt, margin):
    st = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=gpu)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    fq.fp8q_delayed_scaler_init(st, window, MAXF[fmt], EPS, margin)
    o = orc.scaler_new(window, fmt, EPS, margin)
    rng = np.random.default_rng(window)
    seq = list((np.arange(1, 41) * 0.5).astype(np.float32)) + [np.float32(1e5), np.float32(0.0)]
    seq += list((rng.random(window + 20) * 100).astype(np.float32)) + [np.float32(0.0)] * 3
    for a in seq:
        amax.fill_(float(a))
        fq.fp8q_delayed_scaler_update(st, amax)
        orc.scaler_update(o, float(a))
        torch.cuda.synchronize()
        assert amax.item() == 0.0
        assert_scaler_equal(read_scaler(fq, st), o)


@pytest.mark.parametrize("window,fmt,margin,stat,alpha", [(16, E4, 1.0, 1, 0.0), (1024, E5, 1.1, 1, 0.0),
                                                         (37, E4, 1.0, 1, 0.0), (1, E5, 1.0, 1, 0.0),
                                                         (16, E4, 1.0, 2, 0.01), (1, E5, 1.1, 2, 1.0),
                                                         (1024, E4, 1.0, 2, 0.001), (5, E5, 1.0, 2, 0.3)])
def test_scaler_statistics_sequence(fq, orc, gpu, window, fmt, margin, stat, alpha):
    """Window mean (fp64 pairwise) and EMA (fp64 recurrence) scalers: state,
    EMA bits and scale identical to the oracle's after every step, over a
    ramp, a spike, zeros and random magnitudes spanning 30 octaves."""
    st = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=gpu)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    fq.fp8q_delayed_scaler_init_stat(st, window, MAXF[fmt], EPS, margin, stat, alpha)
    o = orc.scaler_new(window, fmt, EPS, margin, stat=stat, alpha=alpha)
    rng = np.random.default_rng(window + 7 * stat)
    seq = list((np.arange(1, 41) * 0.5).astype(np.float32)) + [np.float32(1e5), np.float32(0.0)]
    seq += list(np.exp2(rng.uniform(-15, 15, size=window + 20)).astype(np.float32)) + [np.float32(0.0)] * 3
    check_every = 1 if window < 64 else 17
    for t, a in enumerate(seq):
        amax.fill_(float(a))
        fq.fp8q_delayed_scaler_update(st, amax)
        orc.scaler_update(o, float(a))
        if t % check_every == 0 or t == len(seq) - 1:
            torch.cuda.synchronize()
            assert_scaler_equal(read_scaler(fq, st), o)


@pytest.mark.parametrize("stat,alpha", [(1, 0.0), (2, 0.25)])
def test_scaler_statistics_nan(fq, orc, gpu, stat, alpha):
    st = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=gpu)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    fq.fp8q_delayed_scaler_init_stat(st, 3, 448.0, EPS, 1.0, stat, alpha)
    o = orc.scaler_new(3, E4, stat=stat, alpha=alpha)
    for a in [1.0, 2.0, float("nan"), 3.0, 4.0, 5.0, 6.0]:
        amax.fill_(a)
        fq.fp8q_delayed_scaler_update(st, amax)
        orc.scaler_update(o, a)
        torch.cuda.synchronize()
        assert_scaler_equal(read_scaler(fq, st), o)


def test_scaler_nan_propagates(fq, orc, gpu):
    st = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=gpu)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    fq.fp8q_delayed_scaler_init(st, 3, 448.0, EPS, 1.0)
    o = orc.scaler_new(3, E4)
    for a in [1.0, 2.0, float("nan"), 3.0, 4.0, 5.0, 6.0]:
        amax.fill_(a)
        fq.fp8q_delayed_scaler_update(st, amax)
        orc.scaler_update(o, a)
        torch.cuda.synchronize()
        assert_scaler_equal(read_scaler(fq, st), o)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_delayed_scaling_steps(fq, orc, gpu, fmt):
    """Fused quantize + amax + scaler update over 24 steps of a
    drifting bf16 sequence (window 4): per-step codes and scales."""
    rows, cols, window = 512, 1024, 4
    sig = W.sigma_schedule(24, seed=2)
    st = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=gpu)
    amax = torch.zeros(1, dtype=torch.float32, device=gpu)
    fq.fp8q_delayed_scaler_init(st, window, MAXF[fmt], EPS, 1.0)
    scale_ptr = st.data_ptr() + fq.SCALER_SCALE_OFFSET
    o = orc.scaler_new(window, fmt)
    q = torch.empty(rows * cols, dtype=torch.uint8, device=gpu)
    for t, sg in enumerate(sig):
        if fmt == E4:
            x = W.delayed_step(rows, cols, sg, seed=100 + t)
        else:
            x = W.gradient(rows, cols, seed=100 + t, dtype=torch.bfloat16)
        xn = W.to_numpy_input(x)
        fq.fp8q_quantize_tensor(x.to(gpu), rows * cols, fmt, scale_ptr, q, amax)
        fq.fp8q_delayed_scaler_update(st, amax)
        want = orc.quantize_tensor(xn, fmt, o.scale)
        orc.scaler_update(o, float(orc.amax(xn)))
        torch.cuda.synchronize()
        assert_codes_equal(q.cpu().numpy(), want, f"step {t}")
        assert_scaler_equal(read_scaler(fq, st), o)


def test_delayed_scaling_full_config(fq, orc, gpu):
    """The delayed-scaling workload at its full size: 64 steps over bf16
    8192x8192 tensors, window 16, the activation copy x_t = bf16(sigma_t
    N(0,1)) (sigma_t log-uniform in [0.5, 50]) quantized to E4M3FN with its
    bf16 round trip, and the gradient copy g_t (|g| log-uniform in
    [1e-6, 1e-2], random sign) to E5M2, each with the scale its scaler
    derived from the earlier steps and the amax folded into the scaler's
    accumulator in the same pass (fp8q_quantize_tensor_delayed), then both
    scalers updated.  Every step: both scaler states (the new amax in the
    window, the scale) bit-exact against the oracle's sequence; codes
    bit-exact on 128 sampled rows every step and in full, with x's round
    trip, on the steps where the scale first moves and a few others."""
    rows = cols = 8192
    n = rows * cols
    steps, window = 64, 16
    sig = W.sigma_schedule(steps, seed=2)
    full_steps = {0, 15, 16, 17, 40, steps - 1}
    sample = np.unique(np.concatenate([np.arange(0, rows, 64) + np.arange(rows // 64) % 64, [rows - 1]]))
    si = torch.from_numpy(sample).to(gpu)
    tensors = {
        "x": (E4, lambda t: W.delayed_step(rows, cols, sig[t], seed=200 + t, device=gpu)),
        "g": (E5, lambda t: W.gradient(rows, cols, seed=300 + t, device=gpu, dtype=torch.bfloat16)),
    }
    state = {}
    for name, (fmt, _) in tensors.items():
        st = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=gpu)
        fq.fp8q_delayed_scaler_init(st, window, MAXF[fmt], EPS, 1.0)
        state[name] = (st, torch.empty(n, dtype=torch.uint8, device=gpu), orc.scaler_new(window, fmt, EPS, 1.0))
    y = torch.empty(n, dtype=torch.bfloat16, device=gpu)
    for t in range(steps):
        for name, (fmt, make) in tensors.items():
            st, q, o = state[name]
            x = make(t)
            fq.fp8q_quantize_tensor_delayed(x, n, fmt, st, q, y if name == "x" else None)
            fq.fp8q_delayed_scaler_update(st)
            xn = W.to_numpy_input(x)
            s_used = np.float32(o.scale)
            if t in full_steps:
                want = orc.quantize_tensor(xn, fmt, s_used)
                assert_codes_equal(q.cpu().numpy(), want, f"{name} step {t}")
                if name == "x":
                    wy = orc.dequantize(want.reshape(1, -1), fmt, np.array([s_used], np.float32), orc.GRAN_TENSOR,
                                        out_bf16=True).reshape(-1)
                    assert np.array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), wy), f"x round trip step {t}"
            else:
                want = orc.quantize_tensor(np.ascontiguousarray(xn.reshape(rows, cols)[sample]), fmt, s_used)
                assert_codes_equal(q.view(rows, cols)[si].cpu().numpy(), want, f"{name} step {t} (sampled rows)")
            orc.scaler_update(o, float(orc.amax(xn)))
            got = read_scaler(fq, st)
            assert_scaler_equal(got, o)
            assert got.amax_acc == 0.0, f"{name} accumulator not consumed at step {t}"
        if t in (0, 16, steps - 1):
            print(f"step {t}: s_x {state['x'][2].scale:.6g} s_g {state['g'][2].scale:.6g}", flush=True)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_quantize_tensor_delayed_micro_batches(fq, orc, gpu, fmt):
    """Several micro-batches of one step fold into the one window entry of
    the step (their joint amax, NaN winning), with no reset between steps;
    codes and the round trip as the per-tensor quantizer makes them with the
    state's scale; fp32 and bf16 inputs, ragged lengths."""
    window = 3
    st = torch.zeros(fq.SCALER_BYTES, dtype=torch.uint8, device=gpu)
    fq.fp8q_delayed_scaler_init(st, window, MAXF[fmt], EPS, 1.0)
    o = orc.scaler_new(window, fmt, EPS, 1.0)
    for t in range(7):
        amax_step = np.float32(0.0)
        for mb, (dtype, n) in enumerate([(torch.float32, 70_001), (torch.bfloat16, 4096 * 3 + 5)]):
            x = W.normal((n,), seed=500 + 10 * t + mb, std=float(3.0 ** (t - 2) * (mb + 1)), dtype=dtype)
            if t == 4 and mb == 1:
                x[77] = float("nan")
            xd = x.to(gpu)
            q = torch.empty(n, dtype=torch.uint8, device=gpu)
            y = torch.empty(n, dtype=torch.float32, device=gpu)
            fq.fp8q_quantize_tensor_delayed(xd, n, fmt, st, q, y)
            xn = W.to_numpy_input(x)
            wq = orc.quantize_tensor(xn, fmt, np.float32(o.scale))
            torch.cuda.synchronize()
            assert_codes_equal(q.cpu().numpy(), wq, f"step {t} mb {mb}")
            wy = orc.dequantize(wq.reshape(1, -1), fmt, np.array([o.scale], np.float32), orc.GRAN_TENSOR).reshape(-1)
            assert np.array_equal(f32bits(y.cpu().numpy()), f32bits(wy))
            a = orc.amax(xn)
            amax_step = a if (np.isnan(a) or np.isnan(amax_step)) else max(amax_step, a)
        got = read_scaler(fq, st)
        assert f32bits([got.amax_acc])[0] == f32bits([np.float32(np.nan) if np.isnan(amax_step) else amax_step])[0] \
            or (np.isnan(amax_step) and f32bits([got.amax_acc])[0] == 0x7FC00000)
        fq.fp8q_delayed_scaler_update(st)
        orc.scaler_update(o, float(amax_step))
        torch.cuda.synchronize()
        assert_scaler_equal(read_scaler(fq, st), o)
