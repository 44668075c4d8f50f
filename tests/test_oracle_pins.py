"""Pins for the CPU oracle: facts the pages and the mathematics fix, checked
without trusting the oracle's own formulas.

Each test names what pins it: a printed value on a page (tests/golden/*),
a closed form, an invariant, an independent brute force, or a library
routine (torch's float8/bf16 casts, numpy's IEEE float32 arithmetic,
Python's exact Fractions).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden

E4, E5 = 0, 1
FMT_NAME = {E4: "E4M3FN", E5: "E5M2"}
MAXF = {E4: 448.0, E5: 57344.0}
MAXCODE = {E4: 0x7E, E5: 0x7B}
TORCH_FP8 = {E4: torch.float8_e4m3fn, E5: torch.float8_e5m2}


def f32(v):
    return np.float32(v)


def bits_to_f32(u):
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


# ------------------------------------------------------------------ format table / decode
@pytest.mark.parametrize("fmt", [E4, E5])
def test_format_table_extremes(orc, fmt):
    """PyTorch-native FP8 article, section 1.2 table: max finite, min normal, min subnormal, bias."""
    g = golden("format_table.json")[FMT_NAME[fmt]]
    M, bias = g["mant_bits"], g["bias"]
    assert orc.decode(MAXCODE[fmt], fmt) == g["max_finite"]
    assert orc.decode(1 << M, fmt) == 2.0 ** (1 - bias)       # smallest normal: e=1, m=0
    assert orc.decode(1, fmt) == 2.0 ** (1 - bias - M)        # smallest subnormal: e=0, m=1
    assert orc.decode(bias << M, fmt) == 1.0                  # the exponent bias puts 1.0 at e=bias
    if fmt == E4:
        assert orc.decode(1 << M, fmt) == g["min_normal"]
        assert orc.decode(1, fmt) == g["min_subnormal"]
    else:
        assert orc.decode(1 << M, fmt) == 2.0 ** g["min_normal_pow2"]
        assert abs(orc.decode(1 << M, fmt) - g["min_normal_approx"]) < 1e-6
        assert orc.decode(1, fmt) == 2.0 ** g["min_subnormal_pow2"]
        assert abs(orc.decode(1, fmt) - g["min_subnormal_approx"]) < 1e-7


@pytest.mark.parametrize("fmt", [E4, E5])
def test_decode_exhaustive_structure(orc, fmt):
    """All 256 codes: special-value counts, strict monotonicity of the positive
    finite codes, and sign symmetry (the readings: E4M3FN has only 0x7F/0xFF as
    NaN, E5M2 has IEEE-style Inf/NaN at exponent 31)."""
    t = orc.decode_table(fmt)
    nan = np.isnan(t)
    inf = np.isinf(t)
    if fmt == E4:
        assert nan.sum() == 2 and inf.sum() == 0
        assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    else:
        assert nan.sum() == 6 and inf.sum() == 2
        assert list(np.nonzero(inf)[0]) == [0x7C, 0xFC]
    fin = ~(nan | inf)
    assert fin.sum() == (254 if fmt == E4 else 248)
    pos = [t[c] for c in range(128) if fin[c]]
    assert all(b > a for a, b in zip(pos, pos[1:]))
    assert pos[0] == 0.0 and pos[-1] == MAXF[fmt]
    for c in range(128):
        if fin[c]:
            assert t[c | 0x80] == -t[c]
    assert math.copysign(1.0, t[0x80]) == -1.0  # signed zero


@pytest.mark.parametrize("fmt", [E4, E5])
def test_decode_matches_torch(orc, fmt):
    """Library routine: torch's float8 dtypes decode all 256 bit patterns."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TORCH_FP8[fmt]).to(torch.float64).numpy()
    t = orc.decode_table(fmt)
    assert np.array_equal(np.isnan(ref), np.isnan(t))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], t[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(t[ok]))


# ------------------------------------------------------------------ encoder
@pytest.mark.parametrize("fmt", [E4, E5])
def test_scalar_experiment(orc, fmt):
    """PyTorch-native FP8 article, section 2.2: the scalar experiment."""
    g = golden("scalar_experiment.json")
    for v, code, val in zip(g["inputs"], g[FMT_NAME[fmt]]["codes"], g[FMT_NAME[fmt]]["values"]):
        c = orc.encode(v, fmt)
        assert c == code, (v, hex(c), hex(code))
        assert orc.decode(c, fmt) == val


@pytest.mark.parametrize("fmt", [E4, E5])
def test_round_trip_and_saturation(orc, fmt):
    """Invariant: enc(dec(c)) == c for every finite code (incl. -0 = 0x80);
    every |v| >= MAX and +-Inf saturate; NaN gives 0x7F."""
    for c in range(256):
        v = orc.decode(c, fmt)
        if math.isnan(v):
            continue
        if math.isinf(v):
            assert orc.encode(v, fmt) == (MAXCODE[fmt] | (c & 0x80))
            continue
        assert orc.encode(v, fmt) == c, hex(c)
    for v in (MAXF[fmt], MAXF[fmt] * 1.0001, 1e30, 3.4e38, float("inf")):
        assert orc.encode(v, fmt) == MAXCODE[fmt]
        assert orc.encode(-v, fmt) == MAXCODE[fmt] | 0x80
    assert orc.encode(float("nan"), fmt) == 0x7F
    assert orc.encode(-float("nan"), fmt) == 0x7F
    assert orc.encode(-0.0, fmt) == 0x80
    assert orc.encode(-1e-30, fmt) == 0x80


def _band(fmt):
    """fp32 binades that can produce a nonzero, non-saturated code, one extra on each side."""
    lo_exp, hi_exp = (-12, 9) if fmt == E4 else (-19, 16)
    return (127 + lo_exp) << 23, (127 + hi_exp + 1) << 23


@pytest.mark.parametrize("fmt", [E4, E5])
def test_encoder_matches_bruteforce_band(orc, encb, fmt):
    """Independent brute force (nearest listed value, ties to even code) on
    every non-negative fp32 pattern in the band where codes are non-trivial,
    plus a strided sample of all 2^32 patterns (both signs, subnormals, Inf,
    NaN)."""
    lo, hi = _band(fmt)
    chunk = 1 << 25
    for start in range(lo, hi, chunk):
        n = min(chunk, hi - start)
        a = orc.encode_bits_range(start, n, fmt)
        b = np.empty(n, dtype=np.uint8)
        encb.encb_bits(start, 1, n, fmt, b.ctypes.data)
        bad = np.nonzero(a != b)[0]
        assert bad.size == 0, (hex(start + int(bad[0])), hex(a[bad[0]]), hex(b[bad[0]]))
    stride = 4093
    n = (1 << 32) // stride
    b = np.empty(n, dtype=np.uint8)
    encb.encb_bits(0, stride, n, fmt, b.ctypes.data)
    u = (np.arange(n, dtype=np.uint64) * stride).astype(np.uint32)
    a = orc.encode_array(u.view(np.float32), fmt)
    assert np.array_equal(a, b)


@pytest.mark.skipif(os.environ.get("FP8Q_EXHAUSTIVE") != "1", reason="set FP8Q_EXHAUSTIVE=1 for all 2^32 patterns")
@pytest.mark.parametrize("fmt", [E4, E5])
def test_encoder_matches_bruteforce_all_2p32(orc, encb, fmt):
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        a = orc.encode_bits_range(start, chunk, fmt)
        b = np.empty(chunk, dtype=np.uint8)
        encb.encb_bits(start, 1, chunk, fmt, b.ctypes.data)
        assert np.array_equal(a, b), hex(start)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_encoder_matches_torch_cast(orc, fmt):
    """Library routine: torch's RNE float8 cast after clamping to +-MAX (the
    handbook's quant clamps before the cast).  Every bf16 pattern, and a
    random sample of fp32 patterns; NaN excluded (torch keeps its sign)."""
    h = np.arange(1 << 16, dtype=np.uint32) << 16
    r = np.random.default_rng(0).integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    for u in (h, r):
        x = u.view(np.float32)
        x = x[~np.isnan(x)]
        ref = torch.from_numpy(x.copy()).clamp(-MAXF[fmt], MAXF[fmt]).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
        assert np.array_equal(orc.encode_array(x, fmt), ref)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_encoder_sign_symmetry(orc, fmt):
    """Invariant: code(-v) = code(v) | 0x80 for every non-NaN v."""
    r = np.random.default_rng(1).integers(0, 1 << 31, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = r.view(np.float32)
    x = x[~np.isnan(x)]
    assert np.array_equal(orc.encode_array(-x, fmt), orc.encode_array(x, fmt) | 0x80)


# ------------------------------------------------------------------ amax / scale / quantize
def test_amax_cases(orc):
    x = np.array([0.5, -3.0, 2.0, -0.0], dtype=np.float32)
    assert orc.amax(x) == 3.0
    assert orc.amax(np.zeros(7, np.float32)) == 0.0
    assert orc.amax(np.array([1.0, -np.inf], np.float32)) == np.inf
    m = orc.amax(np.array([1.0, np.nan, 5.0], np.float32))
    assert np.isnan(m) and np.array([m], np.float32).view(np.uint32)[0] == 0x7FC00000
    # bf16 is widened exactly: 0xC040 = -3.0, 0x3F80 = 1.0
    assert orc.amax(np.array([0x3F80, 0xC040], np.uint16)) == 3.0
    rng = np.random.default_rng(2)
    y = rng.standard_normal(100_003).astype(np.float32)
    assert orc.amax(y) == np.abs(y).max()  # library reduction


@pytest.mark.parametrize("fmt", [E4, E5])
def test_scale_closed_forms(orc, fmt):
    """s = fl32(max(amax, eps) * margin / MAX): exact powers of two for
    amax = MAX * 2^k; the eps clamp for an all-zero granule; IEEE float32
    division (numpy) elsewhere."""
    for k in range(-20, 21):
        assert orc.scale(MAXF[fmt] * 2.0 ** k, fmt) == f32(2.0 ** k)
    eps = f32(1e-12)
    assert orc.scale(0.0, fmt) == eps / f32(MAXF[fmt])
    assert np.isnan(orc.scale(float("nan"), fmt))
    rng = np.random.default_rng(3)
    a = (rng.random(1000) * 1e4).astype(np.float32)
    for v in a[:200]:
        assert orc.scale(v, fmt) == f32(v) / f32(MAXF[fmt])
        assert orc.scale(v, fmt, margin=1.1) == (f32(v) * f32(1.1)) / f32(MAXF[fmt])


def test_exercise_outlier_5000(orc):
    """Handbook exercise 2: one value of 5000 sets the per-tensor scale to
    5000/448 ~ 11.2 and 0.01 quantizes to 0."""
    g = golden("exercise_outlier5000.json")
    x = np.concatenate([np.linspace(-1, 1, 1001, dtype=np.float32), np.array([g["outlier"]], np.float32)])
    s = orc.scale(orc.amax(x), E4)
    assert round(float(s), g["scale_approx_digits"]) == g["scale_approx"]
    assert float(s) == float(f32(5000.0) / f32(448.0))
    assert orc.quantize_value(g["small_value"], s, E4) == g["small_value_code"]
    qv = g["small_value"] / float(s)
    assert abs(qv - g["quotient_approx"]) < 0.00005 and qv < g["min_subnormal"] / 2
    q = orc.quantize_tensor(x, E4, s)
    deq = orc.decode_table(E4)[q] * float(s)
    inner = np.abs(x) <= 1
    # "only one or two significant digits": relative error of nonzero results
    # in [-1, 1] is large compared with E4M3's own 2^-4
    nz = inner & (deq != 0)
    assert np.max(np.abs(deq[nz] - x[nz]) / np.abs(x[nz])) > 0.1
    assert orc.quantize_value(5000.0, s, E4) == 0x7E


def _outlier_errors(orc, a):
    x = a.numpy()
    s = orc.scale(orc.amax(x), E4)
    q = orc.quantize_tensor(x, E4, s)
    y = orc.dequantize(q.reshape(x.shape), E4, np.array([s], np.float32), orc.GRAN_TENSOR)
    qb, sb = orc.quantize_1x128(x, E4)
    yb = orc.dequantize(qb, E4, sb, orc.GRAN_1x128)
    return orc.rel_err(y[:, 128:], x[:, 128:]), orc.rel_err(yb[:, 128:], x[:, 128:])


def test_outlier_experiment_printed_table(orc):
    """Handbook 'FP8 训练': the printed per-tensor vs per-1x128 table, reproduced
    digit for digit from the same seeded torch.randn inputs."""
    g = golden("outlier_experiment.json")
    torch.manual_seed(g["seed"])
    for f, pt, pb in zip(g["factors"], g["per_tensor_pct"], g["per_1x128_pct"]):
        a = torch.randn(*g["shape"])
        a[:, : g["outlier_cols"]] *= f
        t, b = _outlier_errors(orc, a)
        assert round(100 * t, 1) == pt, (f, t)
        assert round(100 * b, 1) == pb, (f, b)


def test_outlier_experiment_other_seeds(orc):
    """The same experiment's claim for any seed: 1x128 error stays near 2.6%
    (E4M3's own precision); per-tensor error grows with the outlier."""
    for seed in (1, 2, 3):
        torch.manual_seed(seed)
        prev = 0.0
        for f in (1e2, 1e4, 3e4):
            a = torch.randn(256, 1024)
            a[:, :4] *= f
            t, b = _outlier_errors(orc, a)
            assert 0.024 <= b <= 0.028
            assert t > prev
            prev = t
        assert prev > 0.10


# ------------------------------------------------------------------ the handbook's formula in torch
# Handbook "FP8 训练": quantizing is dividing by the dequantization scale in
# float32, clamping to +-MAX and casting to float8; the per-tensor scale is
# the tensor's amax over MAX, the per-block scale the block's amax, clamped
# below at 1e-12, over MAX.  Written here with torch's own CPU float32
# arithmetic (IEEE division) and its RNE float8 cast, independently of the
# oracle, and compared code for code and scale for scale.  NaN is left out:
# torch's cast keeps a NaN's sign, the reading here maps every NaN to 0x7F.
def _torch_codes(x, s, fmt):
    """(x / s) in float32, clamped to +-MAX, cast to float8: the code bytes."""
    return (x / s).clamp(-MAXF[fmt], MAXF[fmt]).to(TORCH_FP8[fmt]).view(torch.uint8)


def _torch_per_tensor(x, fmt):
    s = x.abs().max() / MAXF[fmt]
    return _torch_codes(x, s, fmt), s


def _torch_per_block(x, rows, cols, fmt):
    R, C = x.shape
    b = x.reshape(R // rows, rows, C // cols, cols)
    s = b.abs().amax(dim=(1, 3), keepdim=True).clamp(min=1e-12) / MAXF[fmt]
    q = _torch_codes(b, s, fmt).reshape(R, C)
    return q, s.reshape(R // rows, C // cols)


def _as_np(t):
    return t.contiguous().numpy()


def test_handbook_formula_outlier_tensors(orc):
    """The printed experiment's tensors (seed 0, columns 0-3 scaled by 1e2,
    1e4, 3e4): per-tensor and 1x128 codes and scales of the oracle equal the
    handbook's formula evaluated by torch, bit for bit, in both formats."""
    g = golden("outlier_experiment.json")
    torch.manual_seed(g["seed"])
    for f in g["factors"]:
        a = torch.randn(*g["shape"])
        a[:, : g["outlier_cols"]] *= f
        x = a.numpy()
        for fmt in (E4, E5):
            qt, st = _torch_per_tensor(a, fmt)
            s = orc.scale(orc.amax(x), fmt)
            assert np.float32(st.item()) == s
            assert np.array_equal(orc.quantize_tensor(x, fmt, s), _as_np(qt)), (f, fmt)
            for br, bc in ((1, 128), (128, 128)):
                qb, sb = _torch_per_block(a, br, bc, fmt)
                oq, os_ = orc.quantize_blocks(x, br, bc, fmt)
                assert np.array_equal(os_, _as_np(sb)), (f, fmt, br)
                assert np.array_equal(oq, _as_np(qb)), (f, fmt, br)


# per-tensor scales across regimes: ordinary non-powers of two, a scale whose
# reciprocal is far from exact, tiny (fp32 subnormal) and huge scales, and one
# where quotients land on FP8 rounding midpoints
_SCALE_REGIMES = [0.0173, 1.0 / 3.0, 11.160714149475098, 7.0e-3, 3.3e-39, 1.7e-42, 2.9e35, 0.5, 1.0]


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_handbook_formula_scale_regimes(orc, fmt, dtype):
    """Random fp32 / bf16 data (magnitudes over many octaves, NaN removed)
    quantized with a given per-tensor scale: oracle codes == torch's
    float32 (x / s).clamp(-MAX, MAX).to(float8), for every scale regime."""
    rng = np.random.default_rng(11)
    for s in _SCALE_REGIMES:
        s32 = np.float32(s)
        base = rng.standard_normal(1 << 16) * np.exp2(rng.uniform(-30, 30, 1 << 16))
        x = (base * float(s32) * MAXF[fmt] / 64.0).astype(np.float32)
        # quotients exactly on rounding midpoints of the format, and +-0
        mids = (np.arange(1, 200, dtype=np.float32) * np.float32(2.0 ** -10)) * s32
        x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0])])
        x = x[np.isfinite(x) | np.isinf(x)]
        if dtype == "bf16":
            xt = torch.from_numpy(x).to(torch.bfloat16)
            xin = xt.view(torch.int16).numpy().view(np.uint16)
            xt = xt.float()
        else:
            xt = torch.from_numpy(x)
            xin = x
        ref = _as_np(_torch_codes(xt, torch.tensor(s32), fmt))
        assert np.array_equal(orc.quantize_tensor(xin, fmt, s32), ref), s


def _midpoints(fmt):
    """Every point halfway between two neighbouring non-negative finite
    values of the format (from its bit layout: bias 7 / 15, 3 / 2 mantissa
    bits), as fp64."""
    M, bias, emax = (3, 7, 15) if fmt == E4 else (2, 15, 30)
    vals = [m * 2.0 ** (1 - bias - M) for m in range(1 << M)]
    for e in range(1, emax + 1):
        vals += [(1 + m / 2 ** M) * 2.0 ** (e - bias) for m in range(1 << M)]
    v = np.array([t for t in vals if t <= MAXF[fmt]])
    return (v[:-1] + v[1:]) / 2


def test_quotient_is_correctly_rounded_float32(orc):
    """The quotient step q = enc(fl32(x / s)) against (float)((double)x /
    (double)s): rounding the double quotient once more to fp32 is the
    correctly rounded fp32 quotient (53 >= 2*24 + 2: double rounding of a
    quotient is innocuous, Figueroa 1995).  Checked through the codes on a
    large random sample of (x, s) pairs, including every exponent range."""
    rng = np.random.default_rng(12)
    ns, per = 256, 1 << 12
    # scales from fp32 subnormals to 2^100, every mantissa; random fp32 data
    sb = rng.integers(0x00000001, 0x71800000, size=ns, dtype=np.uint64).astype(np.uint32)
    scales = sb.view(np.float32)
    for fmt in (E4, E5):
        for i, v in enumerate(scales):
            xb = rng.integers(0, 1 << 32, size=per, dtype=np.uint64).astype(np.uint32)
            x = xb.view(np.float32)
            # half of the data near the scale, where the codes are not all 0 or MAX
            x[: per // 2] = (rng.standard_normal(per // 2) * float(v) * 64.0).astype(np.float32)
            # and values whose quotients lie on or next to the format's rounding
            # midpoints, where one ulp of the quotient decides the code
            mids = _midpoints(fmt)
            near = (mids * np.float64(v)).astype(np.float32)
            near = np.concatenate([np.nextafter(near, np.float32(np.inf)), near, np.nextafter(near, np.float32(0))])
            x = np.concatenate([x, near, -near])
            x = x[~np.isnan(x)]
            y = (x.astype(np.float64) / np.float64(v)).astype(np.float32)
            want = orc.encode_array(y, fmt)
            assert np.array_equal(orc.quantize_tensor(x, fmt, v), want), (fmt, float(v))
            if i < 4:
                got = np.array([orc.quantize_value(float(a), float(v), fmt) for a in x[:512]], dtype=np.uint8)
                assert np.array_equal(got, want[:512])


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("br,bc", [(1, 128), (128, 128)])
def test_block_quantize_invariants(orc, fmt, br, bc):
    """Each block's scale is scale(amax of the block) (numpy reduction and
    float32 division); the block's largest-magnitude element encodes to
    +-MAX; every code equals the per-element quantize with its block's
    scale; an all-zero block takes the eps scale and codes 0x00 / 0x80."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((256, 384)) * np.exp(rng.standard_normal((256, 1)) * 3)).astype(np.float32)
    x[0:128, 0:128] = 0.0
    x[5, 7] = -0.0
    q, s = orc.quantize_blocks(x, br, bc, fmt)
    for rb in range(256 // br):
        for cb in range(384 // bc):
            blk = x[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc]
            am = np.abs(blk).max()
            want = max(am, f32(1e-12)) / f32(MAXF[fmt])
            assert s[rb, cb] == f32(want)
            qb = q[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc]
            if am > 0:
                i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                assert qb[i] & 0x7F == MAXCODE[fmt]
            else:
                assert set(np.unique(qb)) <= {0x00, 0x80}
    assert q[5, 7] == 0x80
    for (r, c) in [(3, 200), (200, 3), (255, 383), (130, 129)]:
        assert q[r, c] == orc.quantize_value(x[r, c], s[r // br, c // bc], fmt)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_dequantize_is_one_float32_product(orc, fmt):
    """x^ = fl32(dec(q) * s): numpy's IEEE float32 multiply of the decoded
    value; the bf16 output is torch's round-to-nearest-even bf16 cast."""
    rng = np.random.default_rng(5)
    q = np.tile(np.arange(256, dtype=np.uint8), 8).reshape(8, 256)
    t = orc.decode_table(fmt)
    fin = ~np.isnan(t) & ~np.isinf(t)
    q = np.where(fin[q], q, 0).astype(np.uint8)
    s = (rng.random((8, 2)) * 10 + 1e-3).astype(np.float32)
    y = orc.dequantize(q, fmt, s, orc.GRAN_1x128)
    ref = t[q].astype(np.float32) * np.repeat(s, 128, axis=1)
    assert np.array_equal(y, ref)
    yb = orc.dequantize(q, fmt, s, orc.GRAN_1x128, out_bf16=True)
    refb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, refb)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_dequantize_nan_results_are_the_quiet_nan(orc, fmt):
    """Every NaN the dequantizer writes is the quiet NaN 0x7FC00000 (0x7FC0
    in bf16), whatever produced it: a NaN code, 0 * Inf (scale +Inf) or a
    NaN scale; +Inf scales give signed infinities for nonzero codes."""
    nan_code = 0x7F
    q = np.array([[0x00, 0x80, nan_code, 0x38, 0xB8]], np.uint8)  # +0, -0, NaN, +1 (E4) / +0.5.. (E5), -
    for s, want_inf in ((np.float32(np.inf), True), (np.float32(np.nan), False), (np.float32(-np.inf), True)):
        y = orc.dequantize(q, fmt, np.array([s], np.float32), orc.GRAN_TENSOR).reshape(-1)
        bits = y.view(np.uint32)
        if want_inf:
            assert bits[0] == bits[1] == bits[2] == 0x7FC00000
            assert np.isinf(y[3]) and np.isinf(y[4]) and np.sign(y[3]) == -np.sign(y[4])
        else:
            assert np.all(bits == 0x7FC00000)
        yb = orc.dequantize(q, fmt, np.array([s], np.float32), orc.GRAN_TENSOR, out_bf16=True).reshape(-1)
        assert np.all(yb[:3] == 0x7FC0)


# ------------------------------------------------------------------ delayed scaler
def test_delayed_scaler_ramp_closed_form(orc):
    """PyTorch-native FP8 article, section 4.2 DelayedScaler(window=16): the
    scale starts at 1.0, stays there until 16 amaxes are seen, then is
    max(last 16 amax) / 448.  With amax_t = t + 1 the scale in force at step
    t >= 16 is fl32(t / 448)."""
    st = orc.scaler_new(16, E4)
    for t in range(64):
        used = st.scale
        if t <= 15:
            assert used == 1.0
        else:
            assert used == f32(t) / f32(448.0)
        orc.scaler_update(st, float(t + 1))
    assert st.count == 16 and st.pos == 64 % 16


def test_delayed_scaler_spike_is_forgotten(orc):
    """A spike at step j sets the scale for steps j+1 .. j+16 and is gone at j+17."""
    j = 30
    st = orc.scaler_new(16, E5)
    used = []
    for t in range(80):
        used.append(st.scale)
        orc.scaler_update(st, 1000.0 if t == j else 2.0)
    spike = f32(1000.0) / f32(57344.0)
    base = f32(2.0) / f32(57344.0)
    for t in range(80):
        if t < 16:
            assert used[t] == 1.0
        elif j + 1 <= t <= j + 16:
            assert used[t] == spike, t
        else:
            assert used[t] == base, t


def test_window_one_is_current_scaling(orc):
    st = orc.scaler_new(1, E4)
    rng = np.random.default_rng(6)
    for a in rng.random(20) * 100:
        orc.scaler_update(st, a)
        assert st.scale == orc.scale(a, E4)
    with pytest.raises(ValueError):
        orc.scaler_new(0, E4)


def fl32_of(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32, ties to even (by exact
    comparison with the neighbouring floats, no double rounding)."""
    c = np.float32(float(fr))
    best = None
    for v in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(v)) - fr)
        if best is None or d < best[0] or (d == best[0] and (int(v.view(np.uint32)) & 1) == 0):
            best = (d, v)
    return best[1]


def test_scaler_mean_of_window_closed_forms(orc):
    """Window mean ([A] 4.2 names the mean as the gentler choice): a ramp
    amax_t = t + 1 gives the mean (2t - W + 3)/2 of the last W values, a
    constant gives the constant; the scale is fl32(fl32(mean)*margin)/MAX and
    stays 1.0 until the window is full."""
    for W in (1, 5, 16, 1024):
        st = orc.scaler_new(W, E4, stat=orc.STAT_MEAN, margin=1.1)
        for t in range(W + 40):
            used = st.scale
            if t < W:
                assert used == 1.0
            else:
                # values 1..t in the ring, the last W of them are t-W+1 .. t
                mean = Fraction(sum(range(t - W + 1, t + 1)), W)
                want = f32(f32(fl32_of(mean)) * f32(1.1)) / f32(448.0)
                assert used == want, (W, t)
            orc.scaler_update(st, float(t + 1))


def test_scaler_mean_random_windows_match_exact_mean(orc):
    """For random amax histories of every magnitude the mean statistic is the
    exact rational mean rounded once to fp32 (the fp64 pairwise sum is far
    more precise than the fp32 result)."""
    rng = np.random.default_rng(31)
    for trial in range(60):
        W = int(rng.integers(1, 1025))
        st = orc.scaler_new(W, E5, stat=orc.STAT_MEAN)
        vals = (np.exp(rng.normal(0, 6, size=W + int(rng.integers(0, 50))))).astype(np.float32)
        for v in vals:
            orc.scaler_update(st, float(v))
        last = vals[-W:]
        mean = sum((Fraction(float(v)) for v in last), Fraction(0)) / W
        m = fl32_of(mean)
        assert st.scale == max(m, f32(orc.EPS)) / f32(57344.0), trial
        assert st.scale <= max(last.max(), f32(orc.EPS)) / f32(57344.0)


def test_scaler_mean_nan_leaves_with_the_window(orc):
    st = orc.scaler_new(4, E4, stat=orc.STAT_MEAN)
    seq = [1.0, 2.0, float("nan"), 3.0, 4.0, 5.0, 6.0, 7.0]
    for t, a in enumerate(seq):
        orc.scaler_update(st, a)
        if 3 <= t <= 5:
            assert np.isnan(st.scale)
    assert st.scale == f32(5.5) / f32(448.0)


def test_scaler_ema_closed_forms(orc):
    """EMA ([A] 4.2: smoothing of amax over the history): alpha = 1/2 after
    one value A and then zeros halves exactly each step, e_t = A*2^-t; alpha
    = 1 is current scaling; a constant history keeps the constant."""
    st = orc.scaler_new(1, E4, stat=orc.STAT_EMA, alpha=0.5)
    A = 3000.0
    orc.scaler_update(st, A)
    assert st.scale == f32(A) / f32(448.0)
    for t in range(1, 60):
        orc.scaler_update(st, 0.0)
        e = f32(A * 2.0 ** -t)
        assert st.ema == A * 2.0 ** -t
        assert st.scale == max(e, f32(orc.EPS)) / f32(448.0), t
    cur = orc.scaler_new(1, E5, stat=orc.STAT_EMA, alpha=1.0)
    rng = np.random.default_rng(8)
    for a in rng.random(30) * 1e4:
        orc.scaler_update(cur, a)
        assert cur.scale == orc.scale(a, E5)
    k = orc.scaler_new(16, E4, stat=orc.STAT_EMA, alpha=0.01, margin=1.1)
    for t in range(40):
        assert k.scale == (1.0 if t < 16 else f32(f32(f32(7.25) * f32(1.1)) / f32(448.0)))
        orc.scaler_update(k, 7.25)
    with pytest.raises(ValueError):
        orc.scaler_new(4, E4, stat=orc.STAT_EMA, alpha=0.0)


def test_scaler_ema_moves_toward_new_values(orc):
    """Between the old EMA and the new amax, never past either, and within
    one fp64 rounding step of alpha*a + (1-alpha)*e computed exactly."""
    rng = np.random.default_rng(9)
    st = orc.scaler_new(1, E4, stat=orc.STAT_EMA, alpha=0.125)
    prev = None
    for a in (rng.random(200) * 100).astype(np.float32):
        orc.scaler_update(st, float(a))
        if prev is not None:
            lo, hi = min(prev, float(a)), max(prev, float(a))
            assert lo <= st.ema <= hi
            exact = Fraction(0.125) * Fraction(float(a)) + Fraction(0.875) * Fraction(prev)
            assert abs(Fraction(st.ema) - exact) <= abs(exact) * Fraction(1, 2 ** 51)
        prev = st.ema


# ------------------------------------------------------------------ GEMM
def _rand_codes(rng, shape, fmt, lim=None):
    t_ok = {E4: [c for c in range(256) if c not in (0x7F, 0xFF)],
            E5: [c for c in range(256) if (c & 0x7F) < 0x7C]}[fmt]
    return rng.choice(np.array(t_ok, dtype=np.uint8), size=shape)


def _exact_gemm(orc, A, fa, sA, B, fb, sB, gb):
    ta = {c: Fraction(orc.decode(c, fa)) for c in range(256) if math.isfinite(orc.decode(c, fa))}
    tb = {c: Fraction(orc.decode(c, fb)) for c in range(256) if math.isfinite(orc.decode(c, fb))}
    M, K = A.shape
    N = B.shape[0]
    C = np.empty((M, N))
    D = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            c = Fraction(0)
            d = Fraction(0)
            for kb in range(K // 128):
                coef = Fraction(float(sA[m, kb])) * Fraction(float(sB[n // 128, kb] if gb == 2 else sB[n, kb]))
                p = sum((ta[A[m, k]] * tb[B[n, k]] for k in range(kb * 128, kb * 128 + 128)), Fraction(0))
                pa = sum((abs(ta[A[m, k]] * tb[B[n, k]]) for k in range(kb * 128, kb * 128 + 128)), Fraction(0))
                c += coef * p
                d += abs(coef) * pa
            C[m, n] = float(c)
            D[m, n] = float(d)
    return C, D


@pytest.mark.parametrize("fa,fb,gb", [(E4, E4, 2), (E5, E4, 2), (E5, E4, 1), (E5, E5, 1), (E4, E5, 2)])
def test_gemm_matches_exact_rationals(orc, fa, fb, gb):
    """Brute force in exact rational arithmetic (Fractions) on tiny inputs."""
    rng = np.random.default_rng(7)
    M, N, K = 2, 256, 256
    A = _rand_codes(rng, (M, K), fa)
    B = _rand_codes(rng, (N, K), fb)
    sA = (rng.random((M, K // 128)) * 3 + 0.01).astype(np.float32)
    sB = (rng.random(((N // 128) if gb == 2 else N, K // 128)) * 3 + 0.01).astype(np.float32)
    C, D = orc.gemm_blockscaled(A, fa, sA, B, fb, sB, gb)
    Ce, De = _exact_gemm(orc, A, fa, sA, B, fb, sB, gb)
    assert np.all(np.abs(C - Ce) <= 4 * 2.0 ** -52 * De)
    assert np.allclose(D, De, rtol=1e-15, atol=0)
    Cr, Dr = orc.gemm_blockscaled(A, fa, sA, B, fb, sB, gb, rows=np.array([1]))
    assert np.array_equal(Cr[0], C[1]) and np.array_equal(Dr[0], D[1])


def test_gemm_unit_scales_is_integer_matmul(orc):
    """With unit scales and K = 128 the GEMM is an integer matmul (numpy int64)."""
    rng = np.random.default_rng(8)
    # E4M3 codes of the integers 1..16: 1.0 is 0x38; integers m in [8,16) sit at 0x50 + (m - 8)
    ints = np.arange(-16, 17)
    code = {0: 0x00}
    for v in range(1, 17):
        c = next(c for c in range(128) if orc.decode(c, E4) == v)
        code[v], code[-v] = c, c | 0x80
    Ai = rng.choice(ints, size=(8, 128))
    Bi = rng.choice(ints, size=(128, 128))
    A = np.vectorize(code.get)(Ai).astype(np.uint8)
    B = np.vectorize(code.get)(Bi).astype(np.uint8)
    C, _ = orc.gemm_blockscaled(A, E4, np.ones((8, 1), np.float32), B, E4, np.ones((1, 1), np.float32), 2)
    assert np.array_equal(C, (Ai @ Bi.T).astype(np.float64))


def test_gemm_identity_b(orc):
    """B = identity codes (1.0 on the diagonal) with unit B scales returns dec(A) * sA."""
    rng = np.random.default_rng(9)
    M, K = 4, 256
    A = _rand_codes(rng, (M, K), E4)
    sA = (rng.random((M, 2)) + 0.5).astype(np.float32)
    B = np.zeros((K, K), np.uint8)
    B[np.arange(K), np.arange(K)] = 0x38
    C, _ = orc.gemm_blockscaled(A, E4, sA, B, E4, np.ones((2, 2), np.float32), 2)
    t = orc.decode_table(E4)
    want = t[A] * np.repeat(sA.astype(np.float64), 128, axis=1)
    assert np.array_equal(C, want)


def test_rel_err_matches_numpy_norm(orc):
    rng = np.random.default_rng(10)
    x = rng.standard_normal((17, 33)).astype(np.float32)
    y = x + rng.standard_normal((17, 33)).astype(np.float32) * 0.01
    want = np.linalg.norm(y.astype(np.float64) - x.astype(np.float64)) / np.linalg.norm(x.astype(np.float64))
    assert abs(orc.rel_err(y, x) - want) < 1e-14


# ------------------------------------------------------------------ MX (microscaling) FP8
# The MX conversion of the OCP MX v1.0 specification (section 6.3): blocks of
# 32 elements share X = 2^(floor(log2 max|V|) - emax_elem), stored as the
# E8M0 byte e + 127; elements are RNE-cast with clamping to the largest normal.
EMAX = {E4: 8, E5: 15}


def _mx_block(vals):
    return np.array([vals + [0.0] * (32 - len(vals))], dtype=np.float32)


@pytest.mark.parametrize("fmt", [E4, E5])
def test_mx_scale_byte_closed_forms(orc, fmt):
    """Scale byte = floor(log2 amax) - emax + 127 at and between powers of two,
    and the block maximum lands in [2^emax, 2^(emax+1)) after scaling."""
    for amax, fl in [(1.0, 0), (1.5, 0), (1.9999, 0), (2.0, 1), (3.0, 1), (448.0, 8), (0.75, -1),
                     (2.0 ** -20, -20), (2.0 ** 100 * 1.3, 100)]:
        _, s = orc.quantize_mx(_mx_block([amax, -amax / 3]), fmt)
        assert int(s[0, 0]) == fl - EMAX[fmt] + 127, (amax, s)
    # the largest representable block maximum with scale 2^0 is exactly the format's max
    q, s = orc.quantize_mx(_mx_block([MAXF[fmt]]), fmt)
    if fmt == E4:
        assert int(s[0, 0]) == 127 and int(q[0, 0]) == MAXCODE[fmt]


@pytest.mark.parametrize("fmt", [E4, E5])
def test_mx_elements_match_torch_cast(orc, fmt):
    """Element codes equal torch's float8 cast of V / X (exact power-of-two
    division) wherever that cast does not overflow; values between the
    format's max and the next binade clamp to the max code."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 4)).astype(np.float32)
    q, s = orc.quantize_mx(x, fmt)
    X = np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)
    y = (x.astype(np.float64) / X).astype(np.float32)
    over = np.abs(y) > MAXF[fmt]
    tq = torch.from_numpy(np.where(over, 0, y)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(q[~over], tq[~over])
    assert np.all((q[over] & 0x7F) == MAXCODE[fmt]) and np.array_equal(q[over] >> 7, (y[over] < 0).astype(np.uint8))


@pytest.mark.parametrize("fmt", [E4, E5])
def test_mx_power_of_two_equivariance(orc, fmt):
    """Scaling a block by 2^k leaves every code unchanged and adds k to the scale byte."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    q0, s0 = orc.quantize_mx(x, fmt)
    for k in (-30, -7, -1, 1, 5, 40):
        q, s = orc.quantize_mx(np.ldexp(x, k).astype(np.float32), fmt)
        assert np.array_equal(q, q0) and np.array_equal(s.astype(np.int64), s0.astype(np.int64) + k)


def test_mx_special_blocks(orc):
    """Zero block: scale byte 0 (2^-127) and zero codes, signs kept; a NaN or an
    Inf anywhere: NaN scale 0xFF and NaN codes."""
    x = np.zeros((4, 32), np.float32)
    x[0, 3] = -0.0
    x[1, 5] = np.nan
    x[2, 7] = -np.inf
    x[3, :] = 1.0
    q, s = orc.quantize_mx(x, E4)
    assert int(s[0, 0]) == 0 and np.all(q[0, :3] == 0) and q[0, 3] == 0x80
    assert int(s[1, 0]) == 0xFF and np.all(q[1] == 0x7F)
    assert int(s[2, 0]) == 0xFF and np.all(q[2] == 0x7F)
    assert int(s[3, 0]) == 119
    y = orc.dequantize_mx(q, E4, s)
    assert np.all(np.isnan(y[1])) and np.all(y[3] == 1.0) and np.signbit(y[0, 3])


@pytest.mark.parametrize("fmt", [E4, E5])
def test_mx_dequantize_closed_form(orc, fmt):
    """Every finite code times 2^(byte - 127), for a spread of scale bytes,
    against Python's exact ldexp of the decoded value."""
    codes = np.array([c for c in range(256) if math.isfinite(orc.decode(c, fmt))], np.uint8)
    n = (codes.size // 32) * 32
    codes = codes[:n].reshape(-1, 32)
    for b in (1, 60, 127, 128, 200, 254):
        s = np.full((codes.shape[0], 1), b, np.uint8)
        y = orc.dequantize_mx(codes, fmt, s)
        want = np.array([[np.float32(math.ldexp(orc.decode(int(c), fmt), b - 127)) for c in row] for row in codes])
        assert np.array_equal(y.view(np.uint32), want.astype(np.float32).view(np.uint32)), b


@pytest.mark.parametrize("fmt", [E4, E5])
def test_mx_round_trip_error_bound(orc, fmt):
    """|dequant(quant(x)) - x| <= max(|x| * 2^-(M+1), X * 2^(emin - M - 1)) for
    unclamped values (half an ulp, or half the subnormal quantum)."""
    M = 3 if fmt == E4 else 2
    emin = -6 if fmt == E4 else -14
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((32, 256)) * np.exp(rng.standard_normal((32, 8)).repeat(32, axis=1) * 3)).astype(np.float32)
    q, s = orc.quantize_mx(x, fmt)
    y = orc.dequantize_mx(q, fmt, s).astype(np.float64)
    X = np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)
    ok = np.abs(x) <= MAXF[fmt] * X
    bound = np.maximum(np.abs(x) * 2.0 ** -(M + 1), X * 2.0 ** (emin - M - 1))
    assert np.all(np.abs(y - x)[ok] <= bound[ok])


def _exact_gemm_mx(orc, A, fa, sA, B, fb, sB):
    ta = {c: Fraction(orc.decode(c, fa)) for c in range(256) if math.isfinite(orc.decode(c, fa))}
    tb = {c: Fraction(orc.decode(c, fb)) for c in range(256) if math.isfinite(orc.decode(c, fb))}
    M, K = A.shape
    N = B.shape[0]
    C = np.zeros((M, N))
    D = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            c = Fraction(0)
            d = Fraction(0)
            for kb in range(K // 32):
                coef = Fraction(2) ** (int(sA[m, kb]) + int(sB[n, kb]) - 254)
                p = sum(ta[A[m, k]] * tb[B[n, k]] for k in range(32 * kb, 32 * kb + 32))
                pa = sum(abs(ta[A[m, k]] * tb[B[n, k]]) for k in range(32 * kb, 32 * kb + 32))
                c += coef * p
                d += coef * pa
            C[m, n] = float(c)
            D[m, n] = float(d)
    return C, D


@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4), (E4, E5)])
def test_gemm_mx_matches_exact_rationals(orc, fa, fb):
    rng = np.random.default_rng(24)
    M, N, K = 2, 16, 128
    A = _rand_codes(rng, (M, K), fa)
    B = _rand_codes(rng, (N, K), fb)
    sA = rng.integers(100, 150, size=(M, K // 32)).astype(np.uint8)
    sB = rng.integers(100, 150, size=(N, K // 32)).astype(np.uint8)
    C, D = orc.gemm_mx(A, fa, sA, B, fb, sB)
    Ce, De = _exact_gemm_mx(orc, A, fa, sA, B, fb, sB)
    assert np.all(np.abs(C - Ce) <= 4 * 2.0 ** -52 * De)
    assert np.allclose(D, De, rtol=1e-15, atol=0)


def test_gemm_mx_unit_scales_is_integer_matmul(orc):
    """Scale bytes 127 (2^0) and codes of small integers: an integer matmul."""
    rng = np.random.default_rng(25)
    ints = np.arange(-16, 17)
    code = {0: 0x00}
    for v in range(1, 17):
        c = next(c for c in range(128) if orc.decode(c, E4) == v)
        code[v], code[-v] = c, c | 0x80
    Ai = rng.choice(ints, size=(8, 96))
    Bi = rng.choice(ints, size=(40, 96))
    A = np.vectorize(code.get)(Ai).astype(np.uint8)
    B = np.vectorize(code.get)(Bi).astype(np.uint8)
    C, _ = orc.gemm_mx(A, E4, np.full((8, 3), 127, np.uint8), B, E4, np.full((40, 3), 127, np.uint8))
    assert np.array_equal(C, (Ai @ Bi.T).astype(np.float64))


# ------------------------------------------------------------------ GEMM with quantized output
def small_int_codes(orc, shape, rng, fmt):
    """Codes whose values are the integers -4 .. 4 (exact in both formats)."""
    vals = rng.integers(-4, 5, size=shape).astype(np.float32)
    return orc.encode_array(vals, fmt).reshape(shape), vals


def test_gemm_q_is_quantized_integer_matmul(orc):
    """With small-integer codes and power-of-two scales every sum is exact, so
    C equals an int64 matmul scaled by powers of two; the codes and scales
    must be quantize_1x128 of that C, blocks running along N (128 columns
    of one output row)."""
    rng = np.random.default_rng(12)
    M, N, K = 5, 256, 384
    for fa, fb, fc in ((E4, E4, E4), (E5, E4, E5)):
        A, av = small_int_codes(orc, (M, K), rng, fa)
        B, bv = small_int_codes(orc, (N, K), rng, fb)
        ea = rng.integers(-2, 3, size=(M, K // 128))
        eb = rng.integers(-2, 3, size=(N // 128, K // 128))
        sA = np.ldexp(np.float32(1), ea).astype(np.float32)
        sB = np.ldexp(np.float32(1), eb).astype(np.float32)
        C = np.zeros((M, N))
        for kb in range(K // 128):
            blk = av[:, 128 * kb:128 * kb + 128].astype(np.int64) @ bv[:, 128 * kb:128 * kb + 128].astype(np.int64).T
            C += blk * np.ldexp(1.0, ea[:, kb])[:, None] * np.repeat(np.ldexp(1.0, eb[:, kb]), 128)[None, :]
        q, s, C32 = orc.gemm_blockscaled_q(A, fa, sA, B, fb, sB, orc.GRAN_128x128, fc)
        assert np.array_equal(C32, C.astype(np.float32))
        for r in range(M):
            for cb in range(N // 128):
                amax = np.float32(np.abs(C[r, 128 * cb:128 * cb + 128]).max())
                assert s[r, cb] == np.float32(max(amax, np.float32(orc.EPS)) / np.float32(orc.MAX_FINITE[fc]))
        wq, _ = orc.quantize_blocks(C.astype(np.float32), 1, 128, fc)
        assert np.array_equal(q, wq)


def test_gemm_q_row_scale_closed_form(orc):
    """One nonzero per A row picks out one B row, so C's row r is B's row
    (r mod N) transposed; its 1x128 scales are fl32(amax / MAX) of those
    128-column pieces and a column of zeros in a block leaves code 0."""
    M, N, K = 3, 128, 128
    A = np.zeros((M, K), np.uint8)
    for r in range(M):
        A[r, r] = 0x38  # 1.0
    rng = np.random.default_rng(2)
    B, bv = small_int_codes(orc, (N, K), rng, E4)
    B[:, 0] = 0
    bv[:, 0] = 0
    q, s, C32 = orc.gemm_blockscaled_q(A, E4, np.ones((M, 1), np.float32), B, E4, np.ones((1, 1), np.float32),
                                       orc.GRAN_128x128, E4)
    for r in range(M):
        assert np.array_equal(C32[r], bv[:, r])
        assert s[r, 0] == np.float32(max(np.abs(bv[:, r]).max(), np.float32(orc.EPS))) / np.float32(448.0)
    assert np.all(q[0] == 0)  # B[:, 0] is zero: row 0 of C is zero, code 0x00
