"""CPU oracle for FP8 amax-scaled quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg use it to check and time the GPU library.  The
product path never imports it.  The arithmetic lives in ``fp8q_oracle.c``
(plain C, fp64 / exact integers, built with gcc); this module only builds
that file and marshals numpy arrays.  ``rel_err`` is the one function
written here, in numpy fp64.

Sources: the PyTorch-native FP8 article (m.nxbn.cn/news/137885), sections
1.2, 1.3, 2.2 and 4.1-4.3, and the handbook chapter "混合精度与 FP8 训练",
section "FP8 训练" and its exercises.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp8q_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

E4M3FN, E5M2 = 0, 1
F32, BF16 = 0, 1
GRAN_TENSOR, GRAN_1x128, GRAN_128x128 = 0, 1, 2
MAX_FINITE = {E4M3FN: 448.0, E5M2: 57344.0}
EPS = np.float32(1e-12)


def build(force: bool = True) -> str:
    """Compile fp8q_oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(LIB)
        vp, i64, i32, f32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_uint32
        sig = {
            "orc_max_finite": (ctypes.c_double, [i32]),
            "orc_set_threads": (None, [i32]),
            "orc_max_threads": (i32, []),
            "orc_decode": (ctypes.c_double, [u32, i32]),
            "orc_encode": (u32, [f32, i32]),
            "orc_encode_array": (None, [vp, i64, i32, vp]),
            "orc_encode_bits_range": (None, [u32, i64, i32, vp]),
            "orc_amax": (f32, [vp, i32, i64]),
            "orc_quantize_mx": (None, [vp, i32, i64, i64, i64, i32, vp, i64, vp, i64]),
            "orc_dequantize_mx": (None, [vp, i32, i64, i64, i64, vp, i64, vp, i64]),
            "orc_gemm_mx": (None, [vp, i32, i64, vp, i64, vp, i32, i64, vp, i64, i64, i64, i64, vp, i64, vp,
                                   vp]),
            "orc_scale": (f32, [f32, f32, f32, f32]),
            "orc_quantize_value": (u32, [f32, f32, i32]),
            "orc_quantize_tensor": (None, [vp, i32, i64, i32, f32, vp]),
            "orc_quantize_blocks": (None, [vp, i32, i64, i64, i64, i64, i64, i32, f32, vp, i64, vp, i64]),
            "orc_dequantize": (None, [vp, i32, i64, i64, i64, vp, i32, i64, vp, i32, i64]),
            "orc_scaler_init": (i32, [vp, i32, f32, f32, f32]),
            "orc_scaler_init_stat": (i32, [vp, i32, f32, f32, f32, i32, f32]),
            "orc_scaler_update": (None, [vp, f32]),
            "orc_scaler_size": (i64, []),
            "orc_gemm_blockscaled": (None, [vp, i32, i64, vp, i64, i64, vp, i32, i64, vp, i32, i64, i64,
                                            i64, i64, i64, vp, i64, vp, vp]),
            "orc_version": (i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"] or a.flags["F_CONTIGUOUS"] or a.ndim <= 1
    return a.ctypes.data


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:  # raw bf16 bits
        return BF16
    raise TypeError(f"oracle inputs are float32 or raw bf16 (uint16), got {x.dtype}")


# ---------------------------------------------------------------- codec
def set_threads(n: int) -> None:
    """OpenMP threads the oracle's loops use (timing only; results do not depend on it)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def decode(code: int, fmt: int) -> float:
    return lib().orc_decode(int(code) & 0xFF, fmt)


def decode_table(fmt: int) -> np.ndarray:
    return np.array([decode(c, fmt) for c in range(256)], dtype=np.float64)


def encode(v: float, fmt: int) -> int:
    return int(lib().orc_encode(float(np.float32(v)), fmt))


def encode_array(v: np.ndarray, fmt: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_encode_array(_ptr(v), v.size, fmt, _ptr(out))
    return out


def encode_bits_range(lo: int, n: int, fmt: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    lib().orc_encode_bits_range(lo, n, fmt, _ptr(out))
    return out


# ---------------------------------------------------------------- scaling
def amax(x: np.ndarray) -> np.float32:
    x = np.ascontiguousarray(x)
    return np.float32(lib().orc_amax(_ptr(x), _dtype_code(x), x.size))


def scale(amax_v: float, fmt: int, eps: float = EPS, margin: float = 1.0) -> np.float32:
    return np.float32(lib().orc_scale(float(np.float32(amax_v)), MAX_FINITE[fmt], float(np.float32(eps)),
                                      float(np.float32(margin))))


def quantize_value(x: float, s: float, fmt: int) -> int:
    return int(lib().orc_quantize_value(float(np.float32(x)), float(np.float32(s)), fmt))


def quantize_tensor(x: np.ndarray, fmt: int, s: float) -> np.ndarray:
    x = np.ascontiguousarray(x)
    q = np.empty(x.shape, dtype=np.uint8)
    lib().orc_quantize_tensor(_ptr(x), _dtype_code(x), x.size, fmt, float(np.float32(s)), _ptr(q))
    return q


def quantize_blocks(x: np.ndarray, br: int, bc: int, fmt: int, eps: float = EPS):
    """Block quantize a 2-D array with br x bc blocks; returns (codes, scales)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    assert rows % br == 0 and cols % bc == 0
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows // br, cols // bc), dtype=np.float32)
    lib().orc_quantize_blocks(_ptr(x), _dtype_code(x), rows, cols, cols, br, bc, fmt,
                              float(np.float32(eps)), _ptr(q), cols, _ptr(s), cols // bc)
    return q, s


def quantize_1x128(x: np.ndarray, fmt: int, eps: float = EPS):
    return quantize_blocks(x, 1, 128, fmt, eps)


def quantize_128x128(x: np.ndarray, fmt: int, eps: float = EPS):
    return quantize_blocks(x, 128, 128, fmt, eps)


def dequantize(q: np.ndarray, fmt: int, scales: np.ndarray, gran: int, out_bf16: bool = False) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    if q.ndim == 1:
        q = q.reshape(1, -1)
    rows, cols = q.shape
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    ld_s = 1 if scales.ndim < 2 else scales.shape[1]
    y = np.empty((rows, cols), dtype=np.uint16 if out_bf16 else np.float32)
    lib().orc_dequantize(_ptr(q), fmt, rows, cols, cols, _ptr(scales), gran, ld_s, _ptr(y),
                         BF16 if out_bf16 else F32, cols)
    return y


def rel_err(qhat: np.ndarray, x: np.ndarray) -> float:
    """||qhat - x||_2 / ||x||_2 in fp64 (the handbook's rel_err)."""
    d = qhat.astype(np.float64) - x.astype(np.float64)
    return float(np.sqrt(np.sum(d * d)) / np.sqrt(np.sum(x.astype(np.float64) ** 2)))


# ---------------------------------------------------------------- delayed scaler
class Scaler(ctypes.Structure):
    _fields_ = [("ring", ctypes.c_float * 1024), ("window", ctypes.c_int32), ("count", ctypes.c_int32),
                ("pos", ctypes.c_int32), ("max_val", ctypes.c_float), ("eps", ctypes.c_float),
                ("margin", ctypes.c_float), ("scale", ctypes.c_float), ("stat", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("pad_", ctypes.c_int32), ("ema", ctypes.c_double)]


STAT_MAX, STAT_MEAN, STAT_EMA = 0, 1, 2


def scaler_new(window: int, fmt: int, eps: float = EPS, margin: float = 1.0, stat: int = STAT_MAX,
               alpha: float = 0.0) -> Scaler:
    """A delayed scaler ([A] 4.2): window statistic max (default), mean, or EMA with coefficient alpha."""
    st = Scaler()
    assert ctypes.sizeof(st) == lib().orc_scaler_size()
    rc = lib().orc_scaler_init_stat(ctypes.addressof(st), window, MAX_FINITE[fmt], float(np.float32(eps)),
                                    float(np.float32(margin)), stat, float(np.float32(alpha)))
    if rc:
        raise ValueError("window must be in [1, 1024], stat in {0, 1, 2}, alpha in (0, 1] for the EMA")
    return st


def scaler_update(st: Scaler, amax_v: float) -> None:
    lib().orc_scaler_update(ctypes.addressof(st), float(np.float32(amax_v)))


# ---------------------------------------------------------------- GEMM
def gemm_blockscaled(A: np.ndarray, fa: int, sA: np.ndarray, B: np.ndarray, fb: int, sB: np.ndarray,
                     gb: int, rows: np.ndarray | None = None):
    """C, D for A [M,K] (codes, 1x128 scales sA [M,K/128]) and B [N,K] (codes; scales sB
    [N/128,K/128] for 128x128 or [N,K/128] for 1x128).  With ``rows`` only those rows of C."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sA = np.ascontiguousarray(sA, dtype=np.float32)
    sB = np.ascontiguousarray(sB, dtype=np.float32)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2 and K % 128 == 0
    if rows is None:
        nr, rp = M, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nr, rp = rows.size, rows
    C = np.empty((nr, N), dtype=np.float64)
    D = np.empty((nr, N), dtype=np.float64)
    lib().orc_gemm_blockscaled(_ptr(A), fa, K, _ptr(sA), sA.shape[1], 1, _ptr(B), fb, K, _ptr(sB), gb,
                               sB.shape[1], 1, M, N, K, None if rp is None else _ptr(rp),
                               0 if rp is None else nr, _ptr(C), _ptr(D))
    return C, D


# ---------------------------------------------------------------- MX (microscaling) FP8
def gemm_blockscaled_q(A: np.ndarray, fa: int, sA: np.ndarray, B: np.ndarray, fb: int, sB: np.ndarray, gb: int,
                       fc: int, eps: float = EPS, rows: np.ndarray | None = None):
    """The GEMM's output quantized 1x128 for the next layer: C = fl32 of the
    exact block-scaled product (gemm_blockscaled), then quantize_blocks(C, 1,
    128, fc, eps).  Returns (codes [rows, N], scales [rows, N/128], C fp32)."""
    C, _ = gemm_blockscaled(A, fa, sA, B, fb, sB, gb, rows=rows)
    C32 = C.astype(np.float32)  # round to nearest even
    q, s = quantize_blocks(C32, 1, 128, fc, eps)
    return q, s, C32


def gemm_blockscaled_qt(A: np.ndarray, fa: int, sA: np.ndarray, B: np.ndarray, fb: int, sB: np.ndarray, gb: int,
                        fc: int, eps: float = EPS):
    """The GEMM's output quantized along M for the weight gradient: C = fl32 of
    the exact block-scaled product (gemm_blockscaled), then quantize_blocks(C,
    128, 1, fc, eps) -- one scale per 128 rows of a column -- returned as the
    codes of C^T [N, M] and their scales [N, M/128], with C fp32."""
    C, _ = gemm_blockscaled(A, fa, sA, B, fb, sB, gb)
    C32 = C.astype(np.float32)  # round to nearest even
    q, s = quantize_blocks(C32, 128, 1, fc, eps)
    return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T), C32


def quantize_mx(x: np.ndarray, fmt: int):
    """32-element blocks along rows with power-of-two E8M0 scales (OCP MX v1.0, 6.3).
    Returns (codes [rows, cols], scale bytes [rows, cols/32])."""
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    rows, cols = x.shape
    assert cols % 32 == 0
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows, cols // 32), dtype=np.uint8)
    lib().orc_quantize_mx(_ptr(x), _dtype_code(x), rows, cols, cols, fmt, _ptr(q), cols, _ptr(s), cols // 32)
    return q, s


def dequantize_mx(q: np.ndarray, fmt: int, scales: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = q.shape
    y = np.empty((rows, cols), dtype=np.float32)
    lib().orc_dequantize_mx(_ptr(q), fmt, rows, cols, cols, _ptr(scales), scales.shape[1], _ptr(y), cols)
    return y


def gemm_mx(A: np.ndarray, fa: int, sA: np.ndarray, B: np.ndarray, fb: int, sB: np.ndarray,
            rows: np.ndarray | None = None):
    """C, D of the MX GEMM: A [M,K], B [N,K] codes, E8M0 scales sA [M,K/32], sB [N,K/32]."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    sA = np.ascontiguousarray(sA, dtype=np.uint8)
    sB = np.ascontiguousarray(sB, dtype=np.uint8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2 and K % 32 == 0
    if rows is None:
        nr, rp = M, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nr, rp = rows.size, rows
    C = np.empty((nr, N), dtype=np.float64)
    D = np.empty((nr, N), dtype=np.float64)
    lib().orc_gemm_mx(_ptr(A), fa, K, _ptr(sA), sA.shape[1], _ptr(B), fb, K, _ptr(sB), sB.shape[1], M, N, K,
                      None if rp is None else _ptr(rp), 0 if rp is None else nr, _ptr(C), _ptr(D))
    return C, D
