"""Python binding of libfp8q.so: amax-scaled FP8 quantization and the
block-scaled FP8 GEMM for AMD Instinct MI355X (gfx950).

Argument marshalling only.  Each function has the name and the argument
order of its C entry point in include/fp8q.h; pointer arguments take torch
tensors (their data_ptr() is passed) or raw integer addresses, the element
dtype argument of the C call is read from the input tensor, and ``stream``
defaults to torch's current stream on the tensor's device.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.
A non-OK status raises Fp8qError with the library's message.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8q.so")

OK, EINVAL, ESHAPE, EALIGN, EHIP, ENOTIMPL = range(6)
F32, BF16 = 0, 1
E4M3FN, E5M2 = 0, 1
GRAN_TENSOR, GRAN_1x128, GRAN_128x128 = 0, 1, 2
MAX_FINITE = {E4M3FN: 448.0, E5M2: 57344.0}

# every exported symbol declared in include/fp8q.h
SYMBOLS = (
    "fp8q_version",
    "fp8q_status_string",
    "fp8q_last_error",
    "fp8q_amax",
    "fp8q_quantize_tensor",
    "fp8q_quantize_1x128",
    "fp8q_quantize_1x128_t",
    "fp8q_quantize_128x128",
    "fp8q_quantize_mx",
    "fp8q_dequantize_mx",
    "fp8q_delayed_scaler_init",
    "fp8q_delayed_scaler_init_stat",
    "fp8q_delayed_scaler_update",
    "fp8q_dequantize",
    "fp8q_gemm_blockscaled",
    "fp8q_gemm_blockscaled_fast",
    "fp8q_gemm_mx",
    "fp8q_gemm_blockscaled_q",
    "fp8q_quantize_tensor_dq",
    "fp8q_quantize_tensor_delayed",
    "fp8q_gemm_blockscaled_qt",
)


class Fp8qError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fp8q status {status}: {msg}")
        self.status = status


class Scaler(ctypes.Structure):
    """Host image of fp8q_scaler (for checkpointing a device-resident state)."""

    _fields_ = [("ring", ctypes.c_float * 1024), ("window", ctypes.c_int32), ("count", ctypes.c_int32),
                ("pos", ctypes.c_int32), ("max_val", ctypes.c_float), ("eps", ctypes.c_float),
                ("margin", ctypes.c_float), ("scale", ctypes.c_float), ("stat", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("amax_acc", ctypes.c_float), ("ema", ctypes.c_double)]


STAT_MAX, STAT_MEAN, STAT_EMA = 0, 1, 2


SCALER_BYTES = ctypes.sizeof(Scaler)
SCALER_SCALE_OFFSET = Scaler.scale.offset

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfp8q.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_scaled_precision_amax_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        sig = {
            "fp8q_version": (i32, []),
            "fp8q_status_string": (ctypes.c_char_p, [i32]),
            "fp8q_last_error": (ctypes.c_char_p, []),
            "fp8q_amax": (i32, [vp, i32, i64, vp, vp]),
            "fp8q_quantize_tensor": (i32, [vp, i32, i64, i32, vp, vp, vp, vp]),
            "fp8q_quantize_1x128": (i32, [vp, i32, i64, i64, i64, i32, f32, vp, i64, vp, i64, vp]),
            "fp8q_quantize_1x128_t": (i32, [vp, i32, i64, i64, i64, i32, f32, vp, i64, vp, i64, vp]),
            "fp8q_quantize_128x128": (i32, [vp, i32, i64, i64, i64, i32, f32, vp, i64, vp, i64, vp]),
            "fp8q_quantize_mx": (i32, [vp, i32, i64, i64, i64, i32, vp, i64, vp, i64, vp]),
            "fp8q_dequantize_mx": (i32, [vp, i32, i64, i64, i64, vp, i64, vp, i32, i64, vp]),
            "fp8q_delayed_scaler_init": (i32, [vp, i32, f32, f32, f32, vp]),
            "fp8q_delayed_scaler_init_stat": (i32, [vp, i32, f32, f32, f32, i32, f32, vp]),
            "fp8q_delayed_scaler_update": (i32, [vp, vp, vp]),
            "fp8q_dequantize": (i32, [vp, i32, i64, i64, i64, vp, i32, i64, vp, i32, i64, vp]),
            "fp8q_gemm_blockscaled": (i32, [vp, i32, i64, vp, i64, i64, vp, i32, i64, vp, i32, i64, i64,
                                            vp, i32, i64, i64, i64, i64, vp]),
            "fp8q_gemm_blockscaled_fast": (i32, [vp, i32, i64, vp, i64, i64, vp, i32, i64, vp, i32, i64, i64,
                                                 vp, i32, i64, i64, i64, i64, vp]),
            "fp8q_gemm_mx": (i32, [vp, i32, i64, vp, i64, vp, i32, i64, vp, i64, vp, i32, i64, i64, i64, i64, vp]),
            "fp8q_quantize_tensor_dq": (i32, [vp, i32, i64, i32, vp, vp, vp, vp, i32, vp]),
            "fp8q_quantize_tensor_delayed": (i32, [vp, i32, i64, i32, vp, vp, vp, i32, vp]),
            "fp8q_gemm_blockscaled_qt": (i32, [vp, i32, i64, vp, i64, i64, vp, i32, i64, vp, i32, i64, i64, i32, f32,
                                               vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]),
            "fp8q_gemm_blockscaled_q": (i32, [vp, i32, i64, vp, i64, i64, vp, i32, i64, vp, i32, i64, i64, i32, f32,
                                              vp, i64, vp, i64, i64, i64, i64, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ---------------------------------------------------------------- marshalling helpers
def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dt(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"fp8q inputs are float32 or bfloat16, got {t.dtype}")


def _stream(stream, t=None) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    dev = t.device if (t is not None and not isinstance(t, int)) else None
    return torch.cuda.current_stream(dev).cuda_stream


def _check(rc: int) -> None:
    if rc != OK:
        raise Fp8qError(rc, lib().fp8q_last_error().decode(errors="replace"))


# ---------------------------------------------------------------- entry points
def fp8q_version() -> int:
    return lib().fp8q_version()


def fp8q_amax(x, n, amax, stream=None) -> None:
    _check(lib().fp8q_amax(_ptr(x), _dt(x), n, _ptr(amax), _stream(stream, x)))


def fp8q_quantize_tensor(x, n, f, scale, q, amax_out=None, stream=None) -> None:
    _check(lib().fp8q_quantize_tensor(_ptr(x), _dt(x), n, f, _ptr(scale), _ptr(q), _ptr(amax_out),
                                      _stream(stream, x)))


def fp8q_quantize_1x128(x, rows, cols, ldx, f, eps, q, ldq, scales, ld_s, stream=None) -> None:
    _check(lib().fp8q_quantize_1x128(_ptr(x), _dt(x), rows, cols, ldx, f, eps, _ptr(q), ldq, _ptr(scales),
                                     ld_s, _stream(stream, x)))


def fp8q_quantize_1x128_t(x, rows, cols, ldx, f, eps, q, ldq, scales, ld_s, stream=None) -> None:
    _check(lib().fp8q_quantize_1x128_t(_ptr(x), _dt(x), rows, cols, ldx, f, eps, _ptr(q), ldq, _ptr(scales),
                                       ld_s, _stream(stream, x)))


def fp8q_quantize_128x128(x, rows, cols, ldx, f, eps, q, ldq, scales, ld_s, stream=None) -> None:
    _check(lib().fp8q_quantize_128x128(_ptr(x), _dt(x), rows, cols, ldx, f, eps, _ptr(q), ldq,
                                       _ptr(scales), ld_s, _stream(stream, x)))


def fp8q_quantize_mx(x, rows, cols, ldx, f, q, ldq, scales, ld_s, stream=None) -> None:
    _check(lib().fp8q_quantize_mx(_ptr(x), _dt(x), rows, cols, ldx, f, _ptr(q), ldq, _ptr(scales), ld_s,
                                  _stream(stream, x)))


def fp8q_dequantize_mx(q, f, rows, cols, ldq, scales, ld_s, y, ldy, stream=None) -> None:
    _check(lib().fp8q_dequantize_mx(_ptr(q), f, rows, cols, ldq, _ptr(scales), ld_s, _ptr(y), _dt(y), ldy,
                                    _stream(stream, q)))


def fp8q_delayed_scaler_init(state, window, max_val, eps, margin, stream=None) -> None:
    _check(lib().fp8q_delayed_scaler_init(_ptr(state), window, max_val, eps, margin, _stream(stream, state)))


def fp8q_delayed_scaler_init_stat(state, window, max_val, eps, margin, stat, alpha=0.0, stream=None) -> None:
    _check(lib().fp8q_delayed_scaler_init_stat(_ptr(state), window, max_val, eps, margin, stat, alpha,
                                               _stream(stream, state)))


def fp8q_delayed_scaler_update(state, amax=None, stream=None) -> None:
    _check(lib().fp8q_delayed_scaler_update(_ptr(state), _ptr(amax), _stream(stream, state)))


def fp8q_dequantize(q, f, rows, cols, ldq, scales, g, ld_s, y, ldy, stream=None) -> None:
    _check(lib().fp8q_dequantize(_ptr(q), f, rows, cols, ldq, _ptr(scales), g, ld_s, _ptr(y), _dt(y), ldy,
                                 _stream(stream, q)))


def fp8q_gemm_blockscaled(A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn, sB_skb, C, ldc, M, N,
                          K, stream=None) -> None:
    _check(lib().fp8q_gemm_blockscaled(_ptr(A), fa, lda, _ptr(sA), sA_sm, sA_skb, _ptr(B), fb, ldb, _ptr(sB),
                                       gb, sB_sn, sB_skb, _ptr(C), _dt(C), ldc, M, N, K, _stream(stream, A)))


def fp8q_gemm_blockscaled_fast(A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn, sB_skb, C, ldc, M, N,
                               K, stream=None) -> None:
    _check(lib().fp8q_gemm_blockscaled_fast(_ptr(A), fa, lda, _ptr(sA), sA_sm, sA_skb, _ptr(B), fb, ldb,
                                            _ptr(sB), gb, sB_sn, sB_skb, _ptr(C), _dt(C), ldc, M, N, K,
                                            _stream(stream, A)))


def fp8q_gemm_mx(A, fa, lda, sA, ld_sa, B, fb, ldb, sB, ld_sb, C, ldc, M, N, K, stream=None) -> None:
    _check(lib().fp8q_gemm_mx(_ptr(A), fa, lda, _ptr(sA), ld_sa, _ptr(B), fb, ldb, _ptr(sB), ld_sb, _ptr(C), _dt(C),
                              ldc, M, N, K, _stream(stream, A)))


def fp8q_gemm_blockscaled_q(A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn, sB_skb, fc, eps, Cq, ldcq, Cs,
                            ld_cs, M, N, K, stream=None) -> None:
    _check(lib().fp8q_gemm_blockscaled_q(_ptr(A), fa, lda, _ptr(sA), sA_sm, sA_skb, _ptr(B), fb, ldb, _ptr(sB), gb,
                                         sB_sn, sB_skb, fc, eps, _ptr(Cq), ldcq, _ptr(Cs), ld_cs, M, N, K,
                                         _stream(stream, A)))


def fp8q_quantize_tensor_dq(x, n, f, scale, q, y, amax_out=None, stream=None) -> None:
    _check(lib().fp8q_quantize_tensor_dq(_ptr(x), _dt(x), n, f, _ptr(scale), _ptr(q), _ptr(amax_out), _ptr(y),
                                         _dt(y), _stream(stream, x)))


def fp8q_quantize_tensor_delayed(x, n, f, state, q, y=None, stream=None) -> None:
    _check(lib().fp8q_quantize_tensor_delayed(_ptr(x), _dt(x), n, f, _ptr(state), _ptr(q), _ptr(y),
                                              _dt(y) if y is not None else F32, _stream(stream, x)))


def fp8q_gemm_blockscaled_qt(A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn, sB_skb, fc, eps, Cqt, ldcqt,
                             Cst, ld_cst, Cq, ldcq, Cs, ld_cs, M, N, K, stream=None) -> None:
    _check(lib().fp8q_gemm_blockscaled_qt(_ptr(A), fa, lda, _ptr(sA), sA_sm, sA_skb, _ptr(B), fb, ldb, _ptr(sB), gb,
                                          sB_sn, sB_skb, fc, eps, _ptr(Cqt), ldcqt, _ptr(Cst), ld_cst, _ptr(Cq), ldcq,
                                          _ptr(Cs), ld_cs, M, N, K, _stream(stream, A)))
