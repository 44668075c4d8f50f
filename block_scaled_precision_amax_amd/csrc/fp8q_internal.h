// Internal declarations shared by the HIP translation units of libfp8q.so.
// Device helpers for the FP8 encode used by every quantizer, the launch
// functions the C ABI calls after validation, and the error plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8q.h"

namespace fp8q {

// ---------------------------------------------------------------- errors
// Records `msg` as this thread's last error text and returns `code`.
int fail(int code, const char* fmt, ...);
// Converts a HIP error from the launch just made into FP8Q_EHIP (or OK).
int check_launch(const char* what);

// ---------------------------------------------------------------- formats
// OCP E4M3FN: max finite 448; OCP E5M2: max finite 57344 (PyTorch-native
// FP8 article, section 1.2 table).
__host__ __device__ constexpr float max_finite(int fmt) { return fmt == FP8Q_E4M3FN ? 448.0f : 57344.0f; }

#ifdef __HIP_DEVICE_COMPILE__
#define FP8Q_DEV __device__ __forceinline__
#else
#define FP8Q_DEV __device__ inline
#endif

// Two fp32 values -> two codes in the low (HI=false) or high (HI=true)
// 16 bits of `old`.  The gfx950 conversion rounds to nearest even; the
// caller has already clamped to +-MAX and removed NaN.
template <int FMT, bool HI>
FP8Q_DEV uint32_t cvt2(float a, float b, uint32_t old) {
  if constexpr (FMT == FP8Q_E4M3FN)
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

// Clamp to the finite range.  Clamping before the cast is what makes the
// cast saturating (the handbook's quant clamps to +-MAX before .to(FP8)).
template <int FMT>
FP8Q_DEV float sat(float y) {
  return __builtin_amdgcn_fmed3f(y, -max_finite(FMT), max_finite(FMT));
}

// Four quotients (already clamped) -> one dword of four codes, byte i = y_i.
template <int FMT>
FP8Q_DEV uint32_t pack4(float y0, float y1, float y2, float y3) {
  uint32_t w = cvt2<FMT, false>(y0, y1, 0u);
  return cvt2<FMT, true>(y2, y3, w);
}

// One value -> one code by the reference definition: NaN -> 0x7F,
// otherwise clamp and round to nearest even.  Used off the fast path.
template <int FMT>
FP8Q_DEV uint32_t enc1(float y) {
  if (y != y) return 0x7Fu;
  return cvt2<FMT, false>(sat<FMT>(y), 0.0f, 0u) & 0xFFu;
}

// Correctly rounded fp32 quotient x / s from r = RN(1/s) with one
// residual correction (Markstein, "Computation of elementary functions on
// the IBM RISC System/6000 processor", IBM J. R&D 34(1), 1990): q0 =
// RN(x*r) is within one ulp, e = q0*s - x is exact in one FMA, and
// RN(q0 - e*r) is the IEEE quotient.  Valid while nothing over- or
// underflows, which the callers guarantee by keeping s in [2^-80, 2^80]
// and |x/s| bounded; the -x / -e form keeps the sign of a zero quotient.
FP8Q_DEV float div_rn(float x, float s, float r) {
  float q0 = x * r;
  float e = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-e, r, q0);
}

// As div_rn for an x that may be arbitrarily large against s (per-tensor
// scales come from earlier steps): q0 is first clamped to +-2^20, far
// above any finite FP8 value, so the residual cannot overflow; when the
// clamp acts, the true quotient exceeds the clamp and the result
// saturates either way.
FP8Q_DEV float div_rn_wide(float x, float s, float r) {
  float q0 = __builtin_amdgcn_fmed3f(x * r, -1048576.0f, 1048576.0f);
  float e = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-e, r, q0);
}

// A scale the fast division handles: finite, positive, in [2^-80, 2^80].
FP8Q_DEV bool scale_ok(float s) { return s >= 0x1p-80f && s <= 0x1p80f; }

// bf16 pair in a dword -> two fp32 (exact widening).
FP8Q_DEV float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
FP8Q_DEV float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Scale from a block amax: s = fl32(max(amax, eps) / MAX).  A NaN amax
// gives a NaN scale (the comparison is false), as torch's clamp does.
template <int FMT>
FP8Q_DEV float block_scale(float amax, float eps) {
  float m = (amax < eps) ? eps : amax;
  return m / max_finite(FMT);
}

// Largest |x| bit pattern -> float, with every NaN made the quiet NaN
// 0x7FC00000 (abs bit patterns of non-negative floats order like the
// floats; NaN patterns sort above +Inf).
FP8Q_DEV uint32_t canon_abs_bits(uint32_t m) { return m > 0x7F800000u ? 0x7FC00000u : m; }

// ---------------------------------------------------------------- DPP max
// Maximum over the 16 lanes of a DPP row; every lane of the row gets it.
FP8Q_DEV uint32_t row16_max(uint32_t v) {
  // xor 1 and xor 2 inside each quad, then half-row and row mirrors.
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
  return v;
}

// Maximum over all 64 lanes of the wavefront, returned to every lane.
FP8Q_DEV uint32_t wave_max(uint32_t v) {
  v = row16_max(v);
  // rows 0..3 -> combine with the row 16 and 32 lanes away
  v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));  // xor 16 within 32
  v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// ---------------------------------------------------------------- launches
int launch_amax(const void* x, int dt, int64_t n, float* amax, hipStream_t st);
// amax (nullable) gets max|x|: overwritten when reset_amax (a one-thread
// reset launch precedes the pass), folded in as a running maximum otherwise.
int launch_quantize_tensor(const void* x, int dt, int64_t n, int fmt, const float* scale, uint8_t* q,
                           float* amax, bool reset_amax, hipStream_t st, void* y = nullptr, int out_dt = -1);
int launch_quantize_1x128(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                          float eps, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                          hipStream_t st);
int launch_quantize_1x128_t(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                            float eps, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                            hipStream_t st);
int launch_quantize_mx(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                       int64_t ldq, uint8_t* scales, int64_t ld_s, hipStream_t st);
int launch_dequantize_mx(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq, const uint8_t* scales,
                         int64_t ld_s, void* y, int out_dt, int64_t ldy, hipStream_t st);
int launch_quantize_128x128(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                            float eps, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                            hipStream_t st);
int launch_scaler_init(fp8q_scaler* st_dev, int32_t window, float max_val, float eps, float margin, int32_t stat,
                       float alpha, hipStream_t st);
int launch_scaler_update(fp8q_scaler* st_dev, float* amax, hipStream_t st);
int launch_dequantize(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                      const float* scales, int gran, int64_t ld_s, void* y, int out_dt, int64_t ldy,
                      hipStream_t st);
int launch_gemm(const uint8_t* A, int fa, int64_t lda, const float* sA, int64_t sA_sm,
                int64_t sA_skb, const uint8_t* B, int fb, int64_t ldb, const float* sB, int gb,
                int64_t sB_sn, int64_t sB_skb, void* C, int out_dt, int64_t ldc, int64_t M,
                int64_t N, int64_t K, bool fast, hipStream_t st);

int launch_gemm_q(const uint8_t* A, int fa, int64_t lda, const float* sA, int64_t sA_sm, int64_t sA_skb,
                  const uint8_t* B, int fb, int64_t ldb, const float* sB, int gb, int64_t sB_sn, int64_t sB_skb,
                  int fc, float eps, uint8_t* Cq, int64_t ldc, float* Cs, int64_t ld_cs, int64_t M, int64_t N,
                  int64_t K, hipStream_t st);
int launch_gemm_qt(const uint8_t* A, int fa, int64_t lda, const float* sA, int64_t sA_sm, int64_t sA_skb,
                   const uint8_t* B, int fb, int64_t ldb, const float* sB, int gb, int64_t sB_sn, int64_t sB_skb,
                   int fc, float eps, uint8_t* Ct, int64_t ldt, float* Cst, int64_t ld_st, uint8_t* Cq, int64_t ldcq,
                   float* Cs, int64_t ld_cs, int64_t M, int64_t N, int64_t K, hipStream_t st);
int launch_gemm_mx(const uint8_t* A, int fa, int64_t lda, const uint8_t* sA, int64_t ld_sa, const uint8_t* B,
                   int fb, int64_t ldb, const uint8_t* sB, int64_t ld_sb, void* C, int out_dt, int64_t ldc,
                   int64_t M, int64_t N, int64_t K, hipStream_t st);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace fp8q
