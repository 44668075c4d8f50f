// C ABI of libfp8q.so: argument validation, then the launches.  Nothing is
// enqueued unless every check passes; no call allocates, frees or
// synchronizes.  The operations themselves are defined in include/fp8q.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>

#include "fp8q_internal.h"

namespace fp8q {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FP8Q_EHIP, "%s: %s", what, hipGetErrorString(e));
  return FP8Q_OK;
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace fp8q

using namespace fp8q;

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool valid_dt(int dt) { return dt == FP8Q_F32 || dt == FP8Q_BF16; }
bool valid_fmt(int f) { return f == FP8Q_E4M3FN || f == FP8Q_E5M2; }
int64_t esize(int dt) { return dt == FP8Q_F32 ? 4 : 2; }
hipStream_t S(void* s) { return (hipStream_t)s; }

// Shared checks of the two block quantizers.
int check_block_quant(const char* fn, const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx,
                      int fmt, float eps, const uint8_t* q, int64_t ldq, const float* scales,
                      int64_t ld_s, int64_t br) {
  if (!x || !q || !scales) return fail(FP8Q_EINVAL, "%s: null pointer", fn);
  if (!valid_dt(dt) || !valid_fmt(fmt)) return fail(FP8Q_EINVAL, "%s: bad dtype or format", fn);
  if (rows <= 0 || cols <= 0) return fail(FP8Q_EINVAL, "%s: rows and cols must be positive", fn);
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(FP8Q_EINVAL, "%s: eps must be finite and > 0", fn);
  if (cols % 128 != 0) return fail(FP8Q_ESHAPE, "%s: cols (%lld) must be a multiple of 128", fn, (long long)cols);
  if (rows % br != 0) return fail(FP8Q_ESHAPE, "%s: rows (%lld) must be a multiple of %lld", fn, (long long)rows, (long long)br);
  if (ldx < cols || ldq < cols || ld_s < cols / 128)
    return fail(FP8Q_EINVAL, "%s: leading dimension smaller than the row", fn);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4))
    return fail(FP8Q_EALIGN, "%s: x and q must be 16-byte aligned, scales 4-byte", fn);
  if ((ldx * esize(dt)) % 16 != 0 || ldq % 16 != 0)
    return fail(FP8Q_EALIGN, "%s: ldx and ldq must keep rows 16-byte aligned", fn);
  return FP8Q_OK;
}

}  // namespace

extern "C" {

int fp8q_version(void) { return 100; }

const char* fp8q_status_string(int status) {
  switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_EINVAL: return "invalid argument";
    case FP8Q_ESHAPE: return "unsupported shape";
    case FP8Q_EALIGN: return "misaligned pointer or leading dimension";
    case FP8Q_EHIP: return "HIP launch failure";
    case FP8Q_ENOTIMPL: return "not implemented";
    default: return "unknown status";
  }
}

const char* fp8q_last_error(void) { return g_err; }

int fp8q_amax(const void* x, fp8q_dtype dt, int64_t n, float* amax, void* stream) {
  if (!x || !amax) return fail(FP8Q_EINVAL, "amax: null pointer");
  if (!valid_dt(dt)) return fail(FP8Q_EINVAL, "amax: bad dtype");
  if (n <= 0) return fail(FP8Q_EINVAL, "amax: n must be positive");
  if (!aligned(x, 16) || !aligned(amax, 4)) return fail(FP8Q_EALIGN, "amax: x must be 16-byte aligned");
  return launch_amax(x, dt, n, amax, S(stream));
}

int fp8q_quantize_tensor(const void* x, fp8q_dtype dt, int64_t n, fp8q_format f, const float* scale,
                         uint8_t* q, float* amax_out, void* stream) {
  if (!x || !scale || !q) return fail(FP8Q_EINVAL, "quantize_tensor: null pointer");
  if (!valid_dt(dt) || !valid_fmt(f)) return fail(FP8Q_EINVAL, "quantize_tensor: bad dtype or format");
  if (n <= 0) return fail(FP8Q_EINVAL, "quantize_tensor: n must be positive");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4) || (amax_out && !aligned(amax_out, 4)))
    return fail(FP8Q_EALIGN, "quantize_tensor: x and q must be 16-byte aligned");
  return launch_quantize_tensor(x, dt, n, f, scale, q, amax_out, true, S(stream));
}

int fp8q_quantize_tensor_dq(const void* x, fp8q_dtype dt, int64_t n, fp8q_format f, const float* scale,
                            uint8_t* q, float* amax_out, void* y, fp8q_dtype out_dt, void* stream) {
  if (!x || !scale || !q || !y) return fail(FP8Q_EINVAL, "quantize_tensor_dq: null pointer");
  if (!valid_dt(dt) || !valid_fmt(f) || !valid_dt(out_dt))
    return fail(FP8Q_EINVAL, "quantize_tensor_dq: bad dtype or format");
  if (n <= 0) return fail(FP8Q_EINVAL, "quantize_tensor_dq: n must be positive");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(y, 16) || !aligned(scale, 4) ||
      (amax_out && !aligned(amax_out, 4)))
    return fail(FP8Q_EALIGN, "quantize_tensor_dq: x, q and y must be 16-byte aligned");
  return launch_quantize_tensor(x, dt, n, f, scale, q, amax_out, true, S(stream), y, out_dt);
}

int fp8q_quantize_tensor_delayed(const void* x, fp8q_dtype dt, int64_t n, fp8q_format f, fp8q_scaler* state,
                                 uint8_t* q, void* y, fp8q_dtype out_dt, void* stream) {
  if (!x || !state || !q) return fail(FP8Q_EINVAL, "quantize_tensor_delayed: null pointer");
  if (!valid_dt(dt) || !valid_fmt(f) || (y && !valid_dt(out_dt)))
    return fail(FP8Q_EINVAL, "quantize_tensor_delayed: bad dtype or format");
  if (n <= 0) return fail(FP8Q_EINVAL, "quantize_tensor_delayed: n must be positive");
  if (!aligned(x, 16) || !aligned(q, 16) || (y && !aligned(y, 16)) || !aligned(state, 8))
    return fail(FP8Q_EALIGN, "quantize_tensor_delayed: x, q and y must be 16-byte aligned, state 8-byte");
  // the scale in force and the step's running amax live in the state
  return launch_quantize_tensor(x, dt, n, f, &state->scale, q, &state->amax_acc, false, S(stream), y,
                                y ? (int)out_dt : -1);
}

int fp8q_quantize_1x128(const void* x, fp8q_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                        fp8q_format f, float eps, uint8_t* q, int64_t ldq, float* scales,
                        int64_t ld_s, void* stream) {
  if (int e = check_block_quant("quantize_1x128", x, dt, rows, cols, ldx, f, eps, q, ldq, scales, ld_s, 1))
    return e;
  return launch_quantize_1x128(x, dt, rows, cols, ldx, f, eps, q, ldq, scales, ld_s, S(stream));
}

int fp8q_quantize_1x128_t(const void* x, fp8q_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                          fp8q_format f, float eps, uint8_t* q, int64_t ldq, float* scales,
                          int64_t ld_s, void* stream) {
  const char* fn = "quantize_1x128_t";
  if (!x || !q || !scales) return fail(FP8Q_EINVAL, "%s: null pointer", fn);
  if (!valid_dt(dt) || !valid_fmt(f)) return fail(FP8Q_EINVAL, "%s: bad dtype or format", fn);
  if (rows <= 0 || cols <= 0) return fail(FP8Q_EINVAL, "%s: rows and cols must be positive", fn);
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(FP8Q_EINVAL, "%s: eps must be finite and > 0", fn);
  if (rows % 128 != 0) return fail(FP8Q_ESHAPE, "%s: rows (%lld) must be a multiple of 128", fn, (long long)rows);
  if (cols % 64 != 0) return fail(FP8Q_ESHAPE, "%s: cols (%lld) must be a multiple of 64", fn, (long long)cols);
  if (ldx < cols || ldq < rows || ld_s < rows / 128)
    return fail(FP8Q_EINVAL, "%s: leading dimension smaller than the row", fn);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4))
    return fail(FP8Q_EALIGN, "%s: x and q must be 16-byte aligned, scales 4-byte", fn);
  if ((ldx * esize(dt)) % 16 != 0 || ldq % 16 != 0)
    return fail(FP8Q_EALIGN, "%s: ldx and ldq must keep rows 16-byte aligned", fn);
  return launch_quantize_1x128_t(x, dt, rows, cols, ldx, f, eps, q, ldq, scales, ld_s, S(stream));
}

int fp8q_quantize_mx(const void* x, fp8q_dtype dt, int64_t rows, int64_t cols, int64_t ldx, fp8q_format f,
                     uint8_t* q, int64_t ldq, uint8_t* scales, int64_t ld_s, void* stream) {
  const char* fn = "quantize_mx";
  if (!x || !q || !scales) return fail(FP8Q_EINVAL, "%s: null pointer", fn);
  if (!valid_dt(dt) || !valid_fmt(f)) return fail(FP8Q_EINVAL, "%s: bad dtype or format", fn);
  if (rows <= 0 || cols <= 0) return fail(FP8Q_EINVAL, "%s: rows and cols must be positive", fn);
  if (cols % 32 != 0) return fail(FP8Q_ESHAPE, "%s: cols (%lld) must be a multiple of 32", fn, (long long)cols);
  if (ldx < cols || ldq < cols || ld_s < cols / 32)
    return fail(FP8Q_EINVAL, "%s: leading dimension smaller than the row", fn);
  if (!aligned(x, 16) || !aligned(q, 16) || (ldx * esize(dt)) % 16 != 0 || ldq % 16 != 0)
    return fail(FP8Q_EALIGN, "%s: x, q and their rows must be 16-byte aligned", fn);
  return launch_quantize_mx(x, dt, rows, cols, ldx, f, q, ldq, scales, ld_s, S(stream));
}

int fp8q_dequantize_mx(const uint8_t* q, fp8q_format f, int64_t rows, int64_t cols, int64_t ldq,
                       const uint8_t* scales, int64_t ld_s, void* y, fp8q_dtype out_dt, int64_t ldy, void* stream) {
  const char* fn = "dequantize_mx";
  if (!q || !scales || !y) return fail(FP8Q_EINVAL, "%s: null pointer", fn);
  if (!valid_fmt(f) || !valid_dt(out_dt)) return fail(FP8Q_EINVAL, "%s: bad format or dtype", fn);
  if (rows <= 0 || cols <= 0) return fail(FP8Q_EINVAL, "%s: rows and cols must be positive", fn);
  if (cols % 32 != 0) return fail(FP8Q_ESHAPE, "%s: cols (%lld) must be a multiple of 32", fn, (long long)cols);
  if (ldq < cols || ldy < cols || ld_s < cols / 32)
    return fail(FP8Q_EINVAL, "%s: leading dimension smaller than the row", fn);
  if (!aligned(q, 16) || !aligned(y, 16) || ldq % 8 != 0 || (ldy * esize(out_dt)) % 16 != 0)
    return fail(FP8Q_EALIGN, "%s: q, y and their rows must be aligned (ldq % 8, y rows 16 bytes)", fn);
  return launch_dequantize_mx(q, f, rows, cols, ldq, scales, ld_s, y, out_dt, ldy, S(stream));
}

int fp8q_quantize_128x128(const void* x, fp8q_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                          fp8q_format f, float eps, uint8_t* q, int64_t ldq, float* scales,
                          int64_t ld_s, void* stream) {
  if (int e = check_block_quant("quantize_128x128", x, dt, rows, cols, ldx, f, eps, q, ldq, scales, ld_s, 128))
    return e;
  return launch_quantize_128x128(x, dt, rows, cols, ldx, f, eps, q, ldq, scales, ld_s, S(stream));
}

int fp8q_delayed_scaler_init_stat(fp8q_scaler* state, int32_t window, float max_val, float eps, float margin,
                                  fp8q_window_stat stat, float alpha, void* stream) {
  if (!state) return fail(FP8Q_EINVAL, "delayed_scaler_init: null pointer");
  if (window < 1 || window > 1024) return fail(FP8Q_EINVAL, "delayed_scaler_init: window must be in [1, 1024]");
  if (!(max_val > 0.0f) || !isfinite(max_val) || !(eps > 0.0f) || !isfinite(eps) ||
      !(margin > 0.0f) || !isfinite(margin))
    return fail(FP8Q_EINVAL, "delayed_scaler_init: max_val, eps and margin must be finite and > 0");
  if (stat != FP8Q_STAT_MAX && stat != FP8Q_STAT_MEAN && stat != FP8Q_STAT_EMA)
    return fail(FP8Q_EINVAL, "delayed_scaler_init: unknown window statistic %d", (int)stat);
  if (stat == FP8Q_STAT_EMA && !(alpha > 0.0f && alpha <= 1.0f))
    return fail(FP8Q_EINVAL, "delayed_scaler_init: the EMA coefficient must be in (0, 1]");
  if (!aligned(state, 8)) return fail(FP8Q_EALIGN, "delayed_scaler_init: state must be 8-byte aligned");
  return launch_scaler_init(state, window, max_val, eps, margin, (int32_t)stat,
                            stat == FP8Q_STAT_EMA ? alpha : 0.0f, S(stream));
}

int fp8q_delayed_scaler_init(fp8q_scaler* state, int32_t window, float max_val, float eps,
                             float margin, void* stream) {
  return fp8q_delayed_scaler_init_stat(state, window, max_val, eps, margin, FP8Q_STAT_MAX, 0.0f, stream);
}

int fp8q_delayed_scaler_update(fp8q_scaler* state, float* amax, void* stream) {
  if (!state) return fail(FP8Q_EINVAL, "delayed_scaler_update: null pointer");
  if (!amax) amax = &state->amax_acc;  // the step's amax folded in by quantize_tensor_delayed
  if (!aligned(state, 8) || !aligned(amax, 4))
    return fail(FP8Q_EALIGN, "delayed_scaler_update: state must be 8-byte and amax 4-byte aligned");
  return launch_scaler_update(state, amax, S(stream));
}

int fp8q_dequantize(const uint8_t* q, fp8q_format f, int64_t rows, int64_t cols, int64_t ldq,
                    const float* scales, fp8q_gran g, int64_t ld_s, void* y, fp8q_dtype out_dt,
                    int64_t ldy, void* stream) {
  if (!q || !scales || !y) return fail(FP8Q_EINVAL, "dequantize: null pointer");
  if (!valid_fmt(f) || !valid_dt(out_dt)) return fail(FP8Q_EINVAL, "dequantize: bad format or dtype");
  if (g != FP8Q_GRAN_TENSOR && g != FP8Q_GRAN_1x128 && g != FP8Q_GRAN_128x128)
    return fail(FP8Q_EINVAL, "dequantize: bad granularity");
  if (rows <= 0 || cols <= 0) return fail(FP8Q_EINVAL, "dequantize: rows and cols must be positive");
  if (g != FP8Q_GRAN_TENSOR && cols % 128 != 0)
    return fail(FP8Q_ESHAPE, "dequantize: cols must be a multiple of 128 for block scales");
  if (rows > 1 && (ldq < cols || ldy < cols)) return fail(FP8Q_EINVAL, "dequantize: leading dimension smaller than the row");
  if (g != FP8Q_GRAN_TENSOR && ld_s < cols / 128) return fail(FP8Q_EINVAL, "dequantize: ld_s too small");
  if (!aligned(q, 16) || !aligned(y, 16) || !aligned(scales, 4))
    return fail(FP8Q_EALIGN, "dequantize: q and y must be 16-byte aligned");
  if (rows > 1 && (ldq % 4 != 0 || ldy % 4 != 0))
    return fail(FP8Q_EALIGN, "dequantize: ldq and ldy must be multiples of 4");
  if (rows == 1) { ldq = cols; ldy = cols; }
  return launch_dequantize(q, f, rows, cols, ldq, scales, g, ld_s, y, out_dt, ldy, S(stream));
}

static int gemm_entry(const char* fn, const uint8_t* A, int fa, int64_t lda, const float* sA,
                      int64_t sA_sm, int64_t sA_skb, const uint8_t* B, int fb, int64_t ldb,
                      const float* sB, int gb, int64_t sB_sn, int64_t sB_skb, void* C, int out_dt,
                      int64_t ldc, int64_t M, int64_t N, int64_t K, bool fast, void* stream) {
  if (!A || !sA || !B || !sB || !C) return fail(FP8Q_EINVAL, "%s: null pointer", fn);
  if (!valid_fmt(fa) || !valid_fmt(fb) || !valid_dt(out_dt))
    return fail(FP8Q_EINVAL, "%s: bad format or dtype", fn);
  if (gb != FP8Q_GRAN_128x128 && gb != FP8Q_GRAN_1x128)
    return fail(FP8Q_EINVAL, "%s: B scales must be 128x128 or 1x128", fn);
  if (M <= 0 || N <= 0 || K <= 0) return fail(FP8Q_EINVAL, "%s: M, N, K must be positive", fn);
  if (K % 128 != 0) return fail(FP8Q_ESHAPE, "%s: K (%lld) must be a multiple of 128", fn, (long long)K);
  if (lda < K || ldb < K || ldc < N) return fail(FP8Q_EINVAL, "%s: leading dimension too small", fn);
  if (sA_sm < 0 || sA_skb < 0 || sB_sn < 0 || sB_skb < 0)
    return fail(FP8Q_EINVAL, "%s: negative scale stride", fn);
  if (!aligned(A, 16) || !aligned(B, 16) || lda % 16 != 0 || ldb % 16 != 0)
    return fail(FP8Q_EALIGN, "%s: A, B and their leading dimensions must be 16-byte aligned", fn);
  if (!aligned(sA, 4) || !aligned(sB, 4) || !aligned(C, out_dt == FP8Q_F32 ? 4 : 2))
    return fail(FP8Q_EALIGN, "%s: misaligned scales or C", fn);
  return launch_gemm(A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn, sB_skb, C, out_dt, ldc, M,
                     N, K, fast, S(stream));
}

int fp8q_gemm_blockscaled(const uint8_t* A, fp8q_format fa, int64_t lda, const float* sA,
                          int64_t sA_sm, int64_t sA_skb, const uint8_t* B, fp8q_format fb,
                          int64_t ldb, const float* sB, fp8q_gran gb, int64_t sB_sn,
                          int64_t sB_skb, void* C, fp8q_dtype out_dt, int64_t ldc, int64_t M,
                          int64_t N, int64_t K, void* stream) {
  return gemm_entry("gemm_blockscaled", A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn, sB_skb,
                    C, out_dt, ldc, M, N, K, false, stream);
}

int fp8q_gemm_blockscaled_q(const uint8_t* A, fp8q_format fa, int64_t lda, const float* sA, int64_t sA_sm,
                            int64_t sA_skb, const uint8_t* B, fp8q_format fb, int64_t ldb, const float* sB,
                            fp8q_gran gb, int64_t sB_sn, int64_t sB_skb, fp8q_format fc, float eps, uint8_t* Cq,
                            int64_t ldcq, float* Cs, int64_t ld_cs, int64_t M, int64_t N, int64_t K,
                            void* stream) {
  const char* fn = "gemm_blockscaled_q";
  if (!A || !sA || !B || !sB || !Cq || !Cs) return fail(FP8Q_EINVAL, "%s: null pointer", fn);
  if (!valid_fmt(fa) || !valid_fmt(fb) || !valid_fmt(fc)) return fail(FP8Q_EINVAL, "%s: bad format", fn);
  if (gb != FP8Q_GRAN_128x128 && gb != FP8Q_GRAN_1x128)
    return fail(FP8Q_EINVAL, "%s: B scales must be 128x128 or 1x128", fn);
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(FP8Q_EINVAL, "%s: eps must be finite and > 0", fn);
  if (M <= 0 || N <= 0 || K <= 0) return fail(FP8Q_EINVAL, "%s: M, N, K must be positive", fn);
  if (K % 128 != 0 || N % 128 != 0)
    return fail(FP8Q_ESHAPE, "%s: K (%lld) and N (%lld) must be multiples of 128", fn, (long long)K, (long long)N);
  if (lda < K || ldb < K || ldcq < N || ld_cs < N / 128) return fail(FP8Q_EINVAL, "%s: leading dimension too small", fn);
  if (sA_sm < 0 || sA_skb < 0 || sB_sn < 0 || sB_skb < 0) return fail(FP8Q_EINVAL, "%s: negative scale stride", fn);
  if (!aligned(A, 16) || !aligned(B, 16) || lda % 16 != 0 || ldb % 16 != 0)
    return fail(FP8Q_EALIGN, "%s: A, B and their leading dimensions must be 16-byte aligned", fn);
  if (!aligned(sA, 4) || !aligned(sB, 4) || !aligned(Cs, 4)) return fail(FP8Q_EALIGN, "%s: misaligned scales", fn);
  return launch_gemm_q(A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn, sB_skb, fc, eps, Cq, ldcq, Cs,
                       ld_cs, M, N, K, S(stream));
}

int fp8q_gemm_blockscaled_qt(const uint8_t* A, fp8q_format fa, int64_t lda, const float* sA, int64_t sA_sm,
                             int64_t sA_skb, const uint8_t* B, fp8q_format fb, int64_t ldb, const float* sB,
                             fp8q_gran gb, int64_t sB_sn, int64_t sB_skb, fp8q_format fc, float eps, uint8_t* Cqt,
                             int64_t ldcqt, float* Cst, int64_t ld_cst, uint8_t* Cq, int64_t ldcq, float* Cs,
                             int64_t ld_cs, int64_t M, int64_t N, int64_t K, void* stream) {
  const char* fn = "gemm_blockscaled_qt";
  if (!A || !sA || !B || !sB || !Cqt || !Cst) return fail(FP8Q_EINVAL, "%s: null pointer", fn);
  if ((Cq == nullptr) != (Cs == nullptr))
    return fail(FP8Q_EINVAL, "%s: the row-wise output needs both Cq and Cs (or neither)", fn);
  if (!valid_fmt(fa) || !valid_fmt(fb) || !valid_fmt(fc)) return fail(FP8Q_EINVAL, "%s: bad format", fn);
  if (gb != FP8Q_GRAN_128x128 && gb != FP8Q_GRAN_1x128)
    return fail(FP8Q_EINVAL, "%s: B scales must be 128x128 or 1x128", fn);
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(FP8Q_EINVAL, "%s: eps must be finite and > 0", fn);
  if (M <= 0 || N <= 0 || K <= 0) return fail(FP8Q_EINVAL, "%s: M, N, K must be positive", fn);
  if (K % 128 != 0 || M % 128 != 0)
    return fail(FP8Q_ESHAPE, "%s: K (%lld) and M (%lld) must be multiples of 128", fn, (long long)K, (long long)M);
  if (Cq && N % 128 != 0)
    return fail(FP8Q_ESHAPE, "%s: N (%lld) must be a multiple of 128 for the row-wise output", fn, (long long)N);
  if (lda < K || ldb < K || ldcqt < M || ld_cst < M / 128 || (Cq && (ldcq < N || ld_cs < N / 128)))
    return fail(FP8Q_EINVAL, "%s: leading dimension too small", fn);
  if (sA_sm < 0 || sA_skb < 0 || sB_sn < 0 || sB_skb < 0) return fail(FP8Q_EINVAL, "%s: negative scale stride", fn);
  if (!aligned(A, 16) || !aligned(B, 16) || lda % 16 != 0 || ldb % 16 != 0 || !aligned(Cqt, 16) || ldcqt % 16 != 0)
    return fail(FP8Q_EALIGN, "%s: A, B, Cqt and their leading dimensions must be 16-byte aligned", fn);
  if (!aligned(sA, 4) || !aligned(sB, 4) || !aligned(Cst, 4) || (Cs && !aligned(Cs, 4)))
    return fail(FP8Q_EALIGN, "%s: misaligned scales", fn);
  return launch_gemm_qt(A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn, sB_skb, fc, eps, Cqt, ldcqt, Cst,
                        ld_cst, Cq, ldcq, Cs, ld_cs, M, N, K, S(stream));
}

int fp8q_gemm_mx(const uint8_t* A, fp8q_format fa, int64_t lda, const uint8_t* sA, int64_t ld_sa,
                 const uint8_t* B, fp8q_format fb, int64_t ldb, const uint8_t* sB, int64_t ld_sb, void* C,
                 fp8q_dtype out_dt, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
  const char* fn = "gemm_mx";
  if (!A || !sA || !B || !sB || !C) return fail(FP8Q_EINVAL, "%s: null pointer", fn);
  if (!valid_fmt(fa) || !valid_fmt(fb) || !valid_dt(out_dt)) return fail(FP8Q_EINVAL, "%s: bad format or dtype", fn);
  if (M <= 0 || N <= 0 || K <= 0) return fail(FP8Q_EINVAL, "%s: M, N, K must be positive", fn);
  if (K % 128 != 0) return fail(FP8Q_ESHAPE, "%s: K (%lld) must be a multiple of 128", fn, (long long)K);
  if (lda < K || ldb < K || ldc < N || ld_sa < K / 32 || ld_sb < K / 32)
    return fail(FP8Q_EINVAL, "%s: leading dimension too small", fn);
  if (!aligned(A, 16) || !aligned(B, 16) || lda % 16 != 0 || ldb % 16 != 0)
    return fail(FP8Q_EALIGN, "%s: A, B and their leading dimensions must be 16-byte aligned", fn);
  if (!aligned(sA, 4) || !aligned(sB, 4) || ld_sa % 4 != 0 || ld_sb % 4 != 0 ||
      !aligned(C, out_dt == FP8Q_F32 ? 4 : 2))
    return fail(FP8Q_EALIGN, "%s: scale rows must be 4-byte aligned; C aligned to its element", fn);
  return launch_gemm_mx(A, fa, lda, sA, ld_sa, B, fb, ldb, sB, ld_sb, C, out_dt, ldc, M, N, K, S(stream));
}

int fp8q_gemm_blockscaled_fast(const uint8_t* A, fp8q_format fa, int64_t lda, const float* sA,
                               int64_t sA_sm, int64_t sA_skb, const uint8_t* B, fp8q_format fb,
                               int64_t ldb, const float* sB, fp8q_gran gb, int64_t sB_sn,
                               int64_t sB_skb, void* C, fp8q_dtype out_dt, int64_t ldc, int64_t M,
                               int64_t N, int64_t K, void* stream) {
  return gemm_entry("gemm_blockscaled_fast", A, fa, lda, sA, sA_sm, sA_skb, B, fb, ldb, sB, gb, sB_sn,
                    sB_skb, C, out_dt, ldc, M, N, K, true, stream);
}

}  // extern "C"
