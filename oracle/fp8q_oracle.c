/*
 * fp8q oracle -- a plain, slow, deliberately obvious CPU implementation of
 * amax-scaled FP8 quantization and the block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the GPU library is
 * checked against; it is never part of the product path.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it.  It
 * shares no header, table, helper or constant generator with the HIP code.
 *
 * Arithmetic: fp64 or exact integers wherever the method leaves a choice;
 * fp32 exactly where the method itself computes in fp32 (x/s, amax/MAX,
 * q*s).  Build with  gcc -O2 -fno-fast-math -ffp-contract=off  so every
 * float operation is one IEEE-754 binary32 operation (x86-64 SSE).
 *
 * Sources.  [A] = the PyTorch-native FP8 article at m.nxbn.cn/news/137885;
 * its sections are cited by its own numbers (1.2 format table, 1.3 "FN"
 * semantics, 2.2 scalar experiment, 4.1-4.3 scale factors / DelayedScaler).
 * [H] = the handbook chapter "混合精度与 FP8 训练" (anrans.github.io
 * ai-infra-handbooks), section "FP8 训练" (quant, per_tensor, per_block,
 * rel_err and the hardware notes on 128-element promotion) and its second
 * exercise (one outlier of 5000).
 *
 * Readings where the pages are silent or disagree (each also listed in the
 * design notes): 0x7F/0xFF of E4M3FN are NaN (max finite is 448 per [A] 1.2
 * and [H]); E5M2 exponent 31 is Inf (m=0) / NaN; rounding is
 * round-to-nearest-even; overflow saturates to +-MAX for both formats;
 * signed zero is kept; a NaN input encodes as 0x7F; NaN propagates through
 * amax; scales are dequant scales s = max(amax, eps)*margin / MAX.
 *
 * MX (microscaling) FP8, which [H] names as the next, hardware-native step
 * of fine-grained scaling without giving its algorithm, follows the public
 * OCP Microscaling Formats (MX) specification v1.0, section 6.3; its
 * readings are listed beside orc_quantize_mx below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E4M3FN 0
#define ORC_E5M2 1
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_GRAN_TENSOR 0
#define ORC_GRAN_1x128 1
#define ORC_GRAN_128x128 2

/* ------------------------------------------------------------------ */
/* Format parameters, [A] 1.2: E4M3 = 1/4/3 bits, bias 7, max 448;     */
/* E5M2 = 1/5/2 bits, bias 15, max 57344.                              */
/* ------------------------------------------------------------------ */
static int mant_bits(int fmt) { return fmt == ORC_E4M3FN ? 3 : 2; }
static int exp_bias(int fmt) { return fmt == ORC_E4M3FN ? 7 : 15; }

double orc_max_finite(int fmt) { return fmt == ORC_E4M3FN ? 448.0 : 57344.0; }

/* bf16 is the top half of a binary32; widening is exact. */
static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float load_elem(const void* x, int dt, int64_t i) {
  if (dt == ORC_F32) return ((const float*)x)[i];
  return bf16_to_f32(((const uint16_t*)x)[i]);
}

static float canonical_nan(void) {
  uint32_t u = 0x7FC00000u;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------ */
/* decode one code to its exact value (every FP8 value is exact in */
/* double).  Field widths and bias from [A] 1.2.                       */
/* ------------------------------------------------------------------ */
double orc_decode(uint32_t code, int fmt) {
  code &= 0xFF;
  double sign = (code & 0x80) ? -1.0 : 1.0;
  int M = mant_bits(fmt), bias = exp_bias(fmt);
  int e = (int)((code & 0x7F) >> M);
  int m = (int)(code & ((1u << M) - 1));
  if (fmt == ORC_E4M3FN) {
    if (e == 15 && m == 7) return NAN; /* only NaN pattern, no Inf */
  } else {
    if (e == 31) return m == 0 ? sign * INFINITY : NAN;
  }
  if (e == 0) /* subnormal: m * 2^(1 - bias - M) */
    return sign * ldexp((double)m, 1 - bias - M);
  return sign * ldexp((double)((1 << M) + m), e - bias - M);
}

/* ------------------------------------------------------------------ */
/* saturating round-to-nearest-even encoder (encoder "A").         */
/* Every rescaling below is by a power of two, so it is exact in       */
/* double; nearbyint() rounds half to even in the default mode.        */
/* ------------------------------------------------------------------ */
uint32_t orc_encode(float v, int fmt) {
  if (isnan(v)) return 0x7F;
  int M = mant_bits(fmt), bias = exp_bias(fmt);
  int emin = 1 - bias; /* exponent of the smallest normal */
  uint32_t sgn = signbit(v) ? 0x80u : 0u;
  double a = fabs((double)v);
  double maxv = orc_max_finite(fmt);
  if (a > maxv) a = maxv; /* saturate; +-Inf also lands here */
  if (a < ldexp(1.0, emin)) {
    /* subnormal range: a count of quanta 2^(emin-M); k == 2^M is exactly
       the code of the smallest normal, so no special case is needed */
    double k = nearbyint(ldexp(a, M - emin));
    return sgn | (uint32_t)k;
  }
  int E;
  (void)frexp(a, &E);
  E -= 1; /* a = f * 2^E with f in [1, 2) */
  double k = nearbyint(ldexp(a, M - E)); /* in [2^M, 2^(M+1)] */
  if (k == ldexp(1.0, M + 1)) {          /* rounded up into the next binade */
    E += 1;
    k = ldexp(1.0, M);
  }
  return sgn | ((uint32_t)(E + bias) << M) | (uint32_t)(k - ldexp(1.0, M));
}

/* Encode a whole fp32 buffer (used by the exhaustive cross-checks). */
void orc_encode_array(const float* v, int64_t n, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_encode(v[i], fmt);
}

/* Encode the fp32 values whose bit patterns are lo, lo+1, ..., lo+n-1. */
void orc_encode_bits_range(uint32_t lo, int64_t n, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = lo + (uint32_t)i;
    float f;
    memcpy(&f, &u, 4);
    out[i] = (uint8_t)orc_encode(f, fmt);
  }
}

/* ------------------------------------------------------------------ */
/* amax = max |x| over a granule; a NaN anywhere makes it NaN.     */
/* ([A] 4.1 and 4.2 update(); [H] per_tensor / per_block)              */
/* ------------------------------------------------------------------ */
float orc_amax(const void* x, int dt, int64_t n) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(load_elem(x, dt, i));
    if (isnan(a)) return canonical_nan();
    if (a > m) m = a;
  }
  return m;
}

/* ------------------------------------------------------------------ */
/* dequant scale s = fl32(fl32(max(amax, eps) * margin) / MAX).    */
/* [H] per_block: amax.clamp(min=1e-12) / MAX; [A] 4.3 margin.         */
/* A NaN amax gives a NaN scale (the comparison below is false).       */
/* ------------------------------------------------------------------ */
float orc_scale(float amax, float max_val, float eps, float margin) {
  float m = (amax < eps) ? eps : amax;
  float t = m * margin;
  return t / max_val;
}

/* one element, q = enc(fl32(x / s)); [H] quant: (x / s).clamp().to(FP8) */
uint32_t orc_quantize_value(float x, float s, int fmt) {
  float y = x / s;
  return orc_encode(y, fmt);
}

/* ------------------------------------------------------------------ */
/* granule drivers                                                  */
/* ------------------------------------------------------------------ */

/* Per-tensor (or delayed) scaling with a given dequant scale s. */
void orc_quantize_tensor(const void* x, int dt, int64_t n, int fmt, float s, uint8_t* q) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) q[i] = (uint8_t)orc_quantize_value(load_elem(x, dt, i), s, fmt);
}

/* Block scaling with br x bc blocks ([H] per_block: reshape into
   (R/br, br, C/bc, bc), amax over dims (1,3), clamp, / MAX).
   Element (r, c) lives at x[r*ldx + c]; its code at q[r*ldq + c];
   the scale of block (rb, cb) at scales[rb*ld_s + cb]. */
void orc_quantize_blocks(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx,
                         int64_t br, int64_t bc, int fmt, float eps, uint8_t* q, int64_t ldq,
                         float* scales, int64_t ld_s) {
  int64_t nrb = rows / br, ncb = cols / bc;
  float max_val = (float)orc_max_finite(fmt);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t rb = 0; rb < nrb; ++rb) {
    for (int64_t cb = 0; cb < ncb; ++cb) {
      float amax = 0.0f;
      int has_nan = 0;
      for (int64_t r = rb * br; r < (rb + 1) * br; ++r)
        for (int64_t c = cb * bc; c < (cb + 1) * bc; ++c) {
          float a = fabsf(load_elem(x, dt, r * ldx + c));
          if (isnan(a)) has_nan = 1;
          else if (a > amax) amax = a;
        }
      if (has_nan) amax = canonical_nan();
      float s = orc_scale(amax, max_val, eps, 1.0f);
      scales[rb * ld_s + cb] = s;
      for (int64_t r = rb * br; r < (rb + 1) * br; ++r)
        for (int64_t c = cb * bc; c < (cb + 1) * bc; ++c)
          q[r * ldq + c] = (uint8_t)orc_quantize_value(load_elem(x, dt, r * ldx + c), s, fmt);
    }
  }
}

/* ------------------------------------------------------------------ */
/* dequantize x^ = fl32(dec(q) * s), optionally rounded to bf16.   */
/* [H] quant: .float() * scale.  dec(q) has <= 4 significant bits and s */
/* 24, so the double product is exact and the cast rounds once.        */
/* ------------------------------------------------------------------ */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return 0x7FC0;
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void orc_dequantize(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                    const float* scales, int gran, int64_t ld_s, void* y, int out_dt, int64_t ldy) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      float s;
      if (gran == ORC_GRAN_TENSOR) s = scales[0];
      else if (gran == ORC_GRAN_1x128) s = scales[r * ld_s + c / 128];
      else s = scales[(r / 128) * ld_s + c / 128];
      float v = (float)(orc_decode(q[r * ldq + c], fmt) * (double)s);
      if (isnan(v)) v = canonical_nan();  /* a NaN the library writes is the quiet NaN */
      if (out_dt == ORC_F32) ((float*)y)[r * ldy + c] = v;
      else ((uint16_t*)y)[r * ldy + c] = f32_to_bf16_rne(v);
    }
}

/* ------------------------------------------------------------------ */
/* delayed scaling ([A] 4.2 DelayedScaler): a window of the last    */
/* `window` amax values; once it is full, the scale becomes             */
/* scale(stat(window)); until then it stays at its initial 1.0.  The    */
/* scale in force at step t quantizes x_t; amax(x_t) is pushed after.   */
/* stat ([A] 4.2: the window maximum, the mean as a gentler option, and */
/* the exponential moving average that smooths amax changes; [A] 4.3):  */
/*   0 max of the window;                                               */
/*   1 mean of the window: the window's values summed in fp64 by        */
/*     pairwise (binary-tree) summation over the 1024 slots, unused      */
/*     slots 0, divided by `window` in fp64, rounded to fp32;            */
/*   2 EMA: e_1 = amax_1, e_t = alpha*amax_t + (1-alpha)*e_{t-1}, each   */
/*     product and the sum rounded to fp64, e kept in fp64; the scale    */
/*     uses fl32(e).  The window only sets when the scale first moves.  */
/* NaN: max and mean propagate a NaN while it is in the window; the     */
/* EMA keeps it for good.                                               */
/* ------------------------------------------------------------------ */
typedef struct {
  float ring[1024];
  int32_t window, count, pos;
  float max_val, eps, margin;
  float scale;
  int32_t stat;
  float alpha;
  int32_t pad_;
  double ema;
} orc_scaler;

int orc_scaler_init_stat(orc_scaler* st, int32_t window, float max_val, float eps, float margin, int32_t stat,
                         float alpha) {
  if (window < 1 || window > 1024) return 1;
  if (stat < 0 || stat > 2) return 1;
  if (stat == 2 && !(alpha > 0.0f && alpha <= 1.0f)) return 1;
  memset(st, 0, sizeof(*st));
  st->window = window;
  st->max_val = max_val;
  st->eps = eps;
  st->margin = margin;
  st->scale = 1.0f;
  st->stat = stat;
  st->alpha = stat == 2 ? alpha : 0.0f;
  return 0;
}

int orc_scaler_init(orc_scaler* st, int32_t window, float max_val, float eps, float margin) {
  return orc_scaler_init_stat(st, window, max_val, eps, margin, 0, 0.0f);
}

/* pairwise sum of n (a power of two) fp64 values */
static double pairwise_sum(const double* v, int n) {
  if (n == 1) return v[0];
  double left = pairwise_sum(v, n / 2);
  double right = pairwise_sum(v + n / 2, n / 2);
  return left + right;
}

void orc_scaler_update(orc_scaler* st, float amax) {
  int first = st->count == 0;
  st->ring[st->pos] = amax;
  st->pos = (st->pos + 1) % st->window;
  if (st->count < st->window) st->count += 1;
  if (st->stat == 2) {
    if (first) {
      st->ema = (double)amax;
    } else {
      double a = (double)st->alpha;
      double t1 = a * (double)amax;
      double t2 = (1.0 - a) * st->ema;
      st->ema = t1 + t2;
    }
  }
  if (st->count < st->window) return;
  float m;
  if (st->stat == 0) {
    m = 0.0f;
    int has_nan = 0;
    for (int32_t i = 0; i < st->window; ++i) {
      if (isnan(st->ring[i])) has_nan = 1;
      else if (st->ring[i] > m) m = st->ring[i];
    }
    if (has_nan) m = canonical_nan();
  } else if (st->stat == 1) {
    double v[1024];
    for (int i = 0; i < 1024; ++i) v[i] = i < st->window ? (double)st->ring[i] : 0.0;
    double mean = pairwise_sum(v, 1024) / (double)st->window;
    m = (float)mean;
  } else {
    m = (float)st->ema;
  }
  if (isnan(m)) m = canonical_nan();
  st->scale = orc_scale(m, st->max_val, st->eps, st->margin);
}

int64_t orc_scaler_size(void) { return (int64_t)sizeof(orc_scaler); }

/* ------------------------------------------------------------------ */
/* block-scaled GEMM                                               */
/*   C[m,n] = sum_kb (sA[m,kb] * sB[.,kb]) * P_kb[m,n],                 */
/*   P_kb[m,n] = sum_{k in block kb} dec(A[m,k]) * dec(B[n,k]).         */
/* ([H] per-op table: FP8 inputs with fp32 accumulation; hardware      */
/* notes: partial sums promoted every 128 elements of K.)               */
/* Every finite E4M3 value is an integer multiple of 2^-9 and every     */
/* E5M2 value a multiple of 2^-16, so dec(.) * 2^16 is an integer and   */
/* P_kb * 2^32 is an exact __int128 sum.  The coefficient sA*sB is      */
/* exact in double (24 x 24 bits).  The outer sum over kb is fp64.      */
/* D[m,n] = sum_kb |sA*sB| * sum_k |dec(a)*dec(b)| is the scale of the  */
/* rounding error any fp32 evaluation may commit.                       */
/* A NaN or Inf code anywhere in a dot product makes C NaN there.       */
/* ------------------------------------------------------------------ */
static void int_table(int fmt, int64_t tab[256], unsigned char ok[256]) {
  for (uint32_t c = 0; c < 256; ++c) {
    double v = orc_decode(c, fmt);
    ok[c] = (unsigned char)(isfinite(v) != 0);
    tab[c] = ok[c] ? (int64_t)ldexp(v, 16) : 0; /* exact: v is a multiple of 2^-16 */
  }
}

void orc_gemm_blockscaled(const uint8_t* A, int fa, int64_t lda, const float* sA, int64_t sA_sm,
                          int64_t sA_skb, const uint8_t* B, int fb, int64_t ldb, const float* sB,
                          int gb, int64_t sB_sn, int64_t sB_skb, int64_t M, int64_t N, int64_t K,
                          const int64_t* rows, int64_t nrows, double* C, double* D) {
  int64_t ta[256], tb[256];
  unsigned char oka[256], okb[256];
  int_table(fa, ta, oka);
  int_table(fb, tb, okb);
  int64_t nkb = K / 128;
  int64_t nr = rows ? nrows : M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ri = 0; ri < nr; ++ri) {
    int64_t m = rows ? rows[ri] : ri;
    const uint8_t* arow = A + m * lda;
    for (int64_t n = 0; n < N; ++n) {
      const uint8_t* brow = B + n * ldb;
      double c = 0.0, d = 0.0;
      int special = 0;
      for (int64_t kb = 0; kb < nkb; ++kb) {
        __int128 p = 0, pabs = 0;
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k) {
          if (!oka[arow[k]] || !okb[brow[k]]) {
            special = 1;
            continue;
          }
          __int128 t = (__int128)ta[arow[k]] * (__int128)tb[brow[k]];
          p += t;
          pabs += t < 0 ? -t : t;
        }
        double sa = (double)sA[m * sA_sm + kb * sA_skb];
        double sb = (gb == ORC_GRAN_128x128) ? (double)sB[(n / 128) * sB_sn + kb * sB_skb]
                                              : (double)sB[n * sB_sn + kb * sB_skb];
        double coef = sa * sb; /* exact */
        c += coef * ldexp((double)p, -32);
        d += fabs(coef) * ldexp((double)pabs, -32);
      }
      if (special) c = NAN;
      C[ri * N + n] = c;
      D[ri * N + n] = d;
    }
  }
}

/* ------------------------------------------------------------------ */
/* MX (microscaling) FP8.  The handbook names hardware-native block     */
/* scaling with 32-element blocks and power-of-two (E8M0) shared scales */
/* as the next step after 1x128 / 128x128 scaling; the pages give no    */
/* algorithm, so this follows the public OCP Microscaling Formats (MX)  */
/* specification v1.0 (section 6.3, conversion of a vector to MX):      */
/*   e = floor(log2(max_i |V_i|)) - emax_elem,  X = 2^e,                */
/*   P_i = quantize_to_element_format(V_i / X)  (RNE, clamped to the    */
/*         largest normal),                                             */
/* emax_elem = exponent of the element format's largest normal: 8 for   */
/* E4M3 (448 = 1.75 * 2^8), 15 for E5M2 (57344 = 1.75 * 2^15).  X is    */
/* stored as the E8M0 byte e + 127 (0xFF = NaN).  Readings where the    */
/* specification leaves room: max |V| == 0 gives e = -127 (every code   */
/* +-0); a NaN or an Inf in the block gives the NaN scale 0xFF and NaN  */
/* codes 0x7F; e is clamped to [-127, 127].  Blocks are 32 consecutive  */
/* elements of a row.                                                   */
/* ------------------------------------------------------------------ */
static int emax_elem(int fmt) { return fmt == ORC_E4M3FN ? 8 : 15; }

void orc_quantize_mx(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                     int64_t ldq, uint8_t* scales, int64_t ld_s) {
  int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      double amax = 0.0;
      int special = 0;
      for (int64_t c = 32 * b; c < 32 * b + 32; ++c) {
        float v = load_elem(x, dt, r * ldx + c);
        if (isnan(v) || isinf(v)) special = 1;
        else if (fabs((double)v) > amax) amax = fabs((double)v);
      }
      if (special) {
        scales[r * ld_s + b] = 0xFF;
        for (int64_t c = 32 * b; c < 32 * b + 32; ++c) q[r * ldq + c] = 0x7F;
        continue;
      }
      int e = -127;
      if (amax > 0.0) {
        int E;
        (void)frexp(amax, &E); /* amax = f * 2^E, f in [0.5, 1): floor(log2 amax) = E - 1 */
        e = (E - 1) - emax_elem(fmt);
      }
      if (e < -127) e = -127;
      if (e > 127) e = 127;
      scales[r * ld_s + b] = (uint8_t)(e + 127);
      for (int64_t c = 32 * b; c < 32 * b + 32; ++c) {
        /* V / 2^e is exact in double; as a float it is exact whenever it
           is at least the smallest FP8 subnormal, and anything below
           half of that encodes as +-0 however it is rounded */
        float y = (float)ldexp((double)load_elem(x, dt, r * ldx + c), -e);
        q[r * ldq + c] = (uint8_t)orc_encode(y, fmt);
      }
    }
}

/* x^ = fl32(dec(q) * 2^(s - 127)); scale byte 0xFF makes NaN. */
void orc_dequantize_mx(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                       const uint8_t* scales, int64_t ld_s, float* y, int64_t ldy) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      uint8_t sb = scales[r * ld_s + c / 32];
      double v = sb == 0xFF ? NAN : ldexp(orc_decode(q[r * ldq + c], fmt), (int)sb - 127);
      float f = (float)v;
      y[r * ldy + c] = isnan(f) ? canonical_nan() : f;
    }
}

/* MX GEMM: C[m,n] = sum_kb 2^(ea + eb) * sum_{k in 32-block kb} dec(A[m,k]) dec(B[n,k]),
   A [M,K] and B [N,K] K-contiguous, E8M0 scales sA[m*ld_sa + kb], sB[n*ld_sb + kb].
   Block sums exact in __int128 (codes times 2^16 are integers), outer sum fp64.
   D = sum_kb 2^(ea+eb) sum_k |dec(a) dec(b)|; a NaN or Inf code or a NaN scale
   in a dot product makes C NaN there. */
void orc_gemm_mx(const uint8_t* A, int fa, int64_t lda, const uint8_t* sA, int64_t ld_sa, const uint8_t* B,
                 int fb, int64_t ldb, const uint8_t* sB, int64_t ld_sb, int64_t M, int64_t N, int64_t K,
                 const int64_t* rows, int64_t nrows, double* C, double* D) {
  int64_t ta[256], tb[256];
  unsigned char oka[256], okb[256];
  int_table(fa, ta, oka);
  int_table(fb, tb, okb);
  int64_t nkb = K / 32;
  int64_t nr = rows ? nrows : M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ri = 0; ri < nr; ++ri) {
    int64_t m = rows ? rows[ri] : ri;
    const uint8_t* arow = A + m * lda;
    for (int64_t n = 0; n < N; ++n) {
      const uint8_t* brow = B + n * ldb;
      double c = 0.0, d = 0.0;
      int special = 0;
      for (int64_t kb = 0; kb < nkb; ++kb) {
        uint8_t ea = sA[m * ld_sa + kb], eb = sB[n * ld_sb + kb];
        if (ea == 0xFF || eb == 0xFF) special = 1;
        __int128 p = 0, pabs = 0;
        for (int64_t k = kb * 32; k < kb * 32 + 32; ++k) {
          if (!oka[arow[k]] || !okb[brow[k]]) {
            special = 1;
            continue;
          }
          __int128 t = (__int128)ta[arow[k]] * (__int128)tb[brow[k]];
          p += t;
          pabs += t < 0 ? -t : t;
        }
        int sh = (int)ea + (int)eb - 254 - 32;
        c += ldexp((double)p, sh);
        d += ldexp((double)pabs, sh);
      }
      if (special) c = NAN;
      C[ri * N + n] = c;
      D[ri * N + n] = d;
    }
  }
}

int orc_version(void) { return 1; }

/* Thread count of the OpenMP loops above (timing of the oracle on one core
 * beside all cores); the results do not depend on it. */
#include <omp.h>
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }
