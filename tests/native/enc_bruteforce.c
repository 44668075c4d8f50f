/*
 * Independent brute-force FP8 encoder, used only by the tests to pin the
 * oracle's formula-based encoder.  It knows nothing about exponents or
 * mantissas: it lists every finite non-negative value of the format once,
 * then encodes by picking the nearest listed value (saturating at the
 * largest), breaking exact ties toward the code whose last bit is 0.
 * NaN encodes as 0x7F; the sign bit is copied, so -0.0 gives 0x80.
 * Value list: for each code c in 0..0x7F, v(c) = m * 2^(e - bias - M) with
 * the implicit leading one added for e > 0 (PyTorch-native FP8 article,
 * section 1.2 format table), skipping the format's NaN/Inf patterns.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef struct { int n; double val[128]; uint8_t code[128]; } table_t;

static void make_table(int fmt, table_t* t) {
  int M = fmt == 0 ? 3 : 2, bias = fmt == 0 ? 7 : 15;
  t->n = 0;
  for (int c = 0; c < 128; ++c) {
    int e = c >> M, m = c & ((1 << M) - 1);
    if (fmt == 0 && e == 15 && m == 7) continue;  /* E4M3FN NaN */
    if (fmt == 1 && e == 31) continue;            /* E5M2 Inf/NaN */
    double v = e == 0 ? ldexp((double)m, 1 - bias - M) : ldexp((double)((1 << M) + m), e - bias - M);
    t->val[t->n] = v;
    t->code[t->n] = (uint8_t)c;
    t->n++;
  }
}

static uint8_t enc_b(const table_t* t, float f) {
  if (isnan(f)) return 0x7F;
  uint8_t sgn = signbit(f) ? 0x80 : 0;
  double a = fabs((double)f);
  /* beyond the largest listed value, distances to neighbouring large values
     can round to the same double, so saturation is taken first */
  if (a >= t->val[t->n - 1]) return sgn | t->code[t->n - 1];
  /* nearest by exhaustive scan of the whole list */
  int best = 0;
  double bd = fabs(a - t->val[0]);
  for (int i = 1; i < t->n; ++i) {
    double d = fabs(a - t->val[i]);
    if (d < bd || (d == bd && (t->code[i] & 1) == 0 && (t->code[best] & 1) == 1)) { best = i; bd = d; }
  }
  return sgn | t->code[best];
}

/* codes for the fp32 bit patterns lo, lo+stride, lo+2*stride, ... (n of them) */
void encb_bits(uint32_t lo, uint32_t stride, int64_t n, int fmt, uint8_t* out) {
  table_t t;
  make_table(fmt, &t);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = lo + (uint32_t)i * stride;
    float f;
    memcpy(&f, &u, 4);
    out[i] = enc_b(&t, f);
  }
}
