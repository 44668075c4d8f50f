/*
 * fp8q.h -- C ABI of libfp8q.so: amax-scaled FP8 quantization and the
 * block-scaled FP8 GEMM on AMD Instinct MI355X (gfx950).
 *
 * Sources cited below:
 *   [A] the PyTorch-native FP8 article, m.nxbn.cn/news/137885 (its own
 *       section numbers: 1.2 format table, 1.3 "FN" semantics, 3.1 FP8
 *       linear, 4.1 scale factors, 4.2 delayed scaling, 4.3 margin);
 *   [H] the handbook chapter "混合精度与 FP8 训练" (anrans.github.io,
 *       ai-infra-handbooks), section "FP8 训练": quant / per_tensor /
 *       per_block, the precision-per-op table, and the hardware notes on
 *       promoting partial sums every 128 elements.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers (hipMalloc'd or torch CUDA tensors)
 *     unless stated otherwise.  The caller owns every buffer: the library
 *     never allocates, frees, synchronizes or copies to the host.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default
 *     stream.  Every call is asynchronous on that stream.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     return other than FP8Q_OK means nothing was enqueued, except
 *     FP8Q_EHIP (a launch failed; fp8q_last_error() has the HIP text).
 *   - Formats: FP8Q_E4M3FN = OCP E4M3FN (bias 7, max 448, no Inf,
 *     0x7F/0xFF are NaN); FP8Q_E5M2 = OCP E5M2 (bias 15, max 57344) ([A]
 *     1.2, 1.3).  One code is one byte.
 *   - Scales are dequantization scales s (x ~= dec(q) * s), fp32:
 *     s = fl32(fl32(max(amax, eps) * margin) / MAX), MAX = 448 or 57344
 *     ([H] per_block: amax.clamp(min=1e-12) / MAX; margin from [A] 4.3).
 *   - Encoding: q = enc(fl32(x / s)) where fl32 is IEEE fp32 division and
 *     enc rounds to nearest, ties to even, saturates at +-MAX, keeps the
 *     sign of zero and maps NaN to 0x7F ([H] quant: (x / s).clamp(-MAX,
 *     MAX).to(FP8)).  Results are bit-identical to that definition.
 *   - Row-major 2-D operands with leading dimensions in elements.
 *   - Reentrant; the only global state is the thread-local error text.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8Q_OK = 0,
  FP8Q_EINVAL = 1,   /* null pointer, non-positive size, bad enum value  */
  FP8Q_ESHAPE = 2,   /* a size is not a multiple of 128 where required    */
  FP8Q_EALIGN = 3,   /* pointer or leading dimension breaks 16-B alignment */
  FP8Q_EHIP = 4,     /* the HIP runtime refused the launch                */
  FP8Q_ENOTIMPL = 5  /* combination not provided by this build            */
} fp8q_status;

typedef enum { FP8Q_F32 = 0, FP8Q_BF16 = 1 } fp8q_dtype;
typedef enum { FP8Q_E4M3FN = 0, FP8Q_E5M2 = 1 } fp8q_format;
typedef enum { FP8Q_GRAN_TENSOR = 0, FP8Q_GRAN_1x128 = 1, FP8Q_GRAN_128x128 = 2 } fp8q_gran;

/* Statistic of the amax history that sets the delayed scale ([A] 4.2: the
 * window maximum; the mean as a gentler choice; an exponential moving
 * average smoothing the amax, as Transformer Engine does; [A] 4.3). */
typedef enum { FP8Q_STAT_MAX = 0, FP8Q_STAT_MEAN = 1, FP8Q_STAT_EMA = 2 } fp8q_window_stat;

/* Delayed-scaling state ([A] 4.2 DelayedScaler): a window of the last
 * `window` amax values and the scale derived from them.  Device-resident,
 * caller-allocated (8-byte aligned), plain data (copy it to the host to
 * checkpoint it).  `ring` holds the history (first `window` entries used),
 * `pos` the next slot, `count` the number of values seen (saturating at
 * window), `scale` the dequantization scale in force, 1.0 until the window
 * fills; `stat` the fp8q_window_stat, `alpha` the EMA coefficient and `ema`
 * the EMA of every amax seen (fp64; 0 unless stat is FP8Q_STAT_EMA).
 * `amax_acc` is the running amax of the current step: the tensors quantized
 * with fp8q_quantize_tensor_delayed fold their max|x| into it, and
 * fp8q_delayed_scaler_update consumes it and sets it back to 0. */
typedef struct {
  float ring[1024];
  int32_t window;
  int32_t count;
  int32_t pos;
  float max_val;
  float eps;
  float margin;
  float scale;
  int32_t stat;
  float alpha;
  float amax_acc;
  double ema;
} fp8q_scaler;

/* Library version (major*100 + minor). */
int fp8q_version(void);

/* Text for a status code; static storage. */
const char* fp8q_status_string(int status);

/* Text of the last FP8Q_EHIP or validation failure on this thread. */
const char* fp8q_last_error(void);

/* amax = max_i |x_i| over n elements ([A] 4.1; [H] per_tensor).
 * x: n elements of dtype dt, 16-B aligned.  amax: one fp32, overwritten
 * by the reduction's last workgroup (one launch; whatever *amax held
 * before is ignored).  A NaN anywhere gives the quiet NaN 0x7FC00000;
 * +-Inf gives +Inf.  Calls in flight at the same time must not share the
 * amax buffer (different buffers are independent). */
int fp8q_amax(const void* x, fp8q_dtype dt, int64_t n, float* amax, void* stream);

/* Per-tensor quantization with a scale held in device memory, the form
 * delayed scaling uses ([A] 4.2: the scale from earlier steps quantizes
 * the current tensor; [H] per_tensor).
 * x: n elements of dtype dt, 16-B aligned.  scale: one fp32 dequant scale
 * s, read on the device when the kernel runs (e.g. &state->scale).
 * q: n codes, 16-B aligned.
 * amax_out: nullable.  When given, *amax_out = max_i |x_i| of this call's
 *   x, overwritten in the same launch (the last workgroup of the quantizing
 *   pass writes it; whatever the buffer held before is ignored).  A NaN
 *   anywhere gives the quiet NaN 0x7FC00000.  This fuses the amax that
 *   delayed scaling records for the next step into the same pass over x
 *   ([A] 4.2); hand it to fp8q_delayed_scaler_update.  Calls in flight at
 *   the same time must not share an amax_out buffer. */
int fp8q_quantize_tensor(const void* x, fp8q_dtype dt, int64_t n, fp8q_format f, const float* scale,
                         uint8_t* q, float* amax_out, void* stream);

/* fp8q_quantize_tensor that also writes the round trip: y = fl32(dec(q) * s)
 * (fp32, or rounded to nearest-even bf16; NaN -> the quiet NaN), bit for bit
 * what fp8q_dequantize makes of the codes, in the same pass over x -- the
 * handbook's quant ([H]: (x / s).clamp().to(FP8).float() * s) and the
 * quantize-dequantize of a fake-quantized forward copy ([A] 4.2).
 * y: n elements of out_dt, 16-B aligned; other arguments and errors as
 * fp8q_quantize_tensor. */
int fp8q_quantize_tensor_dq(const void* x, fp8q_dtype dt, int64_t n, fp8q_format f, const float* scale,
                            uint8_t* q, float* amax_out, void* y, fp8q_dtype out_dt, void* stream);

/* The per-tensor quantization of one delayed-scaling step ([A] 4.2: the
 * scale derived from earlier steps quantizes this step's tensor, and this
 * step's amax is recorded for the next): q = enc(fl32(x / state->scale)),
 * and max|x| is folded into state->amax_acc as a running maximum (NaN
 * winning), so several tensors or micro-batches of one step feed one
 * window entry; fp8q_delayed_scaler_update(state, NULL) then pushes it into
 * the window and sets it back to 0.  No reset launch is needed: the state
 * owns the accumulator.  With y non-null the round trip y = fl32(dec(q) *
 * s) is written in the same pass, as fp8q_quantize_tensor_dq writes it.
 * x: n elements of dtype dt, 16-B aligned; q: n codes, 16-B aligned; y:
 * nullable, n elements of out_dt, 16-B aligned; state: initialized by
 * fp8q_delayed_scaler_init[_stat], 8-B aligned.  Calls that fold into one
 * state may overlap (the fold is atomic); the update must follow them all
 * on the stream. */
int fp8q_quantize_tensor_delayed(const void* x, fp8q_dtype dt, int64_t n, fp8q_format f, fp8q_scaler* state,
                                 uint8_t* q, void* y, fp8q_dtype out_dt, void* stream);

/* Fine-grained 1x128 quantization of activations ([H] per_block(x, 1,
 * 128); DeepSeek-V3 activation tiling).  For row r and column block kb:
 *   s = scale(amax(x[r, 128kb : 128kb+128]), eps), q = enc(fl32(x/s)).
 * x: rows x cols, element (r,c) at x[r*ldx + c]; cols % 128 == 0;
 *   ldx >= cols; x and ldx*sizeof(dt) 16-B aligned.
 * q: codes at q[r*ldq + c]; ldq >= cols, 16-B aligned.
 * scales: fp32 at scales[r*ld_s + kb], ld_s >= cols/128.
 * eps: lower clamp of amax (the pages use 1e-12); must be > 0. */
int fp8q_quantize_1x128(const void* x, fp8q_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                        fp8q_format f, float eps, uint8_t* q, int64_t ldq, float* scales,
                        int64_t ld_s, void* stream);

/* Fine-grained 1x128 quantization of the transpose: the operands of the
 * weight-gradient GEMM are reduced over tokens, so activations and output
 * gradients stored [tokens, features] are needed as [features, tokens]
 * codes with one scale per 128 tokens ([H] fine-grained scaling along the
 * reduced dimension; [A] 6.3 E5M2 gradients).  Equal to fp8q_quantize_1x128
 * of x^T, without materializing x^T:
 *   for column c of x and row block rb:
 *   s = scale(amax(x[128rb : 128rb+128, c]), eps), q[c, r] = enc(fl32(x[r, c]/s)).
 * x: rows x cols, element (r,c) at x[r*ldx + c]; rows % 128 == 0,
 *   cols % 64 == 0; ldx >= cols; x and ldx*sizeof(dt) 16-B aligned.
 * q: codes of x^T at q[c*ldq + r]; ldq >= rows, q and ldq 16-B aligned.
 * scales: fp32 at scales[c*ld_s + rb], ld_s >= rows/128.
 * eps: lower clamp of amax; must be > 0. */
int fp8q_quantize_1x128_t(const void* x, fp8q_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                          fp8q_format f, float eps, uint8_t* q, int64_t ldq, float* scales,
                          int64_t ld_s, void* stream);

/* MX (microscaling) FP8 quantization: every 32 consecutive elements of a
 * row share one power-of-two scale X = 2^e held as an E8M0 byte e + 127
 * (0xFF = NaN); [H] names this hardware-native block scaling as the next
 * step after 1x128 / 128x128.  The conversion follows the OCP Microscaling
 * Formats (MX) specification v1.0, 6.3: e = floor(log2 max|x|) - emax
 * (emax = 8 for E4M3FN, 15 for E5M2), clamped to [-127, 127];
 * q = enc(x / X), round to nearest even, clamped to +-MAX.  An all-zero
 * block has e = -127; a block holding a NaN or an Inf gets scale byte 0xFF
 * and codes 0x7F.
 * x: rows x cols at x[r*ldx + c]; cols % 32 == 0; x and ldx*sizeof(dt)
 *   16-B aligned.  q: codes at q[r*ldq + c], q and ldq 16-B aligned.
 * scales: bytes at scales[r*ld_s + c/32], ld_s >= cols/32. */
int fp8q_quantize_mx(const void* x, fp8q_dtype dt, int64_t rows, int64_t cols, int64_t ldx, fp8q_format f,
                     uint8_t* q, int64_t ldq, uint8_t* scales, int64_t ld_s, void* stream);

/* MX dequantization y = fl32(dec(q) * 2^(s - 127)) (scale byte 0xFF: NaN,
 * the quiet NaN 0x7FC00000), bf16 output as RNE of that fp32.  Layouts as
 * fp8q_quantize_mx; cols % 32 == 0; q 16-B aligned with ldq % 8 == 0; y and
 * its rows 16-B aligned. */
int fp8q_dequantize_mx(const uint8_t* q, fp8q_format f, int64_t rows, int64_t cols, int64_t ldq,
                       const uint8_t* scales, int64_t ld_s, void* y, fp8q_dtype out_dt, int64_t ldy, void* stream);

/* Fine-grained 128x128 quantization of weights ([H] per_block(x, 128,
 * 128)).  As fp8q_quantize_1x128 with one scale per 128x128 tile:
 * scales[rb*ld_s + kb] for rows 128rb.. and columns 128kb..;
 * rows % 128 == 0 and cols % 128 == 0. */
int fp8q_quantize_128x128(const void* x, fp8q_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                          fp8q_format f, float eps, uint8_t* q, int64_t ldq, float* scales,
                          int64_t ld_s, void* stream);

/* Set a device-resident scaler to its initial state ([A] 4.2 __init__):
 * empty history, scale = 1.0, statistic the window maximum.  window in
 * [1, 1024] (1 gives current scaling), max_val > 0 (448 or 57344),
 * eps > 0, margin > 0 ([A] 4.3; 1.0 means none). */
int fp8q_delayed_scaler_init(fp8q_scaler* state, int32_t window, float max_val, float eps,
                             float margin, void* stream);

/* As fp8q_delayed_scaler_init with the history statistic chosen ([A] 4.2,
 * 4.3).  FP8Q_STAT_MAX: max of the window.  FP8Q_STAT_MEAN: mean of the
 * window, its values summed in fp64 by pairwise (binary-tree) summation
 * over the 1024 slots (unused slots 0), divided by window in fp64,
 * rounded to fp32.  FP8Q_STAT_EMA: e = amax for the first value, then
 * e = alpha*amax + (1-alpha)*e with each product and the sum rounded to
 * fp64 (no fused multiply-add); alpha in (0, 1]; the statistic is fl32(e)
 * and the window only sets when the scale first moves.  The scale is then
 * fl32(fl32(max(stat, eps) * margin) / max_val).  A NaN amax makes max and
 * mean NaN while it is in the window and the EMA NaN until re-init.
 * Errors: FP8Q_EINVAL for a bad stat or alpha, as above otherwise. */
int fp8q_delayed_scaler_init_stat(fp8q_scaler* state, int32_t window, float max_val, float eps,
                                  float margin, fp8q_window_stat stat, float alpha, void* stream);

/* One delayed-scaling step ([A] 4.2 update): push *amax into the ring
 * (and into the EMA); amax may be NULL, meaning the state's own amax_acc
 * (filled by fp8q_quantize_tensor_delayed).  Once `window` values have
 * been seen, scale =
 * fl32(fl32(max(stat, eps) * margin) / max_val) with stat the state's
 * statistic (max(ring) by default), otherwise the scale stays at its
 * previous value.  *amax is then reset to 0 (the quantizers overwrite it
 * anyway).  A NaN amax propagates into the scale.
 * Runs as one wavefront; never syncs with the host. */
int fp8q_delayed_scaler_update(fp8q_scaler* state, float* amax, void* stream);

/* Dequantization x^ = fl32(dec(q) * s) ([H] quant: .float() * scale),
 * written as fp32 or rounded to nearest-even bf16 (NaN -> quiet NaN).
 * q: rows x cols codes at q[r*ldq + c].  scales by granularity g:
 *   TENSOR: scales[0]; 1x128: scales[r*ld_s + c/128];
 *   128x128: scales[(r/128)*ld_s + c/128].
 * y: y[r*ldy + c] of dtype out_dt.  cols % 128 == 0 for the block
 * granularities; q and y 16-B aligned; ldq, ldy multiples of 4 (ignored
 * when rows == 1, so a flat tensor of any length is rows=1, cols=n). */
int fp8q_dequantize(const uint8_t* q, fp8q_format f, int64_t rows, int64_t cols, int64_t ldq,
                    const float* scales, fp8q_gran g, int64_t ld_s, void* y, fp8q_dtype out_dt,
                    int64_t ldy, void* stream);

/* Block-scaled FP8 GEMM ([A] 3.1 F.linear(x, w) with w stored [out, in];
 * [H] FP8 inputs with fp32 accumulation, partial sums promoted to fp32
 * every 128 elements of K):
 *   C[m,n] = sum_kb (sA[m,kb] * sB(n,kb)) * P_kb[m,n],
 *   P_kb[m,n] = sum_{k in [128kb, 128kb+128)} dec(A[m,k]) * dec(B[n,k]),
 * each P_kb formed in fp32 and folded into an fp32 accumulator.
 * Every product and every in-block sum is carried out in full fp32 (the
 * codes are decoded exactly and multiplied on the bf16 matrix cores), so
 * |C - C_exact| stays within a few fp32 roundings of
 * D[m,n] = sum_kb |sA*sB| * sum_k |dec(a)*dec(b)|.
 * A: M x K codes of format fa at A[m*lda + k].
 * sA: 1x128 scales along K at sA[m*sA_sm + kb*sA_skb].
 * B: N x K codes of format fb at B[n*ldb + k] (the weight as nn.Linear
 *   stores it, or any K-contiguous operand).
 * sB: gb = FP8Q_GRAN_128x128: sB[(n/128)*sB_sn + kb*sB_skb] (ceil(N/128) rows);
 *     gb = FP8Q_GRAN_1x128:   sB[n*sB_sn + kb*sB_skb].
 * C: M x N at C[m*ldc + n], fp32 or bf16 (round to nearest even).
 * K % 128 == 0 (else FP8Q_ESHAPE); M, N >= 1 with ragged edges masked;
 * lda, ldb >= K and multiples of 16; A, B 16-B aligned; ldc >= N.
 * NaN or Inf codes make the affected outputs non-finite. */
int fp8q_gemm_blockscaled(const uint8_t* A, fp8q_format fa, int64_t lda, const float* sA,
                          int64_t sA_sm, int64_t sA_skb, const uint8_t* B, fp8q_format fb,
                          int64_t ldb, const float* sB, fp8q_gran gb, int64_t sB_sn,
                          int64_t sB_skb, void* C, fp8q_dtype out_dt, int64_t ldc, int64_t M,
                          int64_t N, int64_t K, void* stream);

/* The same GEMM with each 128-wide block product P_kb taken from the FP8
 * matrix cores directly (twice the MFMA rate).  Arguments and layout as
 * fp8q_gemm_blockscaled.  Inside a block the hardware aligns each group of
 * eight products to the largest one and drops what lies about 2^-14 below
 * it -- the limited FP8 accumulator that motivates promotion every 128 K
 * in [H] -- so the error bound is |C - C_exact| <= 2^-10 * D[m,n] rather
 * than a few fp32 roundings; the promotion across blocks is fp32. */
int fp8q_gemm_blockscaled_fast(const uint8_t* A, fp8q_format fa, int64_t lda, const float* sA,
                               int64_t sA_sm, int64_t sA_skb, const uint8_t* B, fp8q_format fb,
                               int64_t ldb, const float* sB, fp8q_gran gb, int64_t sB_sn,
                               int64_t sB_skb, void* C, fp8q_dtype out_dt, int64_t ldc, int64_t M,
                               int64_t N, int64_t K, void* stream);

/* fp8q_gemm_blockscaled with the output quantized in the epilogue, for
 * the next layer's input ([A] 5.1: casts to and from a wide type between
 * FP8 operations eat the gain; [H] fine-grained 1x128 scaling): the fp32
 * C of fp8q_gemm_blockscaled is never written; instead, per row and 128
 * consecutive columns, Cs[m*ld_cs + n/128] = fl32(max(amax, eps) / MAX_fc)
 * and Cq[m*ldcq + n] = enc_fc(fl32(C[m,n] / s)), bit for bit what
 * fp8q_quantize_1x128 makes of that fp32 C (saturating, RNE, NaN -> 0x7F).
 * Arguments as fp8q_gemm_blockscaled (exact path) plus: fc the output
 * format, eps > 0, Cq [M, N] codes with ldcq >= N, Cs [M, N/128] fp32 with
 * ld_cs >= N/128.  N % 128 == 0 and K % 128 == 0 (else FP8Q_ESHAPE). */
int fp8q_gemm_blockscaled_q(const uint8_t* A, fp8q_format fa, int64_t lda, const float* sA, int64_t sA_sm,
                            int64_t sA_skb, const uint8_t* B, fp8q_format fb, int64_t ldb, const float* sB,
                            fp8q_gran gb, int64_t sB_sn, int64_t sB_skb, fp8q_format fc, float eps, uint8_t* Cq,
                            int64_t ldcq, float* Cs, int64_t ld_cs, int64_t M, int64_t N, int64_t K,
                            void* stream);

/* fp8q_gemm_blockscaled with the output quantized along M in the epilogue,
 * for a gradient produced by this GEMM (a dgrad whose output is the
 * previous layer's output gradient): the previous layer's weight-gradient
 * GEMM reduces over tokens (M), so it takes C^T as codes with one scale per
 * 128 tokens ([H] fine-grained 1x128 scaling along the reduced dimension;
 * [A] 6.3 gradients in E5M2; [A] 5.1 casts to and from a wide type between
 * FP8 operations eat the gain).  The fp32 C of fp8q_gemm_blockscaled is
 * never written; instead, per column n and 128 consecutive rows,
 *   Cst[n*ld_cst + m/128] = fl32(max(amax(C[128(m/128) : +128, n]), eps) / MAX_fc),
 *   Cqt[n*ldcqt + m]     = enc_fc(fl32(C[m,n] / s)),
 * bit for bit what fp8q_quantize_1x128_t makes of that fp32 C.  With Cq and
 * Cs non-null the same epilogue also writes the row-wise output of
 * fp8q_gemm_blockscaled_q (what the previous layer's dgrad takes), from the
 * same accumulators.
 * Arguments as fp8q_gemm_blockscaled (exact path) plus: fc the output
 * format, eps > 0; Cqt [N, M] codes, ldcqt >= M, Cqt and ldcqt 16-B
 * aligned; Cst [N, M/128] fp32, ld_cst >= M/128; Cq, Cs nullable together
 * (ldcq >= N, ld_cs >= N/128).  M % 128 == 0 and K % 128 == 0, and
 * N % 128 == 0 when Cq is given (else FP8Q_ESHAPE); otherwise N >= 1. */
int fp8q_gemm_blockscaled_qt(const uint8_t* A, fp8q_format fa, int64_t lda, const float* sA, int64_t sA_sm,
                             int64_t sA_skb, const uint8_t* B, fp8q_format fb, int64_t ldb, const float* sB,
                             fp8q_gran gb, int64_t sB_sn, int64_t sB_skb, fp8q_format fc, float eps, uint8_t* Cqt,
                             int64_t ldcqt, float* Cst, int64_t ld_cst, uint8_t* Cq, int64_t ldcq, float* Cs,
                             int64_t ld_cs, int64_t M, int64_t N, int64_t K, void* stream);

/* MX GEMM ([H] FP8 training, hardware note: 32 elements share one scale
 * factor in hardware): C[m,n] = sum over 32-element K blocks kb of
 *   2^(sA[m,kb] - 127) * 2^(sB[n,kb] - 127) * sum_{k in kb} dec(A[m,k]) dec(B[n,k]),
 * the product of two fp8q_quantize_mx outputs (B as [N,K], K-contiguous).
 * The scaled FP8 MFMA of gfx950 applies both scales and accumulates the
 * whole K in fp32; like fp8q_gemm_blockscaled_fast it is bounded by
 * |C - C_exact| <= 2^-10 * D, D the same sum over |terms|, while the scaled
 * terms stay in fp32's normal range (products of two scales far from 1 can
 * underflow to zero or overflow to Inf in fp32).
 * A [M,K] codes, lda; B [N,K] codes, ldb (16-B aligned rows); sA [M, K/32]
 * and sB [N, K/32] E8M0 bytes with row strides ld_sa, ld_sb (multiples of
 * 4, >= K/32); K % 128 == 0; M, N free.  C [M,N] fp32 or bf16 (RNE), ldc.
 * A scale byte 0xFF makes the result unspecified (NaN blocks). */
int fp8q_gemm_mx(const uint8_t* A, fp8q_format fa, int64_t lda, const uint8_t* sA, int64_t ld_sa,
                 const uint8_t* B, fp8q_format fb, int64_t ldb, const uint8_t* sB, int64_t ld_sb, void* C,
                 fp8q_dtype out_dt, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
