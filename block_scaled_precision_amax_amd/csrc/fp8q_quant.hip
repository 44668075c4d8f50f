// Amax-scaled FP8 quantizers for gfx950: amax, per-tensor (delayed) with a
// fused running amax, fine-grained 1x128 and 128x128, the delayed scaler
// and dequantization.
//
// What is computed follows the handbook chapter "混合精度与 FP8 训练",
// section "FP8 训练" (quant / per_tensor / per_block) and the PyTorch-native
// FP8 article (m.nxbn.cn/news/137885), sections 1.2-1.3 (formats) and
// 4.1-4.3 (amax, scale factors, DelayedScaler, margin).  Every code and
// scale is the one the IEEE definition q = enc(fl32(x / s)),
// s = fl32(max(amax, eps) / MAX) gives; see fp8q_internal.h for the
// division and the cast.
//
// All of these kernels are HBM-bound streams: 16-byte loads with lanes
// on consecutive addresses, the reductions in registers and DPP, codes
// packed four to a dword by the hardware conversion.
#include "fp8q_internal.h"

namespace fp8q {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

static constexpr int kThreads = 256;

// Largest |bf16| bit pattern of a dword pair, by a packed 16-bit max.
__device__ __forceinline__ uint32_t pk_absmax(uint32_t acc, uint32_t v) {
  u16x2 a = __builtin_bit_cast(u16x2, acc);
  u16x2 b = __builtin_bit_cast(u16x2, v & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}
// Fold the two halves of a packed bf16 max into an fp32 abs bit pattern.
__device__ __forceinline__ uint32_t pk_fold(uint32_t acc) {
  return max(acc & 0xFFFFu, acc >> 16) << 16;
}

// Workgroup-wide maximum of one value per thread (TH threads).
template <int TH = kThreads>
__device__ __forceinline__ uint32_t block_max(uint32_t v) {
  __shared__ uint32_t part[TH / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = part[0];
#pragma unroll
  for (int i = 1; i < TH / 64; ++i) m = max(m, part[i]);
  __syncthreads();
  return m;
}

// Folds a workgroup's maximum into *p (a running maximum on the bit pattern;
// non-negative floats order like their bit patterns, NaN patterns above
// +Inf).  The value only grows, so a workgroup whose maximum does not exceed
// the one already there skips the atomic: one relaxed read instead of an
// atomic per workgroup (same-address atomics serialize, tens of
// nanoseconds each on this chip).
__device__ __forceinline__ void fold_max(uint32_t* p, uint32_t m) {
  if (m > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(p, m);
}

// The reset of an output that a reduction then folds into.
__global__ void k_set_u32(uint32_t* p, uint32_t v) { *p = v; }

// ---------------------------------------------------------------- amax
// One read of x; per-thread max of |x| bit patterns, then one atomic max
// per workgroup on the fp32 pattern (non-negative floats order like their
// bit patterns, so the result does not depend on the order).
// Work is cut into contiguous chunks of kU x 256 16-byte vectors;
// each workgroup walks its own chunks, lanes on consecutive addresses in
// every load.  On gfx950 this keeps HBM streaming near its best rate at any
// grid size, where grid-strided vectors lose up to a quarter of it.
// Per-kernel chunk depth (16-byte vectors per lane) and persistent grid
// (workgroups per CU), chosen by measurement on MI355X: the read-only amax
// wants few long-lived workgroups, the quantizers more wavefronts in flight
// to cover their arithmetic.
#ifndef FP8Q_KU_A
#define FP8Q_KU_A 8
#endif
#ifndef FP8Q_G_A
#define FP8Q_G_A 2
#endif
#ifndef FP8Q_KU_T
#define FP8Q_KU_T 2
#endif
#ifndef FP8Q_G_T
#define FP8Q_G_T 8
#endif
#ifndef FP8Q_G_TDQ
#define FP8Q_G_TDQ 32  // the per-tensor quantizer writing the round trip as well
#endif
#ifndef FP8Q_TH_T
#define FP8Q_TH_T 256  // threads per workgroup of the per-tensor quantizer
#endif
#ifndef FP8Q_G_MX
#define FP8Q_G_MX 128
#endif
#ifndef FP8Q_KU_MX
#define FP8Q_KU_MX 1
#endif
#ifndef FP8Q_G_1
#define FP8Q_G_1 64
#endif
#ifndef FP8Q_KU_D
#define FP8Q_KU_D 2
#endif
#ifndef FP8Q_G_D
#define FP8Q_G_D 64
#endif
#ifndef FP8Q_G_DMX
#define FP8Q_G_DMX 128
#endif

template <int DT>
__device__ __forceinline__ uint32_t vec_absmax(uint32_t m, const u32x4& v) {
  if constexpr (DT == FP8Q_F32) {
    m = max(m, max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu));
    return max(m, max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
  } else {
    m = pk_absmax(m, v.x);
    m = pk_absmax(m, v.y);
    m = pk_absmax(m, v.z);
    return pk_absmax(m, v.w);
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_amax(const void* __restrict__ x, int64_t n,
                                                   uint32_t* __restrict__ out) {
  constexpr int kU = FP8Q_KU_A;
  constexpr int64_t kChunk = (int64_t)kU * kThreads;
  const int64_t per_vec = DT == FP8Q_F32 ? 4 : 8;
  const int64_t nvec = n / per_vec;
  const u32x4* xv = (const u32x4*)x;
  uint32_t m = 0;
  for (int64_t c = blockIdx.x; c * kChunk < nvec; c += gridDim.x) {
    const int64_t base = c * kChunk + threadIdx.x;
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      v[u] = base + u * kThreads < nvec ? __builtin_nontemporal_load(xv + base + u * kThreads) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kU; ++u) m = vec_absmax<DT>(m, v[u]);
  }
  if constexpr (DT == FP8Q_BF16) m = pk_fold(m);
  // tail elements (n not a multiple of the vector width)
  if (blockIdx.x == 0) {
    for (int64_t j = nvec * per_vec + threadIdx.x; j < n; j += kThreads) {
      uint32_t b = DT == FP8Q_F32 ? ((const uint32_t*)x)[j]
                                  : (uint32_t)((const uint16_t*)x)[j] << 16;
      m = max(m, b & 0x7FFFFFFFu);
    }
  }
  m = block_max(m);
  if (threadIdx.x == 0) fold_max(out, canon_abs_bits(m));
}

// ---------------------------------------------------------------- per-tensor
// Quantize with the scale at *scale (read on the device), folding max|x|
// into *amax_acc when given.  The fast path divides with div_rn_wide; a
// vector holding a NaN re-encodes its
// elements one by one (NaN -> 0x7F), and a scale outside [2^-80, 2^80] (or
// NaN / zero / Inf) takes IEEE division for every element.
template <int FMT>
__device__ __forceinline__ uint32_t quant4_fast(float a, float b, float c, float d, float s, float r) {
  return pack4<FMT>(sat<FMT>(div_rn_wide(a, s, r)), sat<FMT>(div_rn_wide(b, s, r)),
                    sat<FMT>(div_rn_wide(c, s, r)), sat<FMT>(div_rn_wide(d, s, r)));
}
template <int FMT>
__device__ __forceinline__ uint32_t quant4_exact(float a, float b, float c, float d, float s) {
  return enc1<FMT>(a / s) | (enc1<FMT>(b / s) << 8) | (enc1<FMT>(c / s) << 16) |
         (enc1<FMT>(d / s) << 24);
}

// Code -> fp32 (exact, two codes per conversion) and the canonical NaN.
template <int FMT>
__device__ __forceinline__ float2 dec2(uint32_t w, bool hi) {
  if constexpr (FMT == FP8Q_E4M3FN) {
    auto t = hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    return make_float2(t[0], t[1]);
  } else {
    auto t = hi ? __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    return make_float2(t[0], t[1]);
  }
}

__device__ __forceinline__ float canon_nan(float f) {
  return f != f ? __uint_as_float(0x7FC00000u) : f;
}

// Dequantized values of one codes word (4 codes), y = fl32(dec(q) * s) with
// NaN made 0x7FC00000, written as fp32 or RNE bf16 at element i4 of y --
// the arithmetic of fp8q_dequantize, so the fused output matches it bit
// for bit.
template <int FMT, int ODT>
__device__ __forceinline__ void store_dq4(uint32_t w, float s, void* __restrict__ y, int64_t i4) {
  const float2 lo = dec2<FMT>(w, false), hi = dec2<FMT>(w, true);
  const float o0 = canon_nan(lo.x * s), o1 = canon_nan(lo.y * s), o2 = canon_nan(hi.x * s), o3 = canon_nan(hi.y * s);
  if constexpr (ODT == FP8Q_F32) {
    __builtin_nontemporal_store(u32x4{__float_as_uint(o0), __float_as_uint(o1), __float_as_uint(o2), __float_as_uint(o3)},
                                (u32x4*)((float*)y + i4));
  } else {
    const uint32_t a = __builtin_bit_cast(uint32_t, v2bf16{(__bf16)o0, (__bf16)o1});
    const uint32_t b = __builtin_bit_cast(uint32_t, v2bf16{(__bf16)o2, (__bf16)o3});
    __builtin_nontemporal_store(u32x2{a, b}, (u32x2*)((uint16_t*)y + i4));
  }
}

// The stream of one per-tensor quantization.  FAST selects, once for the
// whole tensor, the corrected-reciprocal division (scale in [2^-80, 2^80])
// or IEEE division for every element; a vector holding a NaN is re-encoded
// element by element either way.  Returns the lane's max |x| bit pattern.
// ODT >= 0 also writes the dequantized codes to y (fp32 or bf16).
template <int DT, int FMT, bool FAST, int ODT>
__device__ __forceinline__ uint32_t tensor_stream(const u32x4* __restrict__ xv, int64_t nvec, float s,
                                                  float r, uint8_t* __restrict__ q, void* __restrict__ y) {
  constexpr int kU = FP8Q_KU_T, TH = FP8Q_TH_T;
  constexpr int64_t kChunk = (int64_t)kU * TH;
  uint32_t m = 0;
  for (int64_t c = blockIdx.x; c * kChunk < nvec; c += gridDim.x) {
    const int64_t base = c * kChunk + threadIdx.x;
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (base + u * TH < nvec) v[u] = __builtin_nontemporal_load(xv + base + u * TH);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = base + u * TH;
      if (i >= nvec) break;
      if constexpr (DT == FP8Q_F32) {
        const uint32_t mv = vec_absmax<DT>(0u, v[u]);
        m = max(m, mv);
        const float a = __uint_as_float(v[u].x), b = __uint_as_float(v[u].y);
        const float c4 = __uint_as_float(v[u].z), d = __uint_as_float(v[u].w);
        uint32_t w = FAST ? quant4_fast<FMT>(a, b, c4, d, s, r) : quant4_exact<FMT>(a, b, c4, d, s);
        if (mv > 0x7F800000u) w = quant4_exact<FMT>(a, b, c4, d, s);
        __builtin_nontemporal_store(w, (uint32_t*)q + i);
        if constexpr (ODT >= 0) store_dq4<FMT, ODT>(w, s, y, 4 * i);
      } else {
        const uint32_t mv = pk_fold(vec_absmax<DT>(0u, v[u]));
        m = max(m, mv);
        const float e0 = bf_lo(v[u].x), e1 = bf_hi(v[u].x), e2 = bf_lo(v[u].y), e3 = bf_hi(v[u].y);
        const float e4 = bf_lo(v[u].z), e5 = bf_hi(v[u].z), e6 = bf_lo(v[u].w), e7 = bf_hi(v[u].w);
        u32x2 w;
        w.x = FAST ? quant4_fast<FMT>(e0, e1, e2, e3, s, r) : quant4_exact<FMT>(e0, e1, e2, e3, s);
        w.y = FAST ? quant4_fast<FMT>(e4, e5, e6, e7, s, r) : quant4_exact<FMT>(e4, e5, e6, e7, s);
        if (mv > 0x7F800000u) {
          w.x = quant4_exact<FMT>(e0, e1, e2, e3, s);
          w.y = quant4_exact<FMT>(e4, e5, e6, e7, s);
        }
        __builtin_nontemporal_store(w, (u32x2*)q + i);
        if constexpr (ODT >= 0) {
          store_dq4<FMT, ODT>(w.x, s, y, 8 * i);
          store_dq4<FMT, ODT>(w.y, s, y, 8 * i + 4);
        }
      }
    }
  }
  return m;
}

template <int DT, int FMT, int ODT>
__global__ __launch_bounds__(FP8Q_TH_T) void k_quant_tensor(const void* __restrict__ x, int64_t n,
                                                           const float* __restrict__ scale,
                                                           uint8_t* __restrict__ q,
                                                           uint32_t* __restrict__ amax_acc,
                                                           void* __restrict__ y) {
  const float s = *scale;
  const float r = 1.0f / s;
  const int64_t per_vec = DT == FP8Q_F32 ? 4 : 8;
  const int64_t nvec = n / per_vec;
  const u32x4* xv = (const u32x4*)x;
  uint32_t m = scale_ok(s) ? tensor_stream<DT, FMT, true, ODT>(xv, nvec, s, r, q, y)
                           : tensor_stream<DT, FMT, false, ODT>(xv, nvec, s, r, q, y);
  if (blockIdx.x == 0) {
    for (int64_t j = nvec * per_vec + threadIdx.x; j < n; j += FP8Q_TH_T) {
      uint32_t b = DT == FP8Q_F32 ? ((const uint32_t*)x)[j]
                                  : (uint32_t)((const uint16_t*)x)[j] << 16;
      m = max(m, b & 0x7FFFFFFFu);
      const uint32_t c = enc1<FMT>(__uint_as_float(b) / s);
      q[j] = (uint8_t)c;
      if constexpr (ODT >= 0) {
        const float o = canon_nan(dec2<FMT>(c, false).x * s);
        if constexpr (ODT == FP8Q_F32)
          ((float*)y)[j] = o;
        else
          ((uint16_t*)y)[j] = __builtin_bit_cast(uint16_t, (__bf16)o);
      }
    }
  }
  if (amax_acc) {
    m = block_max<FP8Q_TH_T>(m);
    if (threadIdx.x == 0) fold_max(amax_acc, canon_abs_bits(m));
  }
}

// ---------------------------------------------------------------- 1x128
// fp32 inputs (bf16 ones take k_quant_1x128_b8 below): each 16-lane DPP row
// of a wavefront owns one 128-element block, two 16-byte loads per lane
// (element offsets 4l and 64+4l).  A wavefront takes kGroups groups of four
// consecutive blocks, all loads in flight at once; a workgroup's four
// wavefronts cover consecutive stretches, so each workgroup streams one
// contiguous chunk of the (row, block) sequence at a time.
#ifndef FP8Q_KGROUPS
#define FP8Q_KGROUPS 2
#endif
static constexpr int kGroups = FP8Q_KGROUPS;

template <int DT, int FMT>
__device__ __forceinline__ void quant_block_regs(const u32x4* v, uint32_t amax_bits, float eps,
                                                 uint8_t* qrow, float* sptr, int l) {
  // v[0] (and v[1] for fp32) hold this lane's 8 elements of the block.
  const float amax = __uint_as_float(canon_abs_bits(amax_bits));
  const float s = block_scale<FMT>(amax, eps);
  if (l == 0) *sptr = s;
  if (scale_ok(s)) {
    const float r = 1.0f / s;
    if constexpr (DT == FP8Q_F32) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w = pack4<FMT>(sat<FMT>(div_rn(__uint_as_float(v[h].x), s, r)),
                                sat<FMT>(div_rn(__uint_as_float(v[h].y), s, r)),
                                sat<FMT>(div_rn(__uint_as_float(v[h].z), s, r)),
                                sat<FMT>(div_rn(__uint_as_float(v[h].w), s, r)));
        __builtin_nontemporal_store(w, (uint32_t*)(qrow + 4 * l + 64 * h));
      }
    } else {
      u32x2 w;
      w.x = pack4<FMT>(sat<FMT>(div_rn(bf_lo(v[0].x), s, r)), sat<FMT>(div_rn(bf_hi(v[0].x), s, r)),
                       sat<FMT>(div_rn(bf_lo(v[0].y), s, r)), sat<FMT>(div_rn(bf_hi(v[0].y), s, r)));
      w.y = pack4<FMT>(sat<FMT>(div_rn(bf_lo(v[0].z), s, r)), sat<FMT>(div_rn(bf_hi(v[0].z), s, r)),
                       sat<FMT>(div_rn(bf_lo(v[0].w), s, r)), sat<FMT>(div_rn(bf_hi(v[0].w), s, r)));
      __builtin_nontemporal_store(w, (u32x2*)(qrow + 8 * l));
    }
  } else {
    if constexpr (DT == FP8Q_F32) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w = quant4_exact<FMT>(__uint_as_float(v[h].x), __uint_as_float(v[h].y),
                                       __uint_as_float(v[h].z), __uint_as_float(v[h].w), s);
        *(uint32_t*)(qrow + 4 * l + 64 * h) = w;
      }
    } else {
      u32x2 w;
      w.x = quant4_exact<FMT>(bf_lo(v[0].x), bf_hi(v[0].x), bf_lo(v[0].y), bf_hi(v[0].y), s);
      w.y = quant4_exact<FMT>(bf_lo(v[0].z), bf_hi(v[0].z), bf_lo(v[0].w), bf_hi(v[0].w), s);
      *(u32x2*)(qrow + 8 * l) = w;
    }
  }
}

template <int DT>
__device__ __forceinline__ uint32_t lane_absmax(const u32x4* v) {
  if constexpr (DT == FP8Q_F32) {
    uint32_t m = max(max(v[0].x & 0x7FFFFFFFu, v[0].y & 0x7FFFFFFFu),
                     max(v[0].z & 0x7FFFFFFFu, v[0].w & 0x7FFFFFFFu));
    uint32_t m2 = max(max(v[1].x & 0x7FFFFFFFu, v[1].y & 0x7FFFFFFFu),
                      max(v[1].z & 0x7FFFFFFFu, v[1].w & 0x7FFFFFFFu));
    return max(m, m2);
  } else {
    uint32_t pm = pk_absmax(pk_absmax(0u, v[0].x), v[0].y);
    pm = pk_absmax(pk_absmax(pm, v[0].z), v[0].w);
    return pk_fold(pm);
  }
}

template <int DT, int FMT>
__global__ __launch_bounds__(kThreads) void k_quant_1x128(const void* __restrict__ x, int64_t nkb,
                                                          int64_t nblocks, int64_t ldx, float eps,
                                                          uint8_t* __restrict__ q, int64_t ldq,
                                                          float* __restrict__ scales, int64_t ld_s) {
  constexpr int esz = DT == FP8Q_F32 ? 4 : 2;
  constexpr int NV = DT == FP8Q_F32 ? 2 : 1;  // 16-byte vectors per lane per block
  constexpr int64_t kWaveBlocks = 4 * kGroups;               // consecutive blocks per wavefront
  constexpr int64_t kBlocks = kWaveBlocks * (kThreads / 64);  // per workgroup chunk
  const int lane = threadIdx.x & 63;
  const int rr = lane >> 4, l = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* xb = (const char*)x;
  for (int64_t c = blockIdx.x; c * kBlocks < nblocks; c += gridDim.x) {
    // (row, column block) of the wavefront's first block, then stepped by 4
    const int64_t b0 = c * kBlocks + wave * kWaveBlocks;  // wave-uniform
    int64_t rg = b0 / nkb, kg = b0 - rg * nkb;
    u32x4 v[kGroups][NV];
    int64_t row[kGroups], kb[kGroups];
    bool ok[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if (g > 0) {
        kg += 4;
        while (kg >= nkb) { kg -= nkb; ++rg; }
      }
      int64_t r0 = rg, k0 = kg + rr;
      while (k0 >= nkb) { k0 -= nkb; ++r0; }
      row[g] = r0;
      kb[g] = k0;
      ok[g] = b0 + 4 * g + rr < nblocks;
      if (ok[g]) {
        const u32x4* p = (const u32x4*)(xb + (r0 * ldx + 128 * k0) * esz);
#pragma unroll
        for (int h = 0; h < NV; ++h) v[g][h] = __builtin_nontemporal_load(p + l + 16 * h);
      } else {
#pragma unroll
        for (int h = 0; h < NV; ++h) v[g][h] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const uint32_t am = row16_max(lane_absmax<DT>(v[g]));
      if (ok[g])
        quant_block_regs<DT, FMT>(v[g], am, eps, q + row[g] * ldq + 128 * kb[g],
                                  scales + row[g] * ld_s + kb[g], l);
    }
  }
}

// bf16 inputs: eight lanes per block.  Lane l of a block holds its elements
// 16l .. 16l+16 (two 16-byte loads), the block maximum is reduced over the
// eight lanes, and the lane's 16 codes leave in one 16-byte store; the
// per-block scale arithmetic is then shared by 16 elements per lane instead
// of 8 (64.7 -> 60.4-60.9 us on the 16384x7168 activation against the
// sixteen-lane form, bit-identical).  A wavefront takes FP8Q_KG8 groups of
// eight consecutive blocks per chunk; FP8Q_G_B8 workgroups per CU.
#ifndef FP8Q_G_B8
#define FP8Q_G_B8 128
#endif
#ifndef FP8Q_KG8
#define FP8Q_KG8 1
#endif
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_quant_1x128_b8(const void* __restrict__ x, int64_t nkb,
                                                             int64_t nblocks, int64_t ldx, float eps,
                                                             uint8_t* __restrict__ q, int64_t ldq,
                                                             float* __restrict__ scales, int64_t ld_s) {
  constexpr int G = FP8Q_KG8;
  constexpr int64_t kWaveBlocks = 8 * G;
  constexpr int64_t kBlocks = kWaveBlocks * (kThreads / 64);
  const int lane = threadIdx.x & 63;
  const int rr = lane >> 3, l = lane & 7;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const char* xb = (const char*)x;
  for (int64_t c = blockIdx.x; c * kBlocks < nblocks; c += gridDim.x) {
    const int64_t b0 = c * kBlocks + wave * kWaveBlocks;
    int64_t rg = b0 / nkb, kg = b0 - rg * nkb;
    u32x4 v[G][2];
    int64_t row[G], kb[G];
    bool ok[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g > 0) {
        kg += 8;
        while (kg >= nkb) { kg -= nkb; ++rg; }
      }
      int64_t r0 = rg, k0 = kg + rr;
      while (k0 >= nkb) { k0 -= nkb; ++r0; }
      row[g] = r0;
      kb[g] = k0;
      ok[g] = b0 + 8 * g + rr < nblocks;
      if (ok[g]) {
        const u32x4* p = (const u32x4*)(xb + (r0 * ldx + 128 * k0) * 2);
        v[g][0] = __builtin_nontemporal_load(p + 2 * l);
        v[g][1] = __builtin_nontemporal_load(p + 2 * l + 1);
      } else {
        v[g][0] = v[g][1] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t pm = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        pm = pk_absmax(pk_absmax(pm, v[g][h].x), v[g][h].y);
        pm = pk_absmax(pk_absmax(pm, v[g][h].z), v[g][h].w);
      }
      uint32_t m = pk_fold(pm);
      m = max(m, (uint32_t)__shfl_xor((int)m, 1));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2));
      m = max(m, (uint32_t)__shfl_xor((int)m, 4));
      if (!ok[g]) continue;
      const float s = block_scale<FMT>(__uint_as_float(canon_abs_bits(m)), eps);
      if (l == 0) scales[row[g] * ld_s + kb[g]] = s;
      uint32_t w[4];
      if (scale_ok(s)) {
        const float r = 1.0f / s;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 t = v[g][h];
          w[2 * h] = pack4<FMT>(sat<FMT>(div_rn(bf_lo(t.x), s, r)), sat<FMT>(div_rn(bf_hi(t.x), s, r)),
                                sat<FMT>(div_rn(bf_lo(t.y), s, r)), sat<FMT>(div_rn(bf_hi(t.y), s, r)));
          w[2 * h + 1] = pack4<FMT>(sat<FMT>(div_rn(bf_lo(t.z), s, r)), sat<FMT>(div_rn(bf_hi(t.z), s, r)),
                                    sat<FMT>(div_rn(bf_lo(t.w), s, r)), sat<FMT>(div_rn(bf_hi(t.w), s, r)));
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 t = v[g][h];
          w[2 * h] = quant4_exact<FMT>(bf_lo(t.x), bf_hi(t.x), bf_lo(t.y), bf_hi(t.y), s);
          w[2 * h + 1] = quant4_exact<FMT>(bf_lo(t.z), bf_hi(t.z), bf_lo(t.w), bf_hi(t.w), s);
        }
      }
      __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, (u32x4*)(q + row[g] * ldq + 128 * kb[g] + 16 * l));
    }
  }
}

// ---------------------------------------------------------------- 1x128 of the transpose
// x [rows, cols] -> the codes of x^T [cols, rows], one scale per 128 rows of
// a column of x (a 1x128 block of x^T: the layout the weight-gradient GEMM
// takes for operands reduced over tokens).  A workgroup of 4W threads takes
// a W-column slab of x (W = 128 when the column count allows, else 64) and
// walks FP8Q_RT consecutive 128-row blocks of it, loading the next block
// while it encodes the current one; each load instruction reads 256-byte
// (bf16, W = 128) pieces of four rows.  Each 128xW tile is staged in LDS in
// its input type, swizzled so that the row-wise staging writes and the
// column-wise reads are free of bank conflicts.  bf16: eight lanes hold a
// pair of columns' 128 values (one dword per row), reduce both amaxes with
// packed 16-bit maxima and three shuffles, and write each column's 128
// codes as one contiguous run of the transposed output; fp32: the four
// lanes of a quad do the same for one column.
#ifndef FP8Q_RT
#define FP8Q_RT 8  // row blocks per workgroup in the transposed quantizer (measured)
#endif
template <int DT, int FMT, int W>
__global__ __launch_bounds__(4 * W) void k_quant_1x128_t(const void* __restrict__ x, int64_t ntc,
                                                            int64_t nrb, int64_t ldx, float eps,
                                                            uint8_t* __restrict__ q, int64_t ldq,
                                                            float* __restrict__ scales, int64_t ld_s) {
  // bf16 stays bf16 in LDS (32 KB per workgroup at W = 128)
  __shared__ __attribute__((aligned(16))) uint32_t tile_raw[DT == FP8Q_F32 ? 128 * W : 128 * W / 2];
  constexpr int TH = 4 * W;
  float* tile = (float*)tile_raw;
  uint16_t* tile16 = (uint16_t*)tile_raw;
  constexpr int esz = DT == FP8Q_F32 ? 4 : 2;
  constexpr int VE = 16 / esz;                 // elements per 16-byte vector
  constexpr int VPR = W / VE;                  // vectors per tile row
  constexpr int NVT = 128 * VPR / TH;          // vectors per thread
  // workgroup -> (group of FP8Q_RT row blocks, W-column slab)
  const int64_t cb = blockIdx.x % ntc, rg = blockIdx.x / ntc;
  const int64_t c0 = cb * W;
  const int64_t rb_begin = rg * FP8Q_RT;
  const int64_t rb_end = rb_begin + FP8Q_RT < nrb ? rb_begin + FP8Q_RT : nrb;
  const int tid = threadIdx.x;
  const char* xb = (const char*)x;
  auto load = [&](int64_t rb, u32x4* v) {
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
      const int vi = tid + i * TH, t = vi / VPR, c = (vi % VPR) * VE;
      v[i] = __builtin_nontemporal_load((const u32x4*)(xb + ((rb * 128 + t) * ldx + c0 + c) * esz));
    }
  };
  // fp32: thread (f, k) takes column f, rows 16k .. 16k+16 and 64+16k ..
  // 64+16k+16, so that each of its two 16-byte code stores lands next to
  // those of the other three lanes of the quad (64 contiguous bytes per
  // store).  bf16: thread (p, k) takes the column pair p (columns 2p, 2p+1,
  // one dword of the tile row) over rows 16k .. 16k+16, so one 4-byte LDS
  // read brings two columns and their amax is one packed 16-bit max; the
  // eight lanes k = 0..7 of a pair write 128 contiguous code bytes per
  // column.  Staging swizzles: fp32 XORs the column by 16*((t/16) mod 4),
  // bf16 XORs the column pair by 8*((t/16) mod W/16); both keep the row-wise
  // 16-byte writes whole and the column-wise reads free of bank conflicts.
  auto swz = [](int t) { return DT == FP8Q_F32 ? 16 * ((t >> 4) & 3) : 16 * ((t >> 4) & (W / 16 - 1)); };
  // One row block: stage the tile, reduce each column's amax, encode, store.
  auto block = [&](int64_t rb, const u32x4* v) {
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
      const int vi = tid + i * TH, t = vi / VPR, c = (vi % VPR) * VE;
      if constexpr (DT == FP8Q_F32)
        *(u32x4*)(tile + t * W + (c ^ swz(t))) = v[i];
      else
        *(u32x4*)(tile16 + t * W + (c ^ swz(t))) = v[i];
    }
    __syncthreads();
    if constexpr (DT == FP8Q_F32) {
      const int f = tid >> 2, k = tid & 3;
      const int fc = f ^ (16 * k);
      const int64_t col = c0 + f;
      float a[32];
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int t = 16 * k + (j & 15) + 64 * (j >> 4);  // swz(t) == 16k
        a[j] = tile[t * W + fc];
        m = max(m, __float_as_uint(a[j]) & 0x7FFFFFFFu);
      }
      __syncthreads();  // the tile is rewritten by the next row block
      m = max(m, (uint32_t)__shfl_xor((int)m, 1));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2));
      const float s = block_scale<FMT>(__uint_as_float(canon_abs_bits(m)), eps);
      if (k == 0) scales[col * ld_s + rb] = s;
      uint32_t w[8];
      if (scale_ok(s)) {
        // |x| <= amax, so x/s stays within the finite range
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          w[i] = pack4<FMT>(sat<FMT>(div_rn(a[4 * i], s, r)), sat<FMT>(div_rn(a[4 * i + 1], s, r)),
                            sat<FMT>(div_rn(a[4 * i + 2], s, r)), sat<FMT>(div_rn(a[4 * i + 3], s, r)));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = quant4_exact<FMT>(a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3], s);
      }
      uint8_t* qrow = q + col * ldq + rb * 128 + 16 * k;
      __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, (u32x4*)qrow);
      __builtin_nontemporal_store(u32x4{w[4], w[5], w[6], w[7]}, (u32x4*)(qrow + 64));
    } else {
      const int p = tid >> 3, k = tid & 7;
      const int pc = p ^ (8 * (k & (W / 16 - 1)));  // the pair's slot in rows 16k .. 16k+16
      const uint32_t* trow = tile_raw + (16 * k) * (W / 2) + pc;
      uint32_t d[16];
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        d[j] = trow[j * (W / 2)];
        m = pk_absmax(m, d[j]);
      }
      __syncthreads();  // the tile is rewritten by the next row block
      // amax of each column over the eight lanes of the pair
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        const uint32_t mo = (uint32_t)__shfl_xor((int)m, o);
        m = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m),
                                                                   __builtin_bit_cast(u16x2, mo)));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t col = c0 + 2 * p + h;
        const uint32_t mb = h ? (m & 0xFFFF0000u) : (m << 16);
        const float s = block_scale<FMT>(__uint_as_float(canon_abs_bits(mb)), eps);
        if (k == 0) scales[col * ld_s + rb] = s;
        auto val = [&](int j) { return h ? bf_hi(d[j]) : bf_lo(d[j]); };
        uint32_t w[4];
        if (scale_ok(s)) {
          const float r = 1.0f / s;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = pack4<FMT>(sat<FMT>(div_rn(val(4 * i), s, r)), sat<FMT>(div_rn(val(4 * i + 1), s, r)),
                              sat<FMT>(div_rn(val(4 * i + 2), s, r)), sat<FMT>(div_rn(val(4 * i + 3), s, r)));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = quant4_exact<FMT>(val(4 * i), val(4 * i + 1), val(4 * i + 2), val(4 * i + 3), s);
        }
        __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, (u32x4*)(q + col * ldq + rb * 128 + 16 * k));
      }
    }
  };
  // The next block's loads are issued unconditionally before the current
  // block is used (the last block is peeled off), so the wait before the
  // tile is staged leaves them in flight: issued under a condition, the
  // compiler cannot count them and waits for every load, the prefetch
  // included, which serializes the loads with the block's work.
  u32x4 v[NVT], vn[NVT];
  load(rb_begin, v);
  int64_t rb = rb_begin;
  for (; rb + 1 < rb_end; ++rb) {
    load(rb + 1, vn);
    block(rb, v);
#pragma unroll
    for (int i = 0; i < NVT; ++i) v[i] = vn[i];
  }
  block(rb, v);
}

// ---------------------------------------------------------------- 128x128
// One workgroup per 128x128 tile: the tile is read into registers once
// (bf16: 8 rows x 16 B per thread; fp32: 16 rows x 16 B), its amax found
// by a workgroup reduction, then quantized from the registers.
template <int DT, int FMT>
__global__ __launch_bounds__(kThreads) void k_quant_128x128(const void* __restrict__ x, int64_t nkb,
                                                            int64_t ldx, float eps,
                                                            uint8_t* __restrict__ q, int64_t ldq,
                                                            float* __restrict__ scales,
                                                            int64_t ld_s) {
  constexpr int esz = DT == FP8Q_F32 ? 4 : 2;
  constexpr int LPR = DT == FP8Q_F32 ? 32 : 16;  // lanes per 128-element row
  constexpr int RSTEP = kThreads / LPR;           // rows covered by one pass
  constexpr int NR = 128 / RSTEP;                 // passes
  const int64_t rb = blockIdx.x / nkb, kb = blockIdx.x - rb * nkb;
  const int c = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
  const char* base = (const char*)x + ((rb * 128 + r0) * ldx + kb * 128) * esz;
  u32x4 v[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i)
    v[i] = __builtin_nontemporal_load((const u32x4*)(base + (int64_t)i * RSTEP * ldx * esz) + c);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if constexpr (DT == FP8Q_F32) {
      m = max(m, max(max(v[i].x & 0x7FFFFFFFu, v[i].y & 0x7FFFFFFFu),
                     max(v[i].z & 0x7FFFFFFFu, v[i].w & 0x7FFFFFFFu)));
    } else {
      m = pk_absmax(pk_absmax(m, v[i].x), v[i].y);
      m = pk_absmax(pk_absmax(m, v[i].z), v[i].w);
    }
  }
  if constexpr (DT == FP8Q_BF16) m = pk_fold(m);
  m = block_max(m);
  const float s = block_scale<FMT>(__uint_as_float(canon_abs_bits(m)), eps);
  if (threadIdx.x == 0) scales[rb * ld_s + kb] = s;
  uint8_t* qb = q + (rb * 128 + r0) * ldq + kb * 128;
  const bool fast = scale_ok(s);
  const float r = 1.0f / s;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    uint8_t* qr = qb + (int64_t)i * RSTEP * ldq;
    if constexpr (DT == FP8Q_F32) {
      float a = __uint_as_float(v[i].x), b = __uint_as_float(v[i].y);
      float cc = __uint_as_float(v[i].z), d = __uint_as_float(v[i].w);
      uint32_t w = fast ? pack4<FMT>(sat<FMT>(div_rn(a, s, r)), sat<FMT>(div_rn(b, s, r)),
                                     sat<FMT>(div_rn(cc, s, r)), sat<FMT>(div_rn(d, s, r)))
                        : quant4_exact<FMT>(a, b, cc, d, s);
      __builtin_nontemporal_store(w, (uint32_t*)(qr + 4 * c));
    } else {
      float e[8] = {bf_lo(v[i].x), bf_hi(v[i].x), bf_lo(v[i].y), bf_hi(v[i].y),
                    bf_lo(v[i].z), bf_hi(v[i].z), bf_lo(v[i].w), bf_hi(v[i].w)};
      u32x2 w;
      if (fast) {
        w.x = pack4<FMT>(sat<FMT>(div_rn(e[0], s, r)), sat<FMT>(div_rn(e[1], s, r)),
                         sat<FMT>(div_rn(e[2], s, r)), sat<FMT>(div_rn(e[3], s, r)));
        w.y = pack4<FMT>(sat<FMT>(div_rn(e[4], s, r)), sat<FMT>(div_rn(e[5], s, r)),
                         sat<FMT>(div_rn(e[6], s, r)), sat<FMT>(div_rn(e[7], s, r)));
      } else {
        w.x = quant4_exact<FMT>(e[0], e[1], e[2], e[3], s);
        w.y = quant4_exact<FMT>(e[4], e[5], e[6], e[7], s);
      }
      __builtin_nontemporal_store(w, (u32x2*)(qr + 8 * c));
    }
  }
}

// ---------------------------------------------------------------- scaler
__global__ void k_scaler_init(fp8q_scaler* st, int32_t window, float max_val, float eps,
                              float margin, int32_t stat, float alpha) {
  for (int i = threadIdx.x; i < 1024; i += blockDim.x) st->ring[i] = 0.0f;
  if (threadIdx.x == 0) {
    st->window = window;
    st->count = 0;
    st->pos = 0;
    st->max_val = max_val;
    st->eps = eps;
    st->margin = margin;
    st->scale = 1.0f;
    st->stat = stat;
    st->alpha = alpha;
    st->amax_acc = 0.0f;
    st->ema = 0.0;
  }
}

// One wavefront: push the amax, then (window full) the window maximum with
// NaN winning, then the scale.  The PyTorch-native FP8 article, section
// 4.2: the amax of earlier steps sets the scale of the next one, and the
// scale is only recomputed once the window holds `window` values.
// Contribution of one history entry to the window maximum: NaN wins,
// values <= 0 contribute nothing (the maximum starts from 0).
__device__ __forceinline__ uint32_t hist_bits(float f) {
  if (f != f) return 0x7FC00000u;
  return f > 0.0f ? __float_as_uint(f) : 0u;
}

// Window mean: lane l holds slots 16l .. 16l+15 (the new value in slot
// pos, zeros past the window), sums them pairwise, and the butterfly over
// lanes continues the same binary tree up to all 1024 slots (fp64 addition
// is commutative, so both lanes of a pair form the same sum).
__device__ double window_mean(const fp8q_scaler* st, int lane, int32_t window, int32_t pos, float a) {
  double v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = 16 * lane + k;
    v[k] = i < window ? (double)(i == pos ? a : st->ring[i]) : 0.0;
  }
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int k = 0; k < w; ++k) v[k] = __dadd_rn(v[2 * k], v[2 * k + 1]);
  double s = v[0];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s = __dadd_rn(s, __shfl_xor(s, o));
  return s / (double)window;
}

__global__ __launch_bounds__(64) void k_scaler_update(fp8q_scaler* st, uint32_t* amax) {
  const int lane = threadIdx.x;
  float a = __uint_as_float(*amax);
  if (a != a) a = __uint_as_float(0x7FC00000u);
  const int32_t window = st->window, pos = st->pos, stat = st->stat;
  int32_t count = st->count;
  double ema = st->ema;
  __syncthreads();
  if (stat == FP8Q_STAT_EMA) {
    // e = alpha*a + (1-alpha)*e, two rounded products and a rounded sum
    const double al = (double)st->alpha;
    ema = count == 0 ? (double)a : __dadd_rn(__dmul_rn(al, (double)a), __dmul_rn(1.0 - al, ema));
  }
  if (lane == 0) {
    *amax = 0u;  // consumed: ready to accumulate the next step
    st->ring[pos] = a;
    st->pos = pos + 1 == window ? 0 : pos + 1;
    st->count = count < window ? count + 1 : count;
    if (stat == FP8Q_STAT_EMA) st->ema = ema;
  }
  count = count < window ? count + 1 : count;
  __syncthreads();
  if (count >= window) {
    float stat_v;
    if (stat == FP8Q_STAT_MEAN) {
      stat_v = (float)window_mean(st, lane, window, pos, a);
    } else if (stat == FP8Q_STAT_EMA) {
      stat_v = (float)ema;
    } else {
      uint32_t m = 0;
      for (int i = lane; i < window; i += 64) m = max(m, hist_bits(i == pos ? a : st->ring[i]));
      stat_v = __uint_as_float(wave_max(m));
    }
    if (lane == 0) {
      if (stat_v != stat_v) stat_v = __uint_as_float(0x7FC00000u);
      const float mm = (stat_v < st->eps) ? st->eps : stat_v;  // NaN stays NaN
      const float t = mm * st->margin;
      st->scale = t / st->max_val;
    }
  }
}

// ---------------------------------------------------------------- dequantize

// Work unit: (row, chunk of kThreads*8*FP8Q_KU_D columns); each thread
// handles FP8Q_KU_D groups of 8 codes, lane l at codes 8l .. 8l+8 of the
// group, so every load and store instruction of a wavefront covers one
// contiguous run (512 bytes of codes, 1 KB of bf16).  V16: rows keep
// 16-byte alignment (8-byte code loads, 16-byte bf16 stores); otherwise
// dword loads and 8-byte stores.  Each workgroup walks a contiguous range
// of units.  y = fl32(dec(q) * s), NaN made 0x7FC00000; bf16 output rounds
// that to nearest even (the hardware conversion, which keeps subnormals and
// maps the quiet NaN to 0x7FC0).
template <int FMT, int GRAN, int ODT, bool V16>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* __restrict__ q, int64_t rows,
                                                      int64_t cols, int64_t ldq,
                                                      const float* __restrict__ scales,
                                                      int64_t ld_s, void* __restrict__ y,
                                                      int64_t ldy, int64_t per_wg) {
  constexpr int64_t CW = kThreads * 8;
  constexpr int64_t UW = CW * FP8Q_KU_D;
  const int64_t nchunk = (cols + UW - 1) / UW;
  const int64_t units = rows * nchunk;
  int64_t u = (int64_t)blockIdx.x * per_wg;
  const int64_t uend = u + per_wg < units ? u + per_wg : units;
  for (; u < uend; ++u) {
    const int64_t r = u / nchunk, ch = u - r * nchunk;
#pragma unroll
    for (int g = 0; g < FP8Q_KU_D; ++g) {
      const int64_t c = ch * UW + g * CW + 8 * threadIdx.x;
      if (c >= cols) break;
      float s;
      if constexpr (GRAN == FP8Q_GRAN_TENSOR) s = scales[0];
      else if constexpr (GRAN == FP8Q_GRAN_1x128) s = scales[r * ld_s + (c >> 7)];
      else s = scales[(r >> 7) * ld_s + (c >> 7)];
      const uint8_t* qp = q + r * ldq + c;
      if (c + 8 <= cols) {
        u32x2 w;
        if constexpr (V16) {
          w = __builtin_nontemporal_load((const u32x2*)qp);
        } else {
          w.x = __builtin_nontemporal_load((const uint32_t*)qp);
          w.y = __builtin_nontemporal_load((const uint32_t*)qp + 1);
        }
        float o[8];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float2 lo = dec2<FMT>(w[k], false), hi = dec2<FMT>(w[k], true);
          o[4 * k] = canon_nan(lo.x * s);
          o[4 * k + 1] = canon_nan(lo.y * s);
          o[4 * k + 2] = canon_nan(hi.x * s);
          o[4 * k + 3] = canon_nan(hi.y * s);
        }
        if constexpr (ODT == FP8Q_F32) {
          float* yp = (float*)y + r * ldy + c;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const u32x4 v = {__float_as_uint(o[4 * k]), __float_as_uint(o[4 * k + 1]), __float_as_uint(o[4 * k + 2]),
                             __float_as_uint(o[4 * k + 3])};
            __builtin_nontemporal_store(v, (u32x4*)yp + k);
          }
        } else {
          uint32_t b[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) b[k] = __builtin_bit_cast(uint32_t, v2bf16{(__bf16)o[2 * k], (__bf16)o[2 * k + 1]});
          uint16_t* yp = (uint16_t*)y + r * ldy + c;
          if constexpr (V16) {
            __builtin_nontemporal_store(u32x4{b[0], b[1], b[2], b[3]}, (u32x4*)yp);
          } else {
            __builtin_nontemporal_store(u32x2{b[0], b[1]}, (u32x2*)yp);
            __builtin_nontemporal_store(u32x2{b[2], b[3]}, (u32x2*)yp + 1);
          }
        }
      } else {
        for (int64_t j = c; j < cols; ++j) {
          const float o = canon_nan(dec2<FMT>(q[r * ldq + j], false).x * s);
          if constexpr (ODT == FP8Q_F32) ((float*)y)[r * ldy + j] = o;
          else ((uint16_t*)y)[r * ldy + j] = __builtin_bit_cast(uint16_t, (__bf16)o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- MX (microscaling) FP8
// Blocks of 32 consecutive elements of a row share X = 2^e, e =
// floor(log2 max|x|) - emax (emax 8 for E4M3, 15 for E5M2; clamped to
// [-127, 127]), stored as the E8M0 byte e + 127; a block holding a NaN or an
// Inf gets the NaN scale 0xFF and NaN codes; an all-zero block e = -127.
// Codes are enc(x * 2^-e), a multiplication by a normal power of two, exact
// wherever the code can be nonzero.  A lane's 16-byte vector holds 8 bf16
// or 4 fp32; the lanes of a block are consecutive (4 or 8) and reduce the
// block maximum with xor shuffles.  Each workgroup walks a contiguous chunk
// of vectors.
template <int FMT>
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
  constexpr int kEmax = FMT == FP8Q_E4M3FN ? 8 : 15;
  if (amax_bits == 0) return -127;
  const int E = (int)(amax_bits >> 23);
  const int fl = E > 0 ? E - 127 : (31 - __builtin_clz(amax_bits)) - 149;  // floor(log2 amax)
  const int e = fl - kEmax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

template <int DT, int FMT>
__global__ __launch_bounds__(kThreads) void k_quant_mx(const void* __restrict__ x, int64_t vpr, int64_t nvec,
                                                       int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                       uint8_t* __restrict__ scales, int64_t ld_s,
                                                       int64_t per_wg) {
  constexpr int VE = DT == FP8Q_F32 ? 4 : 8;   // elements per 16-byte vector
  constexpr int LPB = 32 / VE;                 // lanes per block
  constexpr int esz = DT == FP8Q_F32 ? 4 : 2;
  const char* xb = (const char*)x;
  const int64_t v0 = (int64_t)blockIdx.x * per_wg;
  const int64_t v1 = v0 + per_wg < nvec ? v0 + per_wg : nvec;
  // Each lane takes FP8Q_KU_MX vectors per pass (all loads first, kThreads
  // vectors apart).  Vectors are counted along rows and blocks never
  // straddle a row (cols % 32 == 0); per_wg is a multiple of kThreads and a
  // row a multiple of the block's lane count, so a block's lanes are always
  // active together.  The lane's (row, column) is divided out once and then
  // stepped.
  constexpr int U = FP8Q_KU_MX;
  const int64_t cols = vpr * VE;
  int64_t rn = (v0 + threadIdx.x) / vpr, cn = (v0 + threadIdx.x - rn * vpr) * VE;
  for (int64_t base = v0; base < v1; base += (int64_t)U * kThreads) {
    u32x4 w[U];
    bool on[U];
    int64_t r[U], c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      on[u] = base + u * kThreads + threadIdx.x < v1;
      r[u] = rn;
      c[u] = cn;
      cn += kThreads * VE;
      while (cn >= cols) {
        cn -= cols;
        ++rn;
      }
      w[u] = on[u] ? __builtin_nontemporal_load((const u32x4*)(xb + (r[u] * ldx + c[u]) * esz)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t m;
      if constexpr (DT == FP8Q_F32)
        m = max(max(w[u].x & 0x7FFFFFFFu, w[u].y & 0x7FFFFFFFu), max(w[u].z & 0x7FFFFFFFu, w[u].w & 0x7FFFFFFFu));
      else
        m = pk_fold(pk_absmax(pk_absmax(pk_absmax(pk_absmax(0u, w[u].x), w[u].y), w[u].z), w[u].w));
#pragma unroll
      for (int o = 1; o < LPB; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
      if (!on[u]) continue;
      uint8_t* qp = q + r[u] * ldq + c[u];
      const bool special = m >= 0x7F800000u;  // a NaN or an Inf in the block
      if ((threadIdx.x & (LPB - 1)) == 0)
        scales[r[u] * ld_s + (c[u] >> 5)] = special ? 0xFF : (uint8_t)(mx_exponent<FMT>(m) + 127);
      if (special) {
        if constexpr (DT == FP8Q_F32) *(uint32_t*)qp = 0x7F7F7F7Fu;
        else *(u32x2*)qp = u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu};
        continue;
      }
      const float inv = __uint_as_float((uint32_t)(127 - mx_exponent<FMT>(m)) << 23);  // 2^-e, normal
      if constexpr (DT == FP8Q_F32) {
        const uint32_t o = pack4<FMT>(sat<FMT>(__uint_as_float(w[u].x) * inv), sat<FMT>(__uint_as_float(w[u].y) * inv),
                                      sat<FMT>(__uint_as_float(w[u].z) * inv), sat<FMT>(__uint_as_float(w[u].w) * inv));
        __builtin_nontemporal_store(o, (uint32_t*)qp);
      } else {
        u32x2 o;
        o.x = pack4<FMT>(sat<FMT>(bf_lo(w[u].x) * inv), sat<FMT>(bf_hi(w[u].x) * inv), sat<FMT>(bf_lo(w[u].y) * inv),
                         sat<FMT>(bf_hi(w[u].y) * inv));
        o.y = pack4<FMT>(sat<FMT>(bf_lo(w[u].z) * inv), sat<FMT>(bf_hi(w[u].z) * inv), sat<FMT>(bf_lo(w[u].w) * inv),
                         sat<FMT>(bf_hi(w[u].w) * inv));
        __builtin_nontemporal_store(o, (u32x2*)qp);
      }
    }
  }
}

// x^ = fl32(dec(q) * 2^(s - 127)) (NaN scale byte: NaN), as the block
// dequantizer: 8 codes per lane, contiguous runs per instruction.
template <int FMT, int ODT>
__global__ __launch_bounds__(kThreads) void k_dequant_mx(const uint8_t* __restrict__ q, int64_t rows,
                                                         int64_t cols, int64_t ldq,
                                                         const uint8_t* __restrict__ scales, int64_t ld_s,
                                                         void* __restrict__ y, int64_t ldy, int64_t per_wg) {
  const int64_t gpr = cols / 8;  // 8-code groups per row
  const int64_t total = rows * gpr;
  const int64_t g0 = (int64_t)blockIdx.x * per_wg;
  const int64_t g1 = g0 + per_wg < total ? g0 + per_wg : total;
  // the lane's (row, column) divided out once, then stepped
  int64_t r = (g0 + threadIdx.x) / gpr, c = (g0 + threadIdx.x - r * gpr) * 8;
  for (int64_t g = g0 + threadIdx.x; g < g1; g += kThreads) {
    const uint32_t sb = scales[r * ld_s + (c >> 5)];
    const u32x2 w = __builtin_nontemporal_load((const u32x2*)(q + r * ldq + c));
    // 2^(sb-127): normal for sb >= 1, the subnormal 2^-127 for sb == 0
    const float X = sb == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(sb << 23);
    float o[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float2 lo = dec2<FMT>(w[k], false), hi = dec2<FMT>(w[k], true);
      o[4 * k] = canon_nan(lo.x * X);
      o[4 * k + 1] = canon_nan(lo.y * X);
      o[4 * k + 2] = canon_nan(hi.x * X);
      o[4 * k + 3] = canon_nan(hi.y * X);
    }
    if (sb == 0xFF) {
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = __uint_as_float(0x7FC00000u);
    }
    if constexpr (ODT == FP8Q_F32) {
      float* yp = (float*)y + r * ldy + c;
      __builtin_nontemporal_store(
          u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])}, (u32x4*)yp);
      __builtin_nontemporal_store(
          u32x4{__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])},
          (u32x4*)yp + 1);
    } else {
      uint32_t b[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = __builtin_bit_cast(uint32_t, v2bf16{(__bf16)o[2 * k], (__bf16)o[2 * k + 1]});
      __builtin_nontemporal_store(u32x4{b[0], b[1], b[2], b[3]}, (u32x4*)((uint16_t*)y + r * ldy + c));
    }
    c += kThreads * 8;
    while (c >= cols) {
      c -= cols;
      ++r;
    }
  }
}

// ---------------------------------------------------------------- launches
// Persistent grid for chunked streams: up to per_cu workgroups per CU.
static int chunk_grid(int64_t chunks, int per_cu) {
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  const int64_t g = chunks < cap ? chunks : cap;
  return g < 1 ? 1 : (int)g;
}


int launch_amax(const void* x, int dt, int64_t n, float* amax, hipStream_t st) {
  hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, st, (uint32_t*)amax, 0u);
  if (int e = check_launch("amax reset")) return e;
  const int64_t nvec = n / (dt == FP8Q_F32 ? 4 : 8);
  const int64_t ch = (int64_t)FP8Q_KU_A * kThreads;
  const int grid = chunk_grid((nvec + ch - 1) / ch, FP8Q_G_A);
  if (dt == FP8Q_F32)
    hipLaunchKernelGGL(k_amax<FP8Q_F32>, dim3(grid), dim3(kThreads), 0, st, x, n, (uint32_t*)amax);
  else
    hipLaunchKernelGGL(k_amax<FP8Q_BF16>, dim3(grid), dim3(kThreads), 0, st, x, n, (uint32_t*)amax);
  return check_launch("amax");
}

template <int DT, int FMT>
static void launch_qt(int grid, const void* x, int64_t n, const float* scale, uint8_t* q,
                      float* amax_acc, hipStream_t st, void* y = nullptr, int out_dt = -1) {
  if (out_dt == FP8Q_F32)
    hipLaunchKernelGGL((k_quant_tensor<DT, FMT, FP8Q_F32>), dim3(grid), dim3(FP8Q_TH_T), 0, st, x, n, scale, q,
                       (uint32_t*)amax_acc, y);
  else if (out_dt == FP8Q_BF16)
    hipLaunchKernelGGL((k_quant_tensor<DT, FMT, FP8Q_BF16>), dim3(grid), dim3(FP8Q_TH_T), 0, st, x, n, scale, q,
                       (uint32_t*)amax_acc, y);
  else
    hipLaunchKernelGGL((k_quant_tensor<DT, FMT, -1>), dim3(grid), dim3(FP8Q_TH_T), 0, st, x, n, scale, q,
                       (uint32_t*)amax_acc, y);
}

int launch_quantize_tensor(const void* x, int dt, int64_t n, int fmt, const float* scale, uint8_t* q,
                           float* amax, bool reset_amax, hipStream_t st, void* y, int out_dt) {
  // an overwritten amax is reset on the stream first, then every workgroup
  // folds its maximum into it; a running one (a scaler's accumulator) is not
  if (amax && reset_amax) {
    hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, st, (uint32_t*)amax, 0u);
    if (int e = check_launch("quantize_tensor amax reset")) return e;
  }
  const int64_t nvec = n / (dt == FP8Q_F32 ? 4 : 8);
  const int64_t ch = (int64_t)FP8Q_KU_T * FP8Q_TH_T;
  const int grid = chunk_grid((nvec + ch - 1) / ch, y ? FP8Q_G_TDQ : FP8Q_G_T);
  if (dt == FP8Q_F32 && fmt == FP8Q_E4M3FN)
    launch_qt<FP8Q_F32, FP8Q_E4M3FN>(grid, x, n, scale, q, amax, st, y, out_dt);
  else if (dt == FP8Q_F32)
    launch_qt<FP8Q_F32, FP8Q_E5M2>(grid, x, n, scale, q, amax, st, y, out_dt);
  else if (fmt == FP8Q_E4M3FN)
    launch_qt<FP8Q_BF16, FP8Q_E4M3FN>(grid, x, n, scale, q, amax, st, y, out_dt);
  else
    launch_qt<FP8Q_BF16, FP8Q_E5M2>(grid, x, n, scale, q, amax, st, y, out_dt);
  return check_launch(y ? "quantize_tensor_dq" : "quantize_tensor");
}

template <int DT, int FMT>
static void launch_q1(int grid, const void* x, int64_t nkb, int64_t nblocks, int64_t ldx, float eps,
                      uint8_t* q, int64_t ldq, float* scales, int64_t ld_s, hipStream_t st) {
  hipLaunchKernelGGL((k_quant_1x128<DT, FMT>), dim3(grid), dim3(kThreads), 0, st, x, nkb, nblocks, ldx,
                     eps, q, ldq, scales, ld_s);
}

int launch_quantize_1x128(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                          float eps, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                          hipStream_t st) {
  const int64_t nkb = cols / 128, nblocks = rows * nkb;
  // one workgroup handles 4*kGroups blocks per wavefront per chunk
  const int64_t per_chunk = 4 * kGroups * (kThreads / 64);
  const int grid = chunk_grid((nblocks + per_chunk - 1) / per_chunk, FP8Q_G_1);
  if (dt == FP8Q_F32 && fmt == FP8Q_E4M3FN) launch_q1<FP8Q_F32, FP8Q_E4M3FN>(grid, x, nkb, nblocks, ldx, eps, q, ldq, scales, ld_s, st);
  else if (dt == FP8Q_F32) launch_q1<FP8Q_F32, FP8Q_E5M2>(grid, x, nkb, nblocks, ldx, eps, q, ldq, scales, ld_s, st);
  else {
    const int64_t pc8 = 8 * FP8Q_KG8 * (kThreads / 64);
    const int g8 = chunk_grid((nblocks + pc8 - 1) / pc8, FP8Q_G_B8);
    if (fmt == FP8Q_E4M3FN)
      hipLaunchKernelGGL((k_quant_1x128_b8<FP8Q_E4M3FN>), dim3(g8), dim3(kThreads), 0, st, x, nkb, nblocks, ldx, eps,
                         q, ldq, scales, ld_s);
    else
      hipLaunchKernelGGL((k_quant_1x128_b8<FP8Q_E5M2>), dim3(g8), dim3(kThreads), 0, st, x, nkb, nblocks, ldx, eps,
                         q, ldq, scales, ld_s);
  }
  return check_launch("quantize_1x128");
}

template <int DT, int FMT>
static void launch_q1t(int64_t ngr, const void* x, int64_t ntc, int64_t nrb, int64_t ldx, float eps, uint8_t* q,
                       int64_t ldq, float* scales, int64_t ld_s, hipStream_t st) {
  // ntc 64-column slabs; 128-column slabs when they pair up
  if (ntc % 2 == 0)
    hipLaunchKernelGGL((k_quant_1x128_t<DT, FMT, 128>), dim3((unsigned)(ngr * (ntc / 2))), dim3(512), 0, st, x,
                       ntc / 2, nrb, ldx, eps, q, ldq, scales, ld_s);
  else
    hipLaunchKernelGGL((k_quant_1x128_t<DT, FMT, 64>), dim3((unsigned)(ngr * ntc)), dim3(256), 0, st, x, ntc, nrb,
                       ldx, eps, q, ldq, scales, ld_s);
}

int launch_quantize_1x128_t(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                            float eps, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                            hipStream_t st) {
  const int64_t ntc = cols / 64, nrb = rows / 128;
  const int64_t ngr = (nrb + FP8Q_RT - 1) / FP8Q_RT;  // row-block groups
  if (ngr * ntc > 0x7FFFFFFF) return fail(FP8Q_ESHAPE, "quantize_1x128_t: more than 2^31-1 workgroups");
  if (dt == FP8Q_F32 && fmt == FP8Q_E4M3FN) launch_q1t<FP8Q_F32, FP8Q_E4M3FN>(ngr, x, ntc, nrb, ldx, eps, q, ldq, scales, ld_s, st);
  else if (dt == FP8Q_F32) launch_q1t<FP8Q_F32, FP8Q_E5M2>(ngr, x, ntc, nrb, ldx, eps, q, ldq, scales, ld_s, st);
  else if (fmt == FP8Q_E4M3FN) launch_q1t<FP8Q_BF16, FP8Q_E4M3FN>(ngr, x, ntc, nrb, ldx, eps, q, ldq, scales, ld_s, st);
  else launch_q1t<FP8Q_BF16, FP8Q_E5M2>(ngr, x, ntc, nrb, ldx, eps, q, ldq, scales, ld_s, st);
  return check_launch("quantize_1x128_t");
}

template <int DT, int FMT>
static void launch_q128(int64_t tiles, const void* x, int64_t nkb, int64_t ldx, float eps, uint8_t* q,
                        int64_t ldq, float* scales, int64_t ld_s, hipStream_t st) {
  hipLaunchKernelGGL((k_quant_128x128<DT, FMT>), dim3((unsigned)tiles), dim3(kThreads), 0, st, x, nkb,
                     ldx, eps, q, ldq, scales, ld_s);
}

int launch_quantize_128x128(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                            float eps, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                            hipStream_t st) {
  const int64_t nkb = cols / 128, tiles = (rows / 128) * nkb;
  if (tiles > 0x7FFFFFFF) return fail(FP8Q_ESHAPE, "quantize_128x128: more than 2^31-1 tiles");
  if (dt == FP8Q_F32 && fmt == FP8Q_E4M3FN) launch_q128<FP8Q_F32, FP8Q_E4M3FN>(tiles, x, nkb, ldx, eps, q, ldq, scales, ld_s, st);
  else if (dt == FP8Q_F32) launch_q128<FP8Q_F32, FP8Q_E5M2>(tiles, x, nkb, ldx, eps, q, ldq, scales, ld_s, st);
  else if (fmt == FP8Q_E4M3FN) launch_q128<FP8Q_BF16, FP8Q_E4M3FN>(tiles, x, nkb, ldx, eps, q, ldq, scales, ld_s, st);
  else launch_q128<FP8Q_BF16, FP8Q_E5M2>(tiles, x, nkb, ldx, eps, q, ldq, scales, ld_s, st);
  return check_launch("quantize_128x128");
}

int launch_scaler_init(fp8q_scaler* s, int32_t window, float max_val, float eps, float margin, int32_t stat,
                       float alpha, hipStream_t st) {
  hipLaunchKernelGGL(k_scaler_init, dim3(1), dim3(256), 0, st, s, window, max_val, eps, margin, stat, alpha);
  return check_launch("delayed_scaler_init");
}

int launch_scaler_update(fp8q_scaler* s, float* amax, hipStream_t st) {
  hipLaunchKernelGGL(k_scaler_update, dim3(1), dim3(64), 0, st, s, (uint32_t*)amax);
  return check_launch("delayed_scaler_update");
}

template <int FMT, int GRAN, int ODT>
static void launch_dq(const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const float* scales,
                      int64_t ld_s, void* y, int64_t ldy, hipStream_t st) {
  const int64_t uw = (int64_t)kThreads * 8 * FP8Q_KU_D;
  const int64_t units = rows * ((cols + uw - 1) / uw);
  const int grid = chunk_grid(units, FP8Q_G_D);
  const int64_t per_wg = (units + grid - 1) / grid;
  // 16-byte rows: q and y are 16-byte aligned, so every row is when the
  // leading dimensions keep 16 bytes (a single row always does)
  const bool v16 = rows == 1 || (ldq % 16 == 0 && (ldy * (ODT == FP8Q_F32 ? 4 : 2)) % 16 == 0);
  if (v16)
    hipLaunchKernelGGL((k_dequant<FMT, GRAN, ODT, true>), dim3(grid), dim3(kThreads), 0, st, q, rows, cols, ldq,
                       scales, ld_s, y, ldy, per_wg);
  else
    hipLaunchKernelGGL((k_dequant<FMT, GRAN, ODT, false>), dim3(grid), dim3(kThreads), 0, st, q, rows, cols, ldq,
                       scales, ld_s, y, ldy, per_wg);
}

template <int FMT, int GRAN>
static void launch_dq_o(int out_dt, const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq,
                        const float* scales, int64_t ld_s, void* y, int64_t ldy, hipStream_t st) {
  if (out_dt == FP8Q_F32) launch_dq<FMT, GRAN, FP8Q_F32>(q, rows, cols, ldq, scales, ld_s, y, ldy, st);
  else launch_dq<FMT, GRAN, FP8Q_BF16>(q, rows, cols, ldq, scales, ld_s, y, ldy, st);
}

template <int FMT>
static void launch_dq_g(int gran, int out_dt, const uint8_t* q, int64_t rows, int64_t cols,
                        int64_t ldq, const float* scales, int64_t ld_s, void* y, int64_t ldy,
                        hipStream_t st) {
  if (gran == FP8Q_GRAN_TENSOR) launch_dq_o<FMT, FP8Q_GRAN_TENSOR>(out_dt, q, rows, cols, ldq, scales, ld_s, y, ldy, st);
  else if (gran == FP8Q_GRAN_1x128) launch_dq_o<FMT, FP8Q_GRAN_1x128>(out_dt, q, rows, cols, ldq, scales, ld_s, y, ldy, st);
  else launch_dq_o<FMT, FP8Q_GRAN_128x128>(out_dt, q, rows, cols, ldq, scales, ld_s, y, ldy, st);
}

int launch_dequantize(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                      const float* scales, int gran, int64_t ld_s, void* y, int out_dt, int64_t ldy,
                      hipStream_t st) {
  if (fmt == FP8Q_E4M3FN) launch_dq_g<FP8Q_E4M3FN>(gran, out_dt, q, rows, cols, ldq, scales, ld_s, y, ldy, st);
  else launch_dq_g<FP8Q_E5M2>(gran, out_dt, q, rows, cols, ldq, scales, ld_s, y, ldy, st);
  return check_launch("dequantize");
}

template <int DT, int FMT>
static void launch_qmx(int grid, const void* x, int64_t vpr, int64_t nvec, int64_t ldx, uint8_t* q, int64_t ldq,
                       uint8_t* scales, int64_t ld_s, int64_t per_wg, hipStream_t st) {
  hipLaunchKernelGGL((k_quant_mx<DT, FMT>), dim3(grid), dim3(kThreads), 0, st, x, vpr, nvec, ldx, q, ldq, scales,
                     ld_s, per_wg);
}

int launch_quantize_mx(const void* x, int dt, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                       int64_t ldq, uint8_t* scales, int64_t ld_s, hipStream_t st) {
  const int ve = dt == FP8Q_F32 ? 4 : 8;
  const int64_t vpr = cols / ve, nvec = rows * vpr;
  // contiguous chunks of whole thread-steps; a chunk is a multiple of 32
  // elements' lanes, so no block is split between workgroups
  const int64_t steps = (nvec + kThreads - 1) / kThreads;
  const int grid = chunk_grid(steps, FP8Q_G_MX);
  const int64_t per_wg = ((steps + grid - 1) / grid) * kThreads;
  if (dt == FP8Q_F32 && fmt == FP8Q_E4M3FN) launch_qmx<FP8Q_F32, FP8Q_E4M3FN>(grid, x, vpr, nvec, ldx, q, ldq, scales, ld_s, per_wg, st);
  else if (dt == FP8Q_F32) launch_qmx<FP8Q_F32, FP8Q_E5M2>(grid, x, vpr, nvec, ldx, q, ldq, scales, ld_s, per_wg, st);
  else if (fmt == FP8Q_E4M3FN) launch_qmx<FP8Q_BF16, FP8Q_E4M3FN>(grid, x, vpr, nvec, ldx, q, ldq, scales, ld_s, per_wg, st);
  else launch_qmx<FP8Q_BF16, FP8Q_E5M2>(grid, x, vpr, nvec, ldx, q, ldq, scales, ld_s, per_wg, st);
  return check_launch("quantize_mx");
}

template <int FMT, int ODT>
static void launch_dqmx(int grid, const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const uint8_t* scales,
                        int64_t ld_s, void* y, int64_t ldy, int64_t per_wg, hipStream_t st) {
  hipLaunchKernelGGL((k_dequant_mx<FMT, ODT>), dim3(grid), dim3(kThreads), 0, st, q, rows, cols, ldq, scales, ld_s, y,
                     ldy, per_wg);
}

int launch_dequantize_mx(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq, const uint8_t* scales,
                         int64_t ld_s, void* y, int out_dt, int64_t ldy, hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  const int64_t steps = (total + kThreads - 1) / kThreads;
  const int grid = chunk_grid(steps, FP8Q_G_DMX);
  const int64_t per_wg = ((steps + grid - 1) / grid) * kThreads;
  if (fmt == FP8Q_E4M3FN && out_dt == FP8Q_F32) launch_dqmx<FP8Q_E4M3FN, FP8Q_F32>(grid, q, rows, cols, ldq, scales, ld_s, y, ldy, per_wg, st);
  else if (fmt == FP8Q_E4M3FN) launch_dqmx<FP8Q_E4M3FN, FP8Q_BF16>(grid, q, rows, cols, ldq, scales, ld_s, y, ldy, per_wg, st);
  else if (out_dt == FP8Q_F32) launch_dqmx<FP8Q_E5M2, FP8Q_F32>(grid, q, rows, cols, ldq, scales, ld_s, y, ldy, per_wg, st);
  else launch_dqmx<FP8Q_E5M2, FP8Q_BF16>(grid, q, rows, cols, ldq, scales, ld_s, y, ldy, per_wg, st);
  return check_launch("dequantize_mx");
}

}  // namespace fp8q
