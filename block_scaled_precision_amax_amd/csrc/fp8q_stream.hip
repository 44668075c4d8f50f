// Streaming reference for the HBM-bound quantizers (libfp8q_stream.so, used
// by the benchmark only): the fastest plain pass over HBM that reads and
// writes in the same proportions as a quantizer, so that a quantizer's
// bandwidth can be set against what a hand-written stream reaches on the
// same chip, not only against the HBM3E peak.
//
// Each lane moves items of RB bytes read and WB bytes written:
//   (16, 16)  a copy,
//   (16, 8)   bf16 in, one byte per element out (a bf16 quantizer),
//   (16, 4)   fp32 in, one byte per element out (an fp32 quantizer),
//   (8, 16)   one byte per element in, bf16 out (a dequantizer),
//   (16, 32)  the same proportion with 16-byte reads and two 16-byte writes,
//   (16, 24)  bf16 in, a byte and a bf16 out per element (a quantizer that
//             also writes the round trip; the 8-byte and 16-byte parts go
//             to two regions of the output, as codes and values would).
// The written words are xor folds (or copies) of the read ones, so nothing
// can be dropped, and no arithmetic competes with the memory traffic.  Work
// is cut into contiguous chunks of U items per lane, walked by a persistent
// grid of G workgroups of TH threads per compute unit (the layout the
// quantizers use); U, G and TH are swept by the caller.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int RB>
using rd_t = typename std::conditional<RB == 16, u32x4, u32x2>::type;

template <int RB, int WB, int U, int TH>
__global__ __launch_bounds__(TH) void k_stream(const uint8_t* __restrict__ in, uint8_t* __restrict__ out,
                                               int64_t nitems) {
  constexpr int64_t kChunk = (int64_t)U * TH;
  for (int64_t c = blockIdx.x; c * kChunk < nitems; c += gridDim.x) {
    const int64_t base = c * kChunk + threadIdx.x;
    rd_t<RB> v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + u * TH < nitems) v[u] = __builtin_nontemporal_load((const rd_t<RB>*)in + base + u * TH);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * TH;
      if (i >= nitems) break;
      if constexpr (RB == 8) {
        __builtin_nontemporal_store(u32x4{v[u].x, v[u].y, v[u].x ^ v[u].y, v[u].y}, (u32x4*)out + i);
      } else if constexpr (WB == 32) {
        __builtin_nontemporal_store(v[u], (u32x4*)out + 2 * i);
        __builtin_nontemporal_store(u32x4{v[u].y, v[u].x, v[u].w, v[u].z}, (u32x4*)out + 2 * i + 1);
      } else if constexpr (WB == 24) {
        __builtin_nontemporal_store(u32x2{v[u].x ^ v[u].y, v[u].z ^ v[u].w}, (u32x2*)out + i);
        __builtin_nontemporal_store(v[u], (u32x4*)(out + 8 * nitems) + i);
      } else if constexpr (WB == 16) {
        __builtin_nontemporal_store(v[u], (u32x4*)out + i);
      } else if constexpr (WB == 8) {
        __builtin_nontemporal_store(u32x2{v[u].x ^ v[u].y, v[u].z ^ v[u].w}, (u32x2*)out + i);
      } else {
        __builtin_nontemporal_store(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w, (uint32_t*)out + i);
      }
    }
  }
}

template <int RB, int WB, int TH>
hipError_t launch_u(int u, int grid, const uint8_t* in, uint8_t* out, int64_t n, hipStream_t st) {
  switch (u) {
    case 1: hipLaunchKernelGGL((k_stream<RB, WB, 1, TH>), dim3(grid), dim3(TH), 0, st, in, out, n); break;
    case 2: hipLaunchKernelGGL((k_stream<RB, WB, 2, TH>), dim3(grid), dim3(TH), 0, st, in, out, n); break;
    case 4: hipLaunchKernelGGL((k_stream<RB, WB, 4, TH>), dim3(grid), dim3(TH), 0, st, in, out, n); break;
    default: hipLaunchKernelGGL((k_stream<RB, WB, 8, TH>), dim3(grid), dim3(TH), 0, st, in, out, n); break;
  }
  return hipGetLastError();
}

template <int RB, int WB>
hipError_t launch_k(int u, int threads, int grid, const uint8_t* in, uint8_t* out, int64_t n, hipStream_t st) {
  return threads == 1024 ? launch_u<RB, WB, 1024>(u, grid, in, out, n, st)
                         : launch_u<RB, WB, 256>(u, grid, in, out, n, st);
}

}  // namespace

extern "C" {

// in: items * rd bytes, out: items * wr bytes, both 16-B aligned, with
// (rd, wr) one of (16, 16), (16, 8), (16, 4), (8, 16), (16, 32), (16, 24)
// (for (16, 24) items must be even, so the 16-byte part stays aligned);
// vectors_per_lane in
// {1, 2, 4, 8}; threads (per workgroup) 256 or 1024; the grid is
// wg_per_cu * cu_count workgroups (the caller passes the device's
// compute-unit count, so nothing is queried while a graph is being
// captured).  Returns 0, -1 for bad arguments, or the HIP error code of the
// launch.  Asynchronous on `stream` (a hipStream_t).
int fp8q_stream_ref(const void* in, void* out, int64_t items, int rd, int wr, int vectors_per_lane,
                    int wg_per_cu, int cu_count, int threads, void* stream) {
  if (!in || !out || items <= 0 || ((uintptr_t)in | (uintptr_t)out) % 16 != 0 || wg_per_cu < 1 || cu_count < 1 ||
      (threads != 256 && threads != 1024))
    return -1;
  const bool ok = (rd == 16 && (wr == 32 || wr == 24 || wr == 16 || wr == 8 || wr == 4)) || (rd == 8 && wr == 16);
  if (wr == 24 && (items & 1)) return -1;
  const int u = vectors_per_lane;
  if (!ok || (u != 1 && u != 2 && u != 4 && u != 8)) return -1;
  const int cus = cu_count;
  const int64_t chunks = (items + (int64_t)u * threads - 1) / ((int64_t)u * threads);
  const int64_t g = (int64_t)cus * wg_per_cu;
  const int grid = (int)(chunks < g ? chunks : g);
  hipStream_t st = (hipStream_t)stream;
  const uint8_t* src = (const uint8_t*)in;
  uint8_t* dst = (uint8_t*)out;
  hipError_t e;
  if (rd == 8)
    e = launch_k<8, 16>(u, threads, grid, src, dst, items, st);
  else if (wr == 32)
    e = launch_k<16, 32>(u, threads, grid, src, dst, items, st);
  else if (wr == 24)
    e = launch_k<16, 24>(u, threads, grid, src, dst, items, st);
  else if (wr == 16)
    e = launch_k<16, 16>(u, threads, grid, src, dst, items, st);
  else if (wr == 8)
    e = launch_k<16, 8>(u, threads, grid, src, dst, items, st);
  else
    e = launch_k<16, 4>(u, threads, grid, src, dst, items, st);
  return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
