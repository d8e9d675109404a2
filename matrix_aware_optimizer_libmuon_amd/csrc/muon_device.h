// Device-side helpers shared by the libmuon kernels (gfx950): vector types,
// global-address-space accesses, bf16 conversions and the grouped-launch
// work-unit lookup.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"

namespace muon {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Loads through the global address space: the pointers come from the
// descriptor table, so the compiler would otherwise emit generic (flat)
// accesses.
template <class T>
__device__ __forceinline__ T gld(const void* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}
template <class T>
__device__ __forceinline__ void gst(void* p, T v) {
  *(__attribute__((address_space(1))) T*)(p) = v;
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

// Largest i with prefix[i] <= unit (prefix[0] == 0, every matrix owns >= 1 unit).
__device__ __forceinline__ int find_matrix(const int64_t* __restrict__ prefix, int n,
                                           int64_t unit) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= unit) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Workgroups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
// Map them so each XCD receives one contiguous range of logical units:
// neighbouring tiles share operand rows and then meet in the same L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nb) {
  const int64_t per = nb >> 3, rem = nb & 7;
  const int64_t x = b & 7, i = b >> 3;
  return x * per + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ double block_sum_256(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) s = red[0] + red[1] + red[2] + red[3];
  return s;
}

}  // namespace muon
