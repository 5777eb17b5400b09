// Small device helpers shared by the HIP translation units of libchord.so.
#pragma once

#include "internal.h"

namespace chord {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Two fp32 -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// (a & m) | c in one VALU instruction (the compiler otherwise emits two).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// Exclusive scan of one int per thread across the workgroup (blockDim.x a
// multiple of 64, at most 1024).  `tmp` holds >= 16 ints of LDS.
__device__ inline int block_scan_excl(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0, sum = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = tmp[w];
    if (w < wave) base += t;
    sum += t;
  }
  __syncthreads();
  *total = sum;
  return base + x - v;
}

// Exclusive scans of N ints per thread across the workgroup at once (same
// contract as block_scan_excl; `tmp` holds >= 16 * N ints of LDS): v[i]
// becomes the exclusive prefix of counter i, total[i] its sum.  Two barriers
// for all N counters instead of two per counter.
template <int N>
__device__ inline void block_scan_excl_n(int (&v)[N], int* tmp, int (&total)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = v[i];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int y = __shfl_up(x[i], d, 64);
      if (lane >= d) x[i] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[wave * N + i] = x[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int base = 0, sum = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = tmp[w * N + i];
      if (w < wave) base += t;
      sum += t;
    }
    v[i] = base + x[i] - v[i];
    total[i] = sum;
  }
  __syncthreads();
}

// Resident workgroups per CU of a kernel.
template <typename K>
inline int blocks_per_cu(K kernel, int threads, size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n < 1)
    n = 1;
  return n;
}

}  // namespace chord
