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

// SiLU(g) * u in fp32 for the fused gate_up epilogue: g * rcp(1 + e^-g) * u
// with the hardware exp and reciprocal (each within about 1 ulp; the result
// is rounded to bf16 next).  g -> -inf gives -0, g -> +inf gives g, NaN
// propagates.  Every kernel family uses this one definition, so they agree
// bit for bit.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// (a & m) | c in one VALU instruction (the compiler otherwise emits two).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// Inclusive scan over the 64 lanes of a wave in registers (DPP, no LDS):
// rows of 16 lanes add their left neighbours 1, 2, 4 and 8 places away
// (lanes without one in the row add 0), then rows 1 and 3 add the last lane
// of the row before, and rows 2 and 3 the last lane of row 1.  The first
// four steps alone scan each row of 16.
__device__ __forceinline__ int row_incl_scan16(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x = row_incl_scan16(x);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive scans of N ints per thread across the workgroup (blockDim.x a
// multiple of 64, at most 1024; `tmp` holds >= 17 * N ints of LDS): v[i]
// becomes the exclusive prefix of counter i over the thread order, total[i]
// its sum.  Each wave scans its lanes in registers; wave 0 then scans the
// (at most 16) wave totals the same way and writes back each wave's
// inclusive prefix and the totals, so every thread reads 2N values from LDS
// in one batch (a loop over the wave totals in every thread would wait for
// one LDS read at a time).  Three barriers for all N counters.
template <int N>
__device__ inline void block_scan_excl_n(int (&v)[N], int* tmp, int (&total)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = wave_incl_scan(v[i]);
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[wave * N + i] = x[i];
  }
  __syncthreads();
  if (wave == 0) {
    int s[N];
#pragma unroll
    for (int i = 0; i < N; ++i) s[i] = row_incl_scan16(lane < nw ? tmp[lane * N + i] : 0);
    if (lane < nw) {
#pragma unroll
      for (int i = 0; i < N; ++i) tmp[lane * N + i] = s[i];
    }
    if (lane == nw - 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) tmp[16 * N + i] = s[i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int before = wave > 0 ? tmp[(wave - 1) * N + i] : 0;
    total[i] = tmp[16 * N + i];
    v[i] = before + x[i] - v[i];
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
