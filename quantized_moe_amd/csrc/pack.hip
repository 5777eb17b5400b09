// Weight packing: canonical W4A16 tensors -> the gfx950 block layout
// (described in internal.h).  Load-time work, one 64-lane workgroup per
// 1152-byte block.
#include "internal.h"

namespace chord {
namespace {

// Reorders the 8 codes of a canonical word (code i at bits 4i) so that code
// 2v lands at bits 4v and code 2v+1 at bits 16+4v.
__device__ __forceinline__ uint32_t shuffle_codes(uint32_t w) {
  uint32_t r = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    r |= ((w >> (8 * v)) & 0xFu) << (4 * v);
    r |= ((w >> (8 * v + 4)) & 0xFu) << (16 + 4 * v);
  }
  return r;
}

__global__ __launch_bounds__(64) void pack_kernel(const int32_t* __restrict__ q,
                                                   const uint16_t* __restrict__ s, int N, int K,
                                                   int gate_up, uint8_t* __restrict__ dst) {
  const int n_tiles = N / kTileRows;
  const int n_chunks = K / kChunkK;
  const int64_t blk = blockIdx.x;
  const int c = (int)(blk % n_chunks);
  const int t = (int)((blk / n_chunks) % n_tiles);
  const int e = (int)(blk / ((int64_t)n_chunks * n_tiles));
  const int l = threadIdx.x;
  const int r = l % 16, g = l / 16;
  int n;
  if (gate_up) {
    const int I = N / 2;
    const int qq = r / 4, w = r % 4;
    const int f = 8 * t + 2 * qq + (w >> 1);
    n = f + (w & 1) * I;
  } else {
    n = 16 * t + r;
  }
  const int k0 = c * kChunkK + g * kGroup;
  const int32_t* src = q + ((int64_t)e * N + n) * (K / 8) + k0 / 8;
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = shuffle_codes((uint32_t)src[i]);
  uint8_t* b = dst + blk * kBlockBytes;
  *reinterpret_cast<uint4*>(b + l * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  reinterpret_cast<uint16_t*>(b + kBlockWeightBytes)[l] =
      s[((int64_t)e * N + n) * (K / kGroup) + k0 / kGroup];
}

}  // namespace

hipError_t launch_pack(const int32_t* q, const uint16_t* s, int E, int N, int K, int gate_up,
                       uint8_t* dst, hipStream_t stream) {
  const int64_t blocks = (int64_t)E * (N / kTileRows) * (K / kChunkK);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, q, s, N, K, gate_up,
                     dst);
  return hipGetLastError();
}

}  // namespace chord
