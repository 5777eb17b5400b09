// LDS-tiled expert GEMM for many rows per expert (prefill, contiguous
// segments, hot masked experts): MFMA-bound, so every dequantised weight is
// reused by up to 256 token rows.
//
// Workgroup = 4 waves; wave w owns 4 consecutive 16-row weight tiles (64
// output rows), the workgroup 256 output rows of one expert.  A token tile of
// up to MT*16 rows is staged in LDS one 128-wide K chunk at a time (double
// buffer, one barrier per chunk); each wave streams its weight tiles straight
// from HBM into registers two chunks ahead, dequantises them exactly
// (bf16_rne((q - 8) * s), same scheme as the streaming kernel) and issues
// v_mfma_f32_16x16x32_bf16 with the weights as A and the staged tokens as B.
// Work items are (token tile, 256-row slice); the 256-row slices of one token
// tile run on one XCD so its L2 serves the staged token rows.
#include "device_common.h"

namespace chord {
namespace {

constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kNoRow = 0xC0000000u;
constexpr int kStreamAux = 2;
constexpr int kXcds = 8;
constexpr int kRowPitch = kChunkK * 2 + 16;  // LDS bytes per staged token row (padded)

struct DqScale {
  float s, c, s16, c16;
};
__device__ __forceinline__ DqScale dq_scale(uint32_t bits16) {
  const float s = bf16_to_f32(bits16);
  return DqScale{s, -1032.0f * s, 0.0625f * s, -72.0f * s};
}

// One packed word (8 codes of one row, inside one scale group) -> 8 bf16.
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w, const DqScale& k, uint32_t mlo,
                                                 uint32_t mhi, uint32_t magic) {
  const uint32_t w8 = w >> 8;
  const uint32_t m0 = and_or(w, mlo, magic), m1 = and_or(w, mhi, magic);
  const uint32_t m2 = and_or(w8, mlo, magic), m3 = and_or(w8, mhi, magic);
  const half2_t h0 = __builtin_bit_cast(half2_t, m0), h1 = __builtin_bit_cast(half2_t, m1);
  const half2_t h2 = __builtin_bit_cast(half2_t, m2), h3 = __builtin_bit_cast(half2_t, m3);
  const float f0 = __builtin_fmaf((float)h0[0], k.s, k.c), f1 = __builtin_fmaf((float)h0[1], k.s, k.c);
  const float f2 = __builtin_fmaf((float)h1[0], k.s16, k.c16);
  const float f3 = __builtin_fmaf((float)h1[1], k.s16, k.c16);
  const float f4 = __builtin_fmaf((float)h2[0], k.s, k.c), f5 = __builtin_fmaf((float)h2[1], k.s, k.c);
  const float f6 = __builtin_fmaf((float)h3[0], k.s16, k.c16);
  const float f7 = __builtin_fmaf((float)h3[1], k.s16, k.c16);
  return __builtin_bit_cast(bf16x8_t, make_uint4(pk_bf16(f0, f1), pk_bf16(f2, f3),
                                                 pk_bf16(f4, f5), pk_bf16(f6, f7)));
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

struct RowMap {
  int64_t src;
  int64_t dst;
};
__device__ __forceinline__ RowMap map_row(const GemmArgs& a, int expert, int64_t R) {
  RowMap m{-1, -1};
  if (a.layout == kIndexed) {
    const int64_t f = a.sorted_ids[R];
    if (f < 0 || f >= a.n_flat) return m;
    m.src = a.gate_up ? f / a.topk : R;
    m.dst = a.gate_up ? R : f;
  } else if (a.layout == kContiguous) {
    if (a.m_indices[R] != expert) return m;
    m.src = R;
    m.dst = R;
  } else {
    m.src = R;
    m.dst = R;
  }
  return m;
}

// NT = 16-row weight tiles per wave (the workgroup covers 4*NT tiles);
// MT = maximum 16-row token groups per tile (token tile <= MT*16 rows).
template <int NT, int MT>
__global__ __launch_bounds__(256) void gemm_tile(GemmArgs a) {
  constexpr int kWaves = 4;
  constexpr int BM = MT * 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* xbuf = smem;                                        // [2][BM][kRowPitch]
  int32_t* srcoff = reinterpret_cast<int32_t*>(smem + 2 * BM * kRowPitch);  // [BM] byte offsets
  int64_t* dstrow = reinterpret_cast<int64_t*>(srcoff + BM);   // [BM]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar offsets
  const int q = lane >> 4;
  const int col = lane & 15;
  const uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.bsrc, 0, (int)a.bsrc_bytes, kRsrcWord3);
  const int nslices = a.items_per_tile;  // 256-row slices per expert
  const int nc = a.n_chunks;

  // XCD-aware item order: the tile list is grouped by expert % 8;
  // workgroup b runs on XCD b % 8 and takes the tiles of group b % 8 (all
  // slices), so the token tiles of one expert share that XCD's L2 for its
  // weight slices.  With fewer than 8 workgroups each takes several groups.
  const int G = gridDim.x < kXcds ? (int)gridDim.x : kXcds;
  const int xg = blockIdx.x % G;
  const int nloc = (gridDim.x + G - 1 - xg) / G;  // workgroups serving xg
  const int lidx = blockIdx.x / G;

  for (int g = xg; g < kTileGroups; g += G)
  for (int j = lidx, t0 = a.status->group_start[g],
           n_items = (a.status->group_start[g + 1] - t0) * nslices;
       j < n_items; j += nloc) {
    const int ti = t0 + j / nslices;
    const int ng = j % nslices;
    const TileDesc td = a.tiles[ti];
    const int e = td.expert;
    const int nrows = td.nrows < BM ? td.nrows : BM;
    const int mt_live = (nrows + 15) >> 4;

    // Row maps of the token tile.
    for (int m = tid; m < BM; m += 256) {
      int32_t so = (int32_t)kNoRow;
      int64_t dr = -1;
      if (m < nrows) {
        const RowMap rm = map_row(a, e, (int64_t)td.row_begin + m);
        if (rm.src >= 0) {
          so = (int32_t)(rm.src * (int64_t)a.K * 2);
          dr = rm.dst;
        }
      }
      srcoff[m] = so;
      dstrow[m] = dr;
    }
    __syncthreads();

    // Staging: thread tid moves 16-byte pieces (row r, piece p) of the chunk,
    // in kHalves register batches (two for 256-row tiles to bound registers).
    constexpr int kPieces = BM * 16 / 256;  // per thread per chunk
    constexpr int kHalves = MT > 8 ? 2 : 1;
    constexpr int kBatch = kPieces / kHalves;
    uint4 xr[kBatch];
    auto load_x = [&](int c, int h) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int idx = tid + 256 * (h * kBatch + i);
        const int r = idx >> 4, p = idx & 15;
        const uint32_t off = (uint32_t)srcoff[r];
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xres, off + p * 16, c * kChunkK * 2, 0);
        xr[i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    };
    auto store_x = [&](int slot, int h) {
      uint8_t* base = xbuf + slot * BM * kRowPitch;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int idx = tid + 256 * (h * kBatch + i);
        const int r = idx >> 4, p = idx & 15;
        *reinterpret_cast<uint4*>(base + r * kRowPitch + p * 16) = xr[i];
      }
    };

    // Weights of this wave: NT tiles of the slice.
    const int64_t expert_bytes = (int64_t)a.n_tiles * nc * kBlockBytes;
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.wpack + (int64_t)e * expert_bytes), 0, (int)expert_bytes, kRsrcWord3);
    const int tile0 = (ng * kWaves + wave) * NT;  // first weight tile of this wave
    uint4 wq[2][NT];
    uint32_t sc[2][NT];
    auto load_w = [&](int slot, int c) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t blk = (uint32_t)((tile0 + nt) * nc + c) * kBlockBytes;
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, lane * 16, blk, kStreamAux);
        wq[slot][nt] = make_uint4(v[0], v[1], v[2], v[3]);
        sc[slot][nt] = __builtin_amdgcn_raw_buffer_load_b16(wres, kBlockWeightBytes + lane * 2, blk, 0);
      }
    };

    f32x4_t acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = zero4;

    // One chunk: for each MFMA step st, dequantise word st of every weight
    // tile, then sweep the live token groups (in fours) reading B from LDS.
    auto compute = [&](int slot, int st_lo, int st_hi) {
      const uint8_t* xb = xbuf + slot * BM * kRowPitch;
      DqScale ks[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) ks[nt] = dq_scale(sc[slot][nt]);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st < st_lo || st >= st_hi) continue;
        bf16x8_t av[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint32_t w = st == 0 ? wq[slot][nt].x
                           : st == 1 ? wq[slot][nt].y
                           : st == 2 ? wq[slot][nt].z : wq[slot][nt].w;
          av[nt] = dequant_word(w, ks[nt], kMaskLo, kMaskHi, kMagic);
        }
        // B operand of token group mt: row mt*16 + col, k = q*32 + st*8.
        const uint8_t* bp = xb + col * kRowPitch + (q * 32 + st * 8) * 2;
#pragma unroll
        for (int g4 = 0; g4 < MT / 4; ++g4) {
          if (g4 * 4 < mt_live) {
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
              const int mt = g4 * 4 + mm;
              const bf16x8_t bv =
                  *reinterpret_cast<const bf16x8_t*>(bp + mt * 16 * kRowPitch);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                acc[nt][mt] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[nt], bv, acc[nt][mt], 0, 0, 0);
            }
          }
        }
      }
    };

    // Pipeline: x(c+1) loads -> compute(c) -> weights(c+2) loads ->
    // x(c+1) to LDS -> barrier.
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
      load_x(0, h);
      store_x(0, h);
    }
    load_w(0, 0);
    load_w(1, nc > 1 ? 1 : 0);
    __syncthreads();
    // Unrolled by two so the buffer slot is a compile-time index.
    for (int c0 = 0; c0 < nc; c0 += 2) {
#pragma unroll
      for (int slot = 0; slot < 2; ++slot) {
        const int c = c0 + slot;
        if (c < nc) {
          const bool more = c + 1 < nc;
          if (kHalves == 1) {
            if (more) load_x(c + 1, 0);
            compute(slot, 0, 4);
            if (c + 2 < nc) load_w(slot, c + 2);
            if (more) store_x(slot ^ 1, 0);
          } else {
            if (more) load_x(c + 1, 0);
            compute(slot, 0, 2);
            if (more) {
              store_x(slot ^ 1, 0);
              load_x(c + 1, 1);
            }
            compute(slot, 2, 4);
            if (c + 2 < nc) load_w(slot, c + 2);
            if (more) store_x(slot ^ 1, 1);
          }
          __syncthreads();
        }
      }
    }

    // Epilogue: lane holds rows 4q..4q+3 of weight tile nt for token col of
    // group mt.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t dr = mt < mt_live ? dstrow[mt * 16 + col] : -1;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (dr < 0) continue;
        const f32x4_t v = acc[nt][mt];
        const int tw = tile0 + nt;
        if (a.gate_up) {
          const int f0 = tw * 8 + 2 * q;
          *reinterpret_cast<uint32_t*>(a.out + dr * (int64_t)a.out_ld + f0) =
              pk_bf16(silu_mul(v[0], v[1]), silu_mul(v[2], v[3]));
        } else {
          const int n0 = tw * 16 + 4 * q;
          const float rw = a.row_weights != nullptr ? a.row_weights[dr] : 1.0f;
          *reinterpret_cast<uint2*>(a.out + dr * (int64_t)a.out_ld + n0) =
              make_uint2(pk_bf16(v[0] * rw, v[1] * rw), pk_bf16(v[2] * rw, v[3] * rw));
        }
      }
    }
    __syncthreads();  // row maps and LDS reuse by the next item
  }
}

template <int NT, int MT>
hipError_t launch_tile_t(const GemmArgs& a, int grid, hipStream_t stream) {
  const size_t lds = (size_t)2 * MT * 16 * kRowPitch + (size_t)MT * 16 * (4 + 8);
  static const int per_cu = [&] {
    hipFuncSetAttribute((const void*)gemm_tile<NT, MT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)lds);
    return blocks_per_cu(gemm_tile<NT, MT>, 256, lds);
  }();
  const int cap = per_cu * (a.num_cus > 0 ? a.num_cus : 256);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((gemm_tile<NT, MT>), dim3(grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

// Tile kernel: weight tiles per wave fixed at 4 (256 rows per workgroup);
// mt = 16-row token groups per tile (8 or 16).
hipError_t launch_gemm_tile(int mt, const GemmArgs& a, int grid, hipStream_t stream) {
  switch (mt) {
    case 8: return launch_tile_t<4, 8>(a, grid, stream);
    case 16: return launch_tile_t<4, 16>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace chord
