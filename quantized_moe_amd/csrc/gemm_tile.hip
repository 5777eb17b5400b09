// LDS-tiled expert GEMM for many rows per expert (prefill, contiguous
// segments, hot masked experts): MFMA-bound, so every dequantised weight is
// reused by up to 192 token rows.
//
// Workgroup = W waves (4: one per SIMD, or 8: two per SIMD); wave w owns
// 16 / W consecutive 16-row weight tiles, the workgroup a 256-row slice of one
// expert's output.  A single wave per SIMD cannot issue MFMAs back to back
// (it saturates near 1.5 PFLOP/s on gfx950 whatever its number of independent
// accumulators), two reach about 2.1 PFLOP/s; the 8-wave form gets there by
// halving each wave's tiles (and registers) over the same LDS token stage.
// A token tile of up to 192 rows is staged in LDS one 128-wide K chunk at a
// time (three buffers, one barrier per chunk).  Each wave streams
// its weight tiles straight from HBM into registers two chunks ahead,
// dequantises them exactly (bf16_rne((q - 8) * s)) and issues
// v_mfma_f32_16x16x32_bf16 with the weights as A and the staged tokens as B.
// The number of live 16-row token groups of a tile selects a compile-time
// variant, so the chunk body is one branch-free block in which the
// dequantisation of MFMA step s+1 is interleaved with the MFMAs of step s.
// Work items are (token tile, 256-row slice); the slices of one expert run on
// one XCD so its L2 serves the staged token rows.
#include "device_common.h"

namespace chord {
namespace {

constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kNoRow = 0xC0000000u;  // byte offset past any token buffer
constexpr int kStreamAux = 2;
constexpr int kXcds = 8;
constexpr int kWaves = 4;                     // short-K kernel: waves per workgroup
constexpr int kNT = 4;                        // short-K kernel: weight tiles per wave
constexpr int kSliceTiles = 16;               // 16-row weight tiles per 256-row slice
constexpr int kMaxGroups = 12;                // 16-row token groups per tile (192 rows)
constexpr int kXBufBytes = kMaxGroups * 16 * kChunkK * 2;  // one staged K chunk, 192 rows
constexpr int kStages = 3;                    // token / weight buffers (two chunks in flight)
constexpr size_t kLdsBytes = kStages * (size_t)kXBufBytes + kMaxGroups * 16 * (4 + 8 + 4);

struct DqScale {
  float s, c, s16, c16;
};
__device__ __forceinline__ DqScale dq_scale(uint32_t bits16) {
  const float s = bf16_to_f32(bits16);
  return DqScale{s, -1032.0f * s, 0.0625f * s, -72.0f * s};
}

// One packed word (8 codes of one row, inside one scale group) -> 8 bf16.
// Codes read through the fp16 magic 0x6400 | q = 1024 + q (low nibble of a
// half) or 1024 + 16 q (high nibble), so fma(h, s, -1032 s) and
// fma(h, s/16, -72 s) give (q - 8) * s exactly; v_cvt_pk_bf16_f32 rounds.
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w, const DqScale& k) {
  const uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  const uint32_t w8 = w >> 8;
  const uint32_t m0 = and_or(w, kMaskLo, kMagic), m1 = and_or(w, kMaskHi, kMagic);
  const uint32_t m2 = and_or(w8, kMaskLo, kMagic), m3 = and_or(w8, kMaskHi, kMagic);
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

__device__ __forceinline__ uint32_t word_of(const uint4& v, int st) {
  return st == 0 ? v.x : st == 1 ? v.y : st == 2 ? v.z : v.w;
}

struct RowMap {
  int64_t src;
  int64_t dst;
};
// LDS swizzle key of a token row (row % 16 -> a permutation of 0..15).
__device__ __forceinline__ int swz(int r16) { return ((r16 & 7) << 1) | (r16 >> 3); }

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

// Down epilogue: y = acc * row weight, bf16.  Lane (q, col) holds outputs
// 4q .. 4q+3 of each weight tile for token col; lanes exchange packed halves
// (two register row swaps) so that each lane stores 16 contiguous bytes: lane q
// takes tile 2i + q / 2, outputs 8 (q % 2) .. 8 (q % 2) + 7, from lanes
// 2 (q % 2) and 2 (q % 2) + 1 of its token.  Stores of 16 instead of 8 bytes
// per lane (32 -> 64 contiguous bytes per token row) made the short-K down
// GEMM of the I = 256 slices 17 % faster.
template <int NT, int MG>
__device__ __forceinline__ void store_down_pairs(const GemmArgs& a, const f32x4_t (&acc)[NT][MG],
                                                 const int64_t* dstrow, const float* roww,
                                                 int tile0, int q, int col) {
  static_assert(NT % 2 == 0, "tile pairs");
#pragma unroll
  for (int g = 0; g < MG; ++g) {
    const int64_t dr = dstrow[g * 16 + col];
    const float rw = roww[g * 16 + col];
#pragma unroll
    for (int i = 0; i < NT / 2; ++i) {
      const f32x4_t v0 = acc[2 * i][g], v1 = acc[2 * i + 1][g];
      const uint32_t p0x = pk_bf16(v0[0] * rw, v0[1] * rw), p0y = pk_bf16(v0[2] * rw, v0[3] * rw);
      const uint32_t p1x = pk_bf16(v1[0] * rw, v1[1] * rw), p1y = pk_bf16(v1[2] * rw, v1[3] * rw);
      // Row exchange in registers: swapping the upper two 16-lane rows of the
      // tile-2i values with the lower two of the tile-2i+1 values, then odd
      // with even rows, leaves lane (q, col) with rows (2q & 3) and its
      // successor of tile 2i + q / 2: its 16 contiguous output bytes.
      const auto sx = __builtin_amdgcn_permlane32_swap(p0x, p1x, false, false);
      const auto sy = __builtin_amdgcn_permlane32_swap(p0y, p1y, false, false);
      const auto tx = __builtin_amdgcn_permlane16_swap(sx[0], sx[1], false, false);
      const auto ty = __builtin_amdgcn_permlane16_swap(sy[0], sy[1], false, false);
      if (dr < 0) continue;
      const int tw = tile0 + 2 * i + (q >> 1);
      const int n0 = tw * 16 + (q & 1) * 8;
      *reinterpret_cast<uint4*>(a.out + dr * (int64_t)a.out_ld + n0) =
          make_uint4(tx[0], ty[0], tx[1], ty[1]);
    }
  }
}

// One work item: token tile of MG live 16-row groups x one 256-row slice.
// srcoff / dstrow (LDS) already hold the tile's row maps.
//
// Token staging goes straight from memory to LDS (buffer_load ... lds): one
// instruction moves 4 token rows x 256 bytes (one K chunk) into 1 KB of LDS
// in lane order.  LDS row r holds the row's 16-byte pieces permuted by
// slot = piece ^ swz(r % 16); lane l of the instruction for rows 4j..4j+3
// fetches piece (l % 16) ^ swz(r % 16) of row r = 4j + l / 16, so each row is
// still read as one contiguous 256-byte run.  The MFMA B reads (16 rows, one
// piece each) then hit 16 distinct slots, and the key swz(r) = 2 (r % 8) +
// r / 8 also spreads rows r and r + 8 over different bank halves: gfx950
// serves a 128-bit LDS read in 8-byte halves, 16 lanes at a time, and a plain
// piece ^ r leaves those 16 lanes on 8 bank pairs (2-way conflicts; measured
// 143 vs 245 bytes per clock per CU).
template <int MG, int W>
__device__ __forceinline__ void run_item(const GemmArgs& a, uint8_t* xbuf, const int32_t* srcoff,
                                         const int64_t* dstrow, const float* roww,
                                         const TileDesc& td, int ng) {
  const int e = td.expert;
  constexpr int NT = kSliceTiles / W;  // weight tiles per wave
  constexpr int kDma = (4 * MG + W - 1) / W;  // token DMA instructions per wave and chunk
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int col = lane & 15;
  // K range of this entry: part kpart of ksplit (the whole K when unsplit).
  const int c_lo = td.kpart * a.n_chunks / td.ksplit;
  const int c_hi = (td.kpart + 1) * a.n_chunks / td.ksplit;  // end of the range
  const int nc = a.n_chunks;  // chunks per weight tile (block stride)
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  // Wave w issues the DMA instructions j = w + W i (rows 4j .. 4j+3).  When
  // W does not divide 4 MG, the surplus slots repeat the last row block
  // (j = 4 MG - 1): an identical copy, same source and same LDS bytes, so
  // every wave issues kDma loads and the wait counts below stay exact.
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.bsrc, 0, (int)a.bsrc_bytes, kRsrcWord3);
  uint32_t voff[kDma];
  int jblk[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    jblk[i] = min(wave + W * i, 4 * MG - 1);
    const int row = 4 * jblk[i] + q;
    voff[i] = (uint32_t)srcoff[row] + (uint32_t)((col ^ swz(row & 15)) * 16);
  }
  auto load_x = [&](int slot, int c) {
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      uint8_t* dst = xbuf + slot * kXBufBytes + jblk[i] * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void*)dst, 16, voff[i], c * kChunkK * 2, 0, 0);
    }
  };

  // Weights: NT tiles of the slice per wave.  A wave past the last tile of
  // a partial slice re-reads the slice's last tiles and stores nothing.
  const int64_t expert_bytes = (int64_t)a.n_tiles * nc * kBlockBytes;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.wpack + (int64_t)e * expert_bytes), 0, (int)expert_bytes, kRsrcWord3);
  const int tile0 = (ng * W + wave) * NT;
  const bool wave_live = tile0 < a.n_tiles;
  const int tile_ld = wave_live ? tile0 : a.n_tiles - NT;
  uint4 wq[kStages][NT];
  uint32_t sc[kStages][NT];
  auto load_w = [&](int slot, int c) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t blk = (uint32_t)((tile_ld + nt) * nc + c) * kBlockBytes;
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, lane * 16, blk, kStreamAux);
      wq[slot][nt] = make_uint4(v[0], v[1], v[2], v[3]);
      sc[slot][nt] = __builtin_amdgcn_raw_buffer_load_b16(wres, kBlockWeightBytes + lane * 2, blk, 0);
    }
  };

  // Load piece j of chunk c into buffer `slot`: pieces 0 .. kDma-1 are the
  // token DMA instructions, then per weight tile the codes and the scale,
  // i.e. the order load_x followed by load_w issues them.
  constexpr int kPieces = kDma + 2 * NT;
  auto load_piece = [&](int j, int slot, int c) {
    if (j < kDma) {
      uint8_t* dst = xbuf + slot * kXBufBytes + jblk[j] * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void*)dst, 16, voff[j], c * kChunkK * 2, 0, 0);
      return;
    }
    const int nt = (j - kDma) >> 1;
    const uint32_t blk = (uint32_t)((tile_ld + nt) * nc + c) * kBlockBytes;
    if (((j - kDma) & 1) == 0) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, lane * 16, blk, kStreamAux);
      wq[slot][nt] = make_uint4(v[0], v[1], v[2], v[3]);
    } else {
      sc[slot][nt] = __builtin_amdgcn_raw_buffer_load_b16(wres, kBlockWeightBytes + lane * 2, blk, 0);
    }
  };

  f32x4_t acc[NT][MG];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int g = 0; g < MG; ++g) acc[nt][g] = zero4;

  // B operand of group g, step st: token row g*16 + col, piece q*4 + st.
  uint32_t boff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st)
    boff[st] = (uint32_t)(col * 256 + (((q * 4 + st) ^ swz(col)) * 16));

  // One chunk, software-pipelined by hand (scheduling fences keep the order):
  // the chunk is 4 MFMA steps x MG token groups; each group section issues
  // the LDS read of the B fragment two groups ahead, the 4 MFMAs of its own
  // group, and a share of the dequantisation of the next step (weight tile
  // nt is dequantised in group nt * MG / 4).  av holds the dequantised
  // weights of the current step; the last step dequantises step 0 of the
  // next chunk from the weight slot `next`.  B reads do not cross the chunk
  // boundary: the next chunk's buffer is only valid after the barrier.
  bf16x8_t av[NT];
  auto bread = [&](const uint8_t* xb, int st, int g) {
    return *reinterpret_cast<const bf16x8_t*>(xb + boff[st] + g * 16 * 256);
  };
  auto compute = [&](int slot, int next, int fill, int cfill) {
    const uint8_t* xb = xbuf + slot * kXBufBytes;
    DqScale ks[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ks[nt] = dq_scale(sc[slot][nt]);
    bf16x8_t bwin[3];
    bwin[0] = bread(xb, 0, 0);
    bwin[1] = MG > 1 ? bread(xb, 0, 1) : bread(xb, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8_t an[NT];
#pragma unroll
      for (int g = 0; g < MG; ++g) {
        const int idx = st * MG + g;
        const int ahead = idx + 2;
        if (ahead < 4 * MG) bwin[ahead % 3] = bread(xb, ahead / MG, ahead % MG);
        const bf16x8_t bv = bwin[idx % 3];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[nt], bv, acc[nt][g], 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (nt * MG / NT != g) continue;
          an[nt] = st < 3 ? dequant_word(word_of(wq[slot][nt], st + 1), ks[nt])
                          : dequant_word(wq[next][nt].x, dq_scale(sc[next][nt]));
        }
        // Prefetch pieces of chunk cfill, spread evenly over all but the last
        // two sections (spread over all of them, the 11-group variant
        // spills registers).
#pragma unroll
        for (int j = 0; j < kPieces; ++j)
          if (j * (4 * MG - 2) / kPieces == idx) load_piece(j, fill, cfill);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) av[nt] = an[nt];
    }
  };

  // Chunk c in buffer c % 3: compute(c), issuing the x(c+2) DMA and the
  // weights(c+2) loads into the buffer freed by chunk c-1 one piece at a
  // time between its group sections (issued together at the chunk start,
  // the 8 waves' ~66 KB per CU queued behind each other at the texture unit
  // for ~0.4 us with no math in between), then wait until the DMA of x(c+1)
  // (issued one chunk ago) has landed and pass the workgroup barrier.  The
  // barrier is a bare s_barrier with an explicit vmcnt wait: a fenced
  // __syncthreads would also wait for the x(c+2) DMA just issued.  Loads
  // issued after x(c+1): w(c+1) (NT x 2), x(c+2) (kDma), w(c+2) (NT x 2).
  // Prefetch indices are clamped instead of guarded so every iteration
  // issues the same loads (exact wait counts); the clamped re-reads at the
  // end hit the caches.
  constexpr int kWLoads = 2 * NT;
  constexpr int kVm = kDma + 2 * kWLoads;
  constexpr int kWaitX = (kVm & 15) | (7 << 4) | (15 << 8) | ((kVm >> 4) << 14);
  auto chunk = [&](int slot, int c) {
    const int c2 = c + 2 < c_hi ? c + 2 : c_hi - 1;
    const int fill = slot == 0 ? 2 : slot - 1;
    compute(slot, slot == 2 ? 0 : slot + 1, fill, c2);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitX);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  const int c1 = c_lo + 1 < c_hi ? c_lo + 1 : c_lo;
  load_x(0, c_lo);
  load_w(0, c_lo);
  load_x(1, c1);
  load_w(1, c1);
  __builtin_amdgcn_s_waitcnt(kWaitX);  // x(0) landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) av[nt] = dequant_word(wq[0][nt].x, dq_scale(sc[0][nt]));
  int c = c_lo;
  for (; c + 2 < c_hi; c += 3) {
    chunk(0, c);
    chunk(1, c + 1);
    chunk(2, c + 2);
  }
  if (c < c_hi) chunk(0, c);
  if (c + 1 < c_hi) chunk(1, c + 1);
  // Drain the clamped prefetches (DMA into LDS) before the buffers are
  // reused by the next item.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

  // K split: each part only stores its fp32 accumulators to its partial
  // slot (lane-linear, i.e. the register layout, indexed by the tile's place
  // in the slice); the fixup kernel that follows this launch on the stream
  // adds the parts in part order and runs the epilogue.
  if (td.ksplit > 1) {
    if (!wave_live) return;
    f32x4_t* mine = reinterpret_cast<f32x4_t*>(
        a.partials + (size_t)(td.pbase + (td.kpart * a.max_slices + ng) * MG) * kPartialSlotFloats);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int g = 0; g < MG; ++g) mine[((wave * NT + nt) * MG + g) * 64 + lane] = acc[nt][g];
    return;
  }

  // Epilogue: lane holds rows 4q..4q+3 of weight tile nt for token col of
  // group g.
  if (!wave_live) return;
  if (!a.gate_up) {
    store_down_pairs<NT, MG>(a, acc, dstrow, roww, tile0, q, col);
    return;
  }
#pragma unroll
  for (int g = 0; g < MG; ++g) {
    const int64_t dr = dstrow[g * 16 + col];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (dr < 0) continue;
      const f32x4_t v = acc[nt][g];
      const int tw = tile0 + nt;
      const int f0 = tw * 8 + 2 * q;
      *reinterpret_cast<uint32_t*>(a.out + dr * (int64_t)a.out_ld + f0) =
          pk_bf16(silu_mul(v[0], v[1]), silu_mul(v[2], v[3]));
    }
  }
}

template <int W>
__global__ __launch_bounds__(64 * W) void gemm_tile(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* xbuf = smem;                                                  // [3][192][256 B]
  int32_t* srcoff = reinterpret_cast<int32_t*>(smem + kStages * kXBufBytes);  // [192] byte offsets
  int64_t* dstrow = reinterpret_cast<int64_t*>(srcoff + kMaxGroups * 16);  // [192]
  float* roww = reinterpret_cast<float*>(dstrow + kMaxGroups * 16);        // [192] row weights
  const int tid = threadIdx.x;
  const int nslices = a.items_per_tile;

  // XCD-aware item order: the tile list comes in 8 groups of balanced size;
  // workgroup b runs on XCD b % 8 and takes the tiles of group b % 8 (all
  // slices), so the token rows of one tile stay in that XCD's L2 across its
  // slices.  With fewer than 8 workgroups each takes several groups.
  const int G = gridDim.x < kXcds ? (int)gridDim.x : kXcds;
  const int xg = blockIdx.x % G;
  const int nloc = (gridDim.x + G - 1 - xg) / G;  // workgroups serving xg
  const int lidx = blockIdx.x / G;

  for (int g = xg; g < kTileGroups; g += G)
    for (int j = lidx, t0 = a.status->group_start[g],
             n_items = (a.status->group_start[g + 1] - t0) * nslices;
         j < n_items; j += nloc) {
      const TileDesc td = a.tiles[t0 + j / nslices];
      const int ng = j % nslices;
      const int e = td.expert;
      const int nrows = td.nrows < kMaxGroups * 16 ? td.nrows : kMaxGroups * 16;

      if (tid < kMaxGroups * 16) {  // row maps of the token tile: one row per thread
        const int m = tid;
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
        roww[m] = (dr >= 0 && !a.gate_up && a.row_weights != nullptr) ? a.row_weights[dr] : 1.0f;
      }
      __syncthreads();

      // Live 16-row groups (a 171-row tile computes 176 rows, not 192).
      switch ((nrows + 15) >> 4) {
        case 0: break;
#define CHORD_TILE_CASE(MG) \
  case MG: run_item<MG, W>(a, xbuf, srcoff, dstrow, roww, td, ng); break;
        CHORD_TILE_CASE(1) CHORD_TILE_CASE(2) CHORD_TILE_CASE(3) CHORD_TILE_CASE(4)
        CHORD_TILE_CASE(5) CHORD_TILE_CASE(6) CHORD_TILE_CASE(7) CHORD_TILE_CASE(8)
        CHORD_TILE_CASE(9) CHORD_TILE_CASE(10) CHORD_TILE_CASE(11)
#undef CHORD_TILE_CASE
        default: run_item<12, W>(a, xbuf, srcoff, dstrow, roww, td, ng); break;
      }
      __syncthreads();  // row maps and LDS reuse by the next item
    }
}

// ---------------------------------------------------------------------------
// Producer/consumer form (K > 256, no K split): the dequantisation moves out
// of the MFMA waves.  On gfx950 VALU work that other waves issue overlaps a
// wave's back-to-back MFMAs almost entirely, while the same work interleaved
// in the MFMA wave's own stream slows it by a fifth to a third (measured with
// a timing probe at 1 to 2 dequantised words per 16 MFMAs), so a workgroup of
// 12 waves splits into:
//   * 8 consumers (two per SIMD) owning 2 weight tiles (32 output rows)
//     each: per MFMA step they read their dequantised A fragments and the
//     token B fragments from LDS and issue 2 x MG MFMAs;
//   * 4 producers (one per SIMD) owning 4 tiles each: they stream the packed
//     weights into registers two chunks ahead, dequantise each step two steps
//     ahead of the consumers into a 3-stage LDS ring of bf16 A fragments
//     (16 KB per step: 16 tiles x 64 lanes x 16 B, each lane's fragment where
//     the consumer lane of the same index reads it), and DMA the token chunk
//     one chunk ahead into 2 stages.
// One workgroup barrier per step; both roles pass the same number.  Every
// output is summed over the same chunks and steps in the same order as in
// run_item, so both forms agree bit for bit.
//
// Measured on the prefill EP share it is the slower form (gate_up 542 vs
// 400 us): with the producers' dequantisation switched off (timing only) the
// consumers alone take 376 us, so the A fragments' round trip through LDS and
// the per-step barriers cost nearly all that the overlap gains.  The planner
// therefore keeps the single-role form; this one is opt-in (schedule kernel 5,
// CHORD_W4A16_TILE_PC=1).
// ---------------------------------------------------------------------------
constexpr int kPcWaves = 12;
constexpr int kPcConsumers = 8;
constexpr int kPcXStages = 2;
constexpr int kPcAStages = 3;
constexpr int kPcAStepBytes = kSliceTiles * 64 * 16;
constexpr size_t kPcLdsBytes = kPcXStages * (size_t)kXBufBytes +
                               kPcAStages * (size_t)kPcAStepBytes + kMaxGroups * 16 * (4 + 8 + 4);

// Workgroup barrier of the producer/consumer form: wait for this wave's own
// counters (an s_waitcnt immediate), then s_barrier.  The empty asm with a
// memory clobber on both sides keeps the compiler from moving or merging LDS
// accesses across it (s_barrier alone is not a memory operation to the
// compiler), and the scheduling fences keep the machine scheduler out.
template <int kWait>
__device__ __forceinline__ void pc_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWait);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// s_waitcnt immediates (gfx9 encoding): LDS done and no vector-memory wait;
// LDS done and at most N vector-memory operations in flight.
constexpr int kWaitLds = 15 | (7 << 4) | (0 << 8) | (3 << 14);
template <int N>
constexpr int wait_vm_lds() { return (N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14); }

template <int MG>
__device__ __forceinline__ void run_item_pc(const GemmArgs& a, uint8_t* xbuf, uint8_t* abuf,
                                            const int32_t* srcoff, const int64_t* dstrow,
                                            const float* roww, const TileDesc& td, int ng) {
  constexpr int NTC = kSliceTiles / kPcConsumers;                   // 2 tiles per consumer
  constexpr int NTP = kSliceTiles / (kPcWaves - kPcConsumers);      // 4 tiles per producer
  constexpr int kDma = MG;    // token DMA instructions per producer and chunk (4 MG row blocks)
  constexpr int kWLoads = 2 * NTP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int col = lane & 15;
  const int nc = a.n_chunks;  // > 2 here
  const int e = td.expert;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  // Lane l's 16-byte A fragment of slice tile t in stage st of the ring.
  auto afrag = [&](int stage, int t) {
    return abuf + stage * kPcAStepBytes + (t * 64 + lane) * 16;
  };

  if (wave >= kPcConsumers) {
    // ------------------------------ producer ------------------------------
    const int pw = wave - kPcConsumers;
    const int ptile0 = ng * kSliceTiles + pw * NTP;
    const int tile_ld = ptile0 + NTP <= a.n_tiles ? ptile0 : a.n_tiles - NTP;  // past the end: re-read
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.bsrc, 0, (int)a.bsrc_bytes, kRsrcWord3);
    uint32_t voff[kDma];
    int jblk[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      jblk[i] = pw + 4 * i;  // row blocks 4 jblk .. 4 jblk + 3 (all < 4 MG)
      const int row = 4 * jblk[i] + q;
      voff[i] = (uint32_t)srcoff[row] + (uint32_t)((col ^ swz(row & 15)) * 16);
    }
    auto dma_x = [&](int c) {  // token chunk c into stage c % 2
#pragma unroll
      for (int i = 0; i < kDma; ++i) {
        uint8_t* dst = xbuf + (c & 1) * kXBufBytes + jblk[i] * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xres, (__attribute__((address_space(3))) void*)dst, 16, voff[i], c * kChunkK * 2, 0, 0);
      }
    };
    const int64_t expert_bytes = (int64_t)a.n_tiles * nc * kBlockBytes;
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.wpack + (int64_t)e * expert_bytes), 0, (int)expert_bytes, kRsrcWord3);
    uint4 wq[3][NTP];
    uint32_t sc[3][NTP];
    auto load_w = [&](int slot, int c) {
#pragma unroll
      for (int nt = 0; nt < NTP; ++nt) {
        const uint32_t blk = (uint32_t)((tile_ld + nt) * nc + c) * kBlockBytes;
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, lane * 16, blk, kStreamAux);
        wq[slot][nt] = make_uint4(v[0], v[1], v[2], v[3]);
        sc[slot][nt] = __builtin_amdgcn_raw_buffer_load_b16(wres, kBlockWeightBytes + lane * 2, blk, 0);
      }
    };
    // Dequantise MFMA step st of the chunk in weight slot `slot` into stage
    // `stage` of the A ring (tiles of a clamped re-read land in the slots of
    // the slice's last tiles with the same values, or past n_tiles where no
    // consumer reads them).
    auto produce = [&](int slot, int st, int stage) {
#pragma unroll
      for (int nt = 0; nt < NTP; ++nt) {
        const bf16x8_t w = dequant_word(word_of(wq[slot][nt], st), dq_scale(sc[slot][nt]));
        *reinterpret_cast<bf16x8_t*>(afrag(stage, pw * NTP + nt)) = w;
      }
    };
    dma_x(0);
    load_w(0, 0);
    load_w(1, 1);
    produce(0, 0, 0);
    produce(0, 1, 1);
    // x(0) landed (only w(1) may still be in flight), A stages 0 and 1 written
    pc_barrier<wait_vm_lds<kWLoads>()>();
    // Chunk c in weight slot cs = c % 3.  Step st dequantises step 4c + st + 2
    // into ring stage (4c + st + 2) % 3 = (cs + st + 2) % 3.
    auto chunk = [&](int cs, int c) {
      if (c >= nc) return;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st == 0) {
          dma_x(c + 1 < nc ? c + 1 : nc - 1);                     // into the stage chunk c-1 used
          load_w((cs + 2) % 3, c + 2 < nc ? c + 2 : nc - 1);      // into the slot chunk c-1 used
        }
        if (4 * c + st + 2 < 4 * nc) {
          if (st < 2) produce(cs, st + 2, (cs + st + 2) % 3);
          else produce((cs + 1) % 3, st - 2, (cs + st + 2) % 3);
        }
        if (st == 3)
          pc_barrier<wait_vm_lds<kWLoads>()>();  // x(c+1) landed: only w(c+2) may be in flight
        else
          pc_barrier<kWaitLds>();                // A writes done
      }
    };
    for (int c = 0; c < nc; c += 3) {
      chunk(0, c);
      chunk(1, c + 1);
      chunk(2, c + 2);
    }
    // drain everything (the clamped prefetches) before the next item
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  // ------------------------------ consumer ------------------------------
  const int tile0 = ng * kSliceTiles + wave * NTC;
  const bool live = tile0 < a.n_tiles;
  f32x4_t acc[NTC][MG];
#pragma unroll
  for (int nt = 0; nt < NTC; ++nt)
#pragma unroll
    for (int g = 0; g < MG; ++g) acc[nt][g] = zero4;
  uint32_t boff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st)
    boff[st] = (uint32_t)(col * 256 + (((q * 4 + st) ^ swz(col)) * 16));
  auto bread = [&](const uint8_t* xb, int st, int g) {
    return *reinterpret_cast<const bf16x8_t*>(xb + boff[st] + g * 16 * 256);
  };
  auto aread = [&](int stage, bf16x8_t (&av)[NTC]) {
#pragma unroll
    for (int nt = 0; nt < NTC; ++nt)
      av[nt] = *reinterpret_cast<const bf16x8_t*>(afrag(stage, wave * NTC + nt));
  };
  pc_barrier<kWaitLds>();  // the producers' prologue
  bf16x8_t av[NTC], an[NTC];
  aread(0, av);
  // Step 4c + st reads ring stage (4c + st) % 3; the next step's A (written
  // a step ago) is read during this step, ahead of its use.
  int stage = 0;  // (4c) % 3
  for (int c = 0; c < nc; ++c) {
    const uint8_t* xb = xbuf + (c & 1) * kXBufBytes;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int next = stage == 2 ? 0 : stage + 1;
      if (4 * c + st + 1 < 4 * nc) aread(next, an);
      bf16x8_t bwin[3];
      bwin[0] = bread(xb, st, 0);
      if (MG > 1) bwin[1] = bread(xb, st, 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < MG; ++g) {
        if (g + 2 < MG) bwin[(g + 2) % 3] = bread(xb, st, g + 2);
        const bf16x8_t bv = bwin[g % 3];
#pragma unroll
        for (int nt = 0; nt < NTC; ++nt)
          acc[nt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[nt], bv, acc[nt][g], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // keep the B reads two groups ahead, no further
      }
#pragma unroll
      for (int nt = 0; nt < NTC; ++nt) av[nt] = an[nt];
      stage = next;
      pc_barrier<kWaitLds>();  // this step's LDS reads done
    }
  }
  if (!live) return;
  if (!a.gate_up) {
    store_down_pairs<NTC, MG>(a, acc, dstrow, roww, tile0, q, col);
    return;
  }
#pragma unroll
  for (int g = 0; g < MG; ++g) {
    const int64_t dr = dstrow[g * 16 + col];
#pragma unroll
    for (int nt = 0; nt < NTC; ++nt) {
      if (dr < 0) continue;
      const f32x4_t v = acc[nt][g];
      const int f0 = (tile0 + nt) * 8 + 2 * q;
      *reinterpret_cast<uint32_t*>(a.out + dr * (int64_t)a.out_ld + f0) =
          pk_bf16(silu_mul(v[0], v[1]), silu_mul(v[2], v[3]));
    }
  }
}

__global__ __launch_bounds__(64 * kPcWaves) void gemm_tile_pc(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* xbuf = smem;                                                   // [2][192][256 B]
  uint8_t* abuf = smem + kPcXStages * kXBufBytes;                         // [3][16][64][16 B]
  int32_t* srcoff = reinterpret_cast<int32_t*>(abuf + kPcAStages * kPcAStepBytes);  // [192]
  int64_t* dstrow = reinterpret_cast<int64_t*>(srcoff + kMaxGroups * 16);           // [192]
  float* roww = reinterpret_cast<float*>(dstrow + kMaxGroups * 16);                 // [192]
  const int tid = threadIdx.x;
  const int nslices = a.items_per_tile;
  // XCD-aware item order as in gemm_tile.
  const int G = gridDim.x < kXcds ? (int)gridDim.x : kXcds;
  const int xg = blockIdx.x % G;
  const int nloc = (gridDim.x + G - 1 - xg) / G;
  const int lidx = blockIdx.x / G;
  for (int g = xg; g < kTileGroups; g += G)
    for (int j = lidx, t0 = a.status->group_start[g],
             n_items = (a.status->group_start[g + 1] - t0) * nslices;
         j < n_items; j += nloc) {
      const TileDesc td = a.tiles[t0 + j / nslices];
      const int ng = j % nslices;
      const int e = td.expert;
      const int nrows = td.nrows < kMaxGroups * 16 ? td.nrows : kMaxGroups * 16;
      if (tid < kMaxGroups * 16) {
        const int m = tid;
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
        roww[m] = (dr >= 0 && !a.gate_up && a.row_weights != nullptr) ? a.row_weights[dr] : 1.0f;
      }
      __syncthreads();
      switch ((nrows + 15) >> 4) {
        case 0: break;
#define CHORD_PC_CASE(MG) \
  case MG: run_item_pc<MG>(a, xbuf, abuf, srcoff, dstrow, roww, td, ng); break;
        CHORD_PC_CASE(1) CHORD_PC_CASE(2) CHORD_PC_CASE(3) CHORD_PC_CASE(4)
        CHORD_PC_CASE(5) CHORD_PC_CASE(6) CHORD_PC_CASE(7) CHORD_PC_CASE(8)
        CHORD_PC_CASE(9) CHORD_PC_CASE(10) CHORD_PC_CASE(11)
#undef CHORD_PC_CASE
        default: run_item_pc<12>(a, xbuf, abuf, srcoff, dstrow, roww, td, ng); break;
      }
      __syncthreads();  // row maps, token stages and A ring reused by the next item
    }
}

// ---------------------------------------------------------------------------
// Short-K variant (K <= 256, e.g. the down GEMM of an 8-way intermediate
// split): the whole token tile (all K) is staged in LDS once per work item,
// and the item covers `slices_per_item` consecutive 256-row slices.  The
// weights of a slice (NC chunks x 4 tiles per wave) sit in registers, double
// buffered by slice: the next slice's weights load while this slice
// computes.  No barrier is needed after staging.
// ---------------------------------------------------------------------------
template <int MG, int NC>
__device__ __forceinline__ void run_item_shortk(const GemmArgs& a, uint8_t* xbuf,
                                                const int32_t* srcoff, const int64_t* dstrow,
                                                const float* roww, int e, int ng0, int ns) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int col = lane & 15;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  // Stage all NC chunks of the token tile (same DMA layout as run_item).
  {
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.bsrc, 0, (int)a.bsrc_bytes, kRsrcWord3);
    const int rsub = 4 * wave + q;
    const uint32_t pbytes = (uint32_t)((col ^ swz(rsub)) * 16);
#pragma unroll
    for (int i = 0; i < MG; ++i) {
      const uint32_t voff = (uint32_t)srcoff[rsub + 16 * i] + pbytes;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint8_t* dst = xbuf + c * kXBufBytes + (wave + 4 * i) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xres, (__attribute__((address_space(3))) void*)dst, 16, voff, c * kChunkK * 2, 0, 0);
      }
    }
  }

  const int64_t expert_bytes = (int64_t)a.n_tiles * NC * kBlockBytes;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.wpack + (int64_t)e * expert_bytes), 0, (int)expert_bytes, kRsrcWord3);
  auto tile_first = [&](int s) { return ((ng0 + s) * kWaves + wave) * kNT; };
  uint4 wq[2][NC][kNT];
  uint32_t sc[2][NC][kNT];
  auto load_slice = [&](int slot, int s) {
    int t0 = tile_first(s);
    if (t0 > a.n_tiles - kNT) t0 = a.n_tiles - kNT;  // past the end: re-read, store nothing
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const uint32_t blk = (uint32_t)((t0 + nt) * NC + c) * kBlockBytes;
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, lane * 16, blk, kStreamAux);
        wq[slot][c][nt] = make_uint4(v[0], v[1], v[2], v[3]);
        sc[slot][c][nt] =
            __builtin_amdgcn_raw_buffer_load_b16(wres, kBlockWeightBytes + lane * 2, blk, 0);
      }
  };

  f32x4_t acc[kNT][MG];
  uint32_t boff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st)
    boff[st] = (uint32_t)(col * 256 + (((q * 4 + st) ^ swz(col)) * 16));

  // One slice: NC chunks x 4 MFMA steps over MG token groups, B reads two
  // groups ahead, the next step's dequantisation spread over the groups
  // (the last step of the slice prepares nothing: the next slice starts by
  // dequantising its first step).
  auto compute_slice = [&](int slot) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int g = 0; g < MG; ++g) acc[nt][g] = zero4;
    bf16x8_t av[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) av[nt] = dequant_word(wq[slot][0][nt].x, dq_scale(sc[slot][0][nt]));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint8_t* xb = xbuf + c * kXBufBytes;
      DqScale ks[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) ks[nt] = dq_scale(sc[slot][c][nt]);
      bf16x8_t bwin[3];
      bwin[0] = *reinterpret_cast<const bf16x8_t*>(xb + boff[0]);
      bwin[1] = *reinterpret_cast<const bf16x8_t*>(xb + (MG > 1 ? boff[0] + 16 * 256 : boff[1]));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8_t an[kNT];
#pragma unroll
        for (int g = 0; g < MG; ++g) {
          const int idx = st * MG + g;
          const int ahead = idx + 2;
          if (ahead < 4 * MG)
            bwin[ahead % 3] = *reinterpret_cast<const bf16x8_t*>(
                xb + boff[ahead / MG] + (ahead % MG) * 16 * 256);
          const bf16x8_t bv = bwin[idx % 3];
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            acc[nt][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[nt], bv, acc[nt][g], 0, 0, 0);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            if (nt * MG / kNT != g) continue;
            if (st < 3) an[nt] = dequant_word(word_of(wq[slot][c][nt], st + 1), ks[nt]);
            else if (c + 1 < NC)
              an[nt] = dequant_word(wq[slot][c + 1][nt].x, dq_scale(sc[slot][c + 1][nt]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (st < 3 || c + 1 < NC) {
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) av[nt] = an[nt];
        }
      }
    }
  };

  auto epilogue = [&](int s) {
    const int tile0 = tile_first(s);
    if (tile0 >= a.n_tiles) return;
    if (!a.gate_up) {
      store_down_pairs<kNT, MG>(a, acc, dstrow, roww, tile0, q, col);
      return;
    }
#pragma unroll
    for (int g = 0; g < MG; ++g) {
      const int64_t dr = dstrow[g * 16 + col];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        if (dr < 0) continue;
        const f32x4_t v = acc[nt][g];
        const int f0 = (tile0 + nt) * 8 + 2 * q;
        *reinterpret_cast<uint32_t*>(a.out + dr * (int64_t)a.out_ld + f0) =
            pk_bf16(silu_mul(v[0], v[1]), silu_mul(v[2], v[3]));
      }
    }
  };

  load_slice(0, 0);
  __syncthreads();  // fenced: the token DMA has landed for every wave
  // Slices in pairs so the weight buffer index is compile-time; the next
  // slice's load is clamped to the last one (a redundant, in-bounds re-read).
  for (int s = 0; s < ns; s += 2) {
    load_slice(1, s + 1 < ns ? s + 1 : ns - 1);
    __builtin_amdgcn_sched_barrier(0);
    compute_slice(0);
    __builtin_amdgcn_sched_barrier(0);
    epilogue(s);
    if (s + 1 >= ns) break;
    load_slice(0, s + 2 < ns ? s + 2 : ns - 1);
    __builtin_amdgcn_sched_barrier(0);
    compute_slice(1);
    __builtin_amdgcn_sched_barrier(0);
    epilogue(s + 1);
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // drain before the LDS is reused
}

__global__ __launch_bounds__(256) void gemm_tile_shortk(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* xbuf = smem;                                                  // [NC][192][256 B]
  int32_t* srcoff = reinterpret_cast<int32_t*>(smem + kStages * kXBufBytes);
  int64_t* dstrow = reinterpret_cast<int64_t*>(srcoff + kMaxGroups * 16);
  float* roww = reinterpret_cast<float*>(dstrow + kMaxGroups * 16);
  const int tid = threadIdx.x;
  const int nslices = a.items_per_tile;
  const int S = a.slices_per_item;
  const int ipt = (nslices + S - 1) / S;  // items per tile
  const int G = gridDim.x < kXcds ? (int)gridDim.x : kXcds;
  const int xg = blockIdx.x % G;
  const int nloc = (gridDim.x + G - 1 - xg) / G;
  const int lidx = blockIdx.x / G;

  for (int g = xg; g < kTileGroups; g += G)
    for (int j = lidx, t0 = a.status->group_start[g],
             n_items = (a.status->group_start[g + 1] - t0) * ipt;
         j < n_items; j += nloc) {
      const TileDesc td = a.tiles[t0 + j / ipt];
      const int ng0 = (j % ipt) * S;
      const int ns = nslices - ng0 < S ? nslices - ng0 : S;
      const int e = td.expert;
      const int nrows = td.nrows < kMaxGroups * 16 ? td.nrows : kMaxGroups * 16;
      if (tid < kMaxGroups * 16) {
        const int m = tid;
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
        roww[m] = (dr >= 0 && !a.gate_up && a.row_weights != nullptr) ? a.row_weights[dr] : 1.0f;
      }
      __syncthreads();
#define CHORD_SHORTK(NC)                                                                   \
  switch ((nrows + 31) >> 5) {                                                             \
    case 0: break;                                                                         \
    case 1: run_item_shortk<2, NC>(a, xbuf, srcoff, dstrow, roww, e, ng0, ns); break; \
    case 2: run_item_shortk<4, NC>(a, xbuf, srcoff, dstrow, roww, e, ng0, ns); break; \
    case 3: run_item_shortk<6, NC>(a, xbuf, srcoff, dstrow, roww, e, ng0, ns); break; \
    case 4:                                                                                \
      run_item_shortk<8, NC>(a, xbuf, srcoff, dstrow, roww, e, ng0, ns); \
      break;                                                                               \
    case 5:                                                                                \
      run_item_shortk<10, NC>(a, xbuf, srcoff, dstrow, roww, e, ng0, ns); \
      break;                                                                               \
    default:                                                                               \
      run_item_shortk<12, NC>(a, xbuf, srcoff, dstrow, roww, e, ng0, ns); \
      break;                                                                               \
  }
      if (a.n_chunks == 1) {
        CHORD_SHORTK(1)
      } else {
        CHORD_SHORTK(2)
      }
#undef CHORD_SHORTK
      __syncthreads();  // row maps and LDS reuse by the next item
    }
}

// ---------------------------------------------------------------------------
// K-split fixup: one workgroup per (split tile, 256-row slice, weight tile t
// of the slice); wave w handles the token groups g = w, w + 4, w + 8 of the
// tile.  Lane (q, col) reads its f32x4 of every part (all loads in flight
// together), adds them in part order and applies the same epilogue as the
// GEMM.  The parts stored the layout index (t * MG + g) * 64 + lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_split_fixup(GemmArgs a) {
  const int nslices = a.items_per_tile;
  const int t = blockIdx.x % kSliceTiles;
  const int ng = (blockIdx.x / kSliceTiles) % nslices;
  const int sid = blockIdx.x / (kSliceTiles * nslices);
  if (sid >= a.status->nsplit) return;
  const int tw = ng * kSliceTiles + t;  // tile of the GEMM
  if (tw >= a.n_tiles) return;
  const TileDesc td = a.split_tiles[sid];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4, col = lane & 15;
  const int nrows = td.nrows < kMaxGroups * 16 ? td.nrows : kMaxGroups * 16;
  const int MG = (nrows + 15) >> 4;
  for (int g = wave; g < MG; g += 4) {
    const int m = g * 16 + col;
    int64_t dr = -1;
    if (m < nrows) dr = map_row(a, td.expert, (int64_t)td.row_begin + m).dst;
    f32x4_t part[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      part[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (p < td.ksplit)
        part[p] = reinterpret_cast<const f32x4_t*>(
            a.partials + (size_t)(td.pbase + (p * a.max_slices + ng) * MG) *
                             kPartialSlotFloats)[(t * MG + g) * 64 + lane];
    }
    if (dr < 0) continue;
    f32x4_t v = part[0];
#pragma unroll
    for (int p = 1; p < 4; ++p)
      if (p < td.ksplit) v += part[p];
    if (a.gate_up) {
      const int f0 = tw * 8 + 2 * q;
      *reinterpret_cast<uint32_t*>(a.out + dr * (int64_t)a.out_ld + f0) =
          pk_bf16(silu_mul(v[0], v[1]), silu_mul(v[2], v[3]));
    } else {
      const float rw = a.row_weights != nullptr ? a.row_weights[dr] : 1.0f;
      const int n0 = tw * 16 + 4 * q;
      *reinterpret_cast<uint2*>(a.out + dr * (int64_t)a.out_ld + n0) =
          make_uint2(pk_bf16(v[0] * rw, v[1] * rw), pk_bf16(v[2] * rw, v[3] * rw));
    }
  }
}

}  // namespace

hipError_t launch_tile_split_fixup(const GemmArgs& a, hipStream_t stream) {
  const int slices = a.items_per_tile;
  hipLaunchKernelGGL(tile_split_fixup, dim3((unsigned)(kMaxSplitTiles * slices * kSliceTiles)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_tile(const GemmArgs& a, int grid, hipStream_t stream) {
  if (a.n_chunks <= 2) {  // short K: token tile resident, several slices per item
    static const int per_cu_s = [] {
      hipFuncSetAttribute((const void*)gemm_tile_shortk,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
      return blocks_per_cu(gemm_tile_shortk, 256, kLdsBytes);
    }();
    const int cap = per_cu_s * (a.num_cus > 0 ? a.num_cus : 256);
    hipLaunchKernelGGL(gemm_tile_shortk, dim3(grid > cap ? cap : grid), dim3(256), kLdsBytes,
                       stream, a);
    return hipGetLastError();
  }
  const int cus = a.num_cus > 0 ? a.num_cus : 256;
  if (a.tile_waves == 2) {  // producer/consumer form (no K split)
    static const int per_cu_pc = [] {
      hipFuncSetAttribute((const void*)gemm_tile_pc, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kPcLdsBytes);
      return blocks_per_cu(gemm_tile_pc, 64 * kPcWaves, kPcLdsBytes);
    }();
    if (grid > per_cu_pc * cus) grid = per_cu_pc * cus;
    hipLaunchKernelGGL(gemm_tile_pc, dim3(grid), dim3(64 * kPcWaves), kPcLdsBytes, stream, a);
    return hipGetLastError();
  }
  if (a.tile_waves == 8) {
    static const int per_cu8 = [] {
      hipFuncSetAttribute((const void*)gemm_tile<8>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kLdsBytes);
      return blocks_per_cu(gemm_tile<8>, 512, kLdsBytes);
    }();
    if (grid > per_cu8 * cus) grid = per_cu8 * cus;
    hipLaunchKernelGGL(gemm_tile<8>, dim3(grid), dim3(512), kLdsBytes, stream, a);
    return hipGetLastError();
  }
  static const int per_cu = [] {
    hipFuncSetAttribute((const void*)gemm_tile<4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)kLdsBytes);
    return blocks_per_cu(gemm_tile<4>, 256, kLdsBytes);
  }();
  if (grid > per_cu * cus) grid = per_cu * cus;
  hipLaunchKernelGGL(gemm_tile<4>, dim3(grid), dim3(256), kLdsBytes, stream, a);
  return hipGetLastError();
}

}  // namespace chord
