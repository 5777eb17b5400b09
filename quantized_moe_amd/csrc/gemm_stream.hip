// Weight-streaming expert GEMM for few rows per expert (decode, TP slices,
// masked tails): the layer is HBM-bound there, so every workgroup streams its
// packed weight tiles straight from HBM into registers, dequantises them and
// feeds v_mfma_f32_16x16x32_bf16 with the weights as the A operand (16 weight
// rows) and up to MT x 16 tokens as B operands.
//
// Dequantisation is exact: each weight becomes bf16_rne((q - 8) * s), the
// subtract-then-scale order with one bf16 rounding that the pages keep in
// their fused nibble extraction ("vLLM x Novita AI: Chord W4A16 INT4 MoE
// Kernel fuer Kimi K2.x", section "H200 und Blackwell indexierter Decode"):
//   * one shift + one mask-or turns two codes into the fp16 halves 1024 + q;
//   * v_fma_mix_f32 computes (1024 + q) * s - 1032 * s with one rounding,
//     which is exactly (q - 8) * s (at most 11 significant bits);
//   * v_cvt_pk_bf16_f32 rounds two of them to bf16, nearest-even.
#include <type_traits>

#include "device_common.h"

namespace chord {
namespace {

// Buffer resource word 3 for raw (untyped) buffer accesses on gfx9-family
// chips; out-of-range offsets read as zero.
constexpr int kRsrcWord3 = 0x00020000;
// Offset that lies past every buffer resource used here (sizes < 3 GiB).
constexpr uint32_t kNoRow = 0xC0000000u;
// Cache policy of the one-touch weight stream: non-temporal.
constexpr int kStreamAux = 2;

// Per-scale constants of the exact dequantisation.  Codes sitting in bits 0..3
// of a 16-bit half read as fp16 1024 + q; codes in bits 4..7 read as
// 1024 + 16q (no shift needed).  Then
//   (1024 + q) * s - 1032 s  =  (1024 + 16q) * (s / 16) - 72 s  =  (q - 8) s,
// each exact in one fma (the product has at most 11 significant bits).
struct DqScale {
  float s, c, s16, c16;
};
__device__ __forceinline__ DqScale dq_scale(uint32_t bits16) {
  const float s = bf16_to_f32(bits16);
  return DqScale{s, -1032.0f * s, 0.0625f * s, -72.0f * s};
}

// Four packed words (32 codes of one row, one scale group) -> 4 x 8 bf16
// weights bf16_rne((q - 8) * s).  Staged so that no result is consumed by the
// next instruction: masks, then fmas, then conversions.
__device__ __forceinline__ void dequant_words(const uint4& wq, const DqScale& k, uint32_t mlo,
                                              uint32_t mhi, uint32_t magic, bf16x8_t out[4]) {
  const uint32_t w[4] = {wq.x, wq.y, wq.z, wq.w};
  uint32_t m[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w8 = w[i] >> 8;
    m[i][0] = and_or(w[i], mlo, magic);  // k = 0, 1     (1024 + q)
    m[i][1] = and_or(w[i], mhi, magic);  // k = 2, 3     (1024 + 16q)
    m[i][2] = and_or(w8, mlo, magic);    // k = 4, 5
    m[i][3] = and_or(w8, mhi, magic);    // k = 6, 7
  }
  float f[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const half2_t h = __builtin_bit_cast(half2_t, m[i][v]);
      const float sv = (v & 1) ? k.s16 : k.s;
      const float cv = (v & 1) ? k.c16 : k.c;
      f[i][2 * v] = __builtin_fmaf((float)h[0], sv, cv);
      f[i][2 * v + 1] = __builtin_fmaf((float)h[1], sv, cv);
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    out[i] = __builtin_bit_cast(
        bf16x8_t, make_uint4(pk_bf16(f[i][0], f[i][1]), pk_bf16(f[i][2], f[i][3]),
                             pk_bf16(f[i][4], f[i][5]), pk_bf16(f[i][6], f[i][7])));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Row mapping of one tile row: the B source row and the output row, or -1.
struct RowMap {
  int64_t src;
  int64_t dst;
};

__device__ __forceinline__ RowMap map_row(const GemmArgs& a, int expert, int64_t R) {
  RowMap m{-1, -1};
  if (a.layout == kIndexed) {
    const int64_t f = a.sorted_ids[R];
    if (f < 0 || f >= a.n_flat) return m;
    if (a.gate_up) {
      m.src = f / a.topk;
      m.dst = R;
    } else {
      m.src = a.h_by_slot ? f : R;
      m.dst = f;
    }
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

// Number of tiles (device tile list, or one tile per alignment block).
__device__ __forceinline__ int num_tiles(const GemmArgs& a) {
  if (a.tiles != nullptr) return a.status->ntiles;
  int64_t ntpp = *a.ntpp;
  ntpp = ntpp < 0 ? 0 : (ntpp > a.max_padded ? a.max_padded : ntpp);
  return (int)(ntpp / a.block_m);
}

// Tile `ti`; expert -1 means "skip" (an out-of-range expert id).
__device__ __forceinline__ TileDesc get_tile(const GemmArgs& a, int ti) {
  if (a.tiles != nullptr) return a.tiles[ti];
  const int e = a.expert_ids[ti];
  TileDesc t{e, ti * a.block_m, a.block_m, 0, 1, 0, 0, 0};
  if (e < 0 || e >= a.num_experts) t.expert = -1;
  return t;
}

// Routing tables of a routed call, built in LDS by every workgroup of the
// gate_up launch from topk_ids (T * k <= kRoutedMaxSlots): the local slots
// grouped by expert (`list`), each expert's first and past-the-end row and
// first tile in that list, and the expert of every tile of `tok` rows.  The
// order of the slots inside an expert's group is not fixed: each output row
// depends only on its own slot (h and y are stored per flat slot), so which
// rows share a tile changes no value.  Workgroup 0 also stores the list and
// the tiles for the down launch.
struct Routes {
  const int* rowoff;   // [E]: first row of each active expert in `list`
  const int* rowend;   // [E]: past its last row
  const int* tileoff;  // [E]: its first tile
  const int* list;     // [n]
  const int* tile_e;   // [tiles]
  int ntiles;
  int nrows;
  int tok;
  __device__ TileDesc tile(int ti) const {
    const int e = tile_e[ti];
    const int r0 = rowoff[e] + (ti - tileoff[e]) * tok;
    const int nr = min(tok, rowend[e] - r0);
    return TileDesc{e, r0, nr, 0, 1, 0, 0, 0};
  }
};

__device__ Routes build_routes(const GemmArgs& a, int* lds, int tok) {
  __shared__ int scan_tmp[17 * 2];
  __shared__ int totals[2];
  const int E = a.num_experts, n = a.route_n;
  const int tid = threadIdx.x, nth = blockDim.x;
  int* rowoff = lds;
  int* rowend = rowoff + E;
  int* tileoff = rowend + E;
  int* list = tileoff + E;
  int* tile_e = list + n;
  int* cnt = tile_e + n;  // [E + 2], general path only
  int nrows, ntiles;
  if (n <= 64) {
    // One wave, one ballot per distinct local expert (experts in the order of
    // their first slot): no LDS atomics, no scan.
    if (tid < 64) {
      const int idv = tid < n ? a.route_ids[tid] - a.route_eb : -1;
      const bool loc = tid < n && (unsigned)idv < (unsigned)E;
      uint64_t rem = __builtin_amdgcn_ballot_w64(loc);
      int rows = 0, tiles = 0;
      while (rem != 0) {
        const int leader = __builtin_ctzll(rem);
        const int e = __builtin_amdgcn_readlane(idv, leader);
        const uint64_t same = __builtin_amdgcn_ballot_w64(loc && idv == e);
        rem &= ~same;
        const int c = __builtin_popcountll(same);
        const int nt = (c + tok - 1) / tok;
        if (tid == 0) {
          rowoff[e] = rows;
          rowend[e] = rows + c;
          tileoff[e] = tiles;
        }
        if ((same >> tid) & 1ull)
          list[rows + __builtin_popcountll(same & ((1ull << tid) - 1ull))] = tid;
        if (tid < nt) tile_e[tiles + tid] = e;
        rows += c;
        tiles += nt;
      }
      if (tid == 0) {
        totals[0] = rows;
        totals[1] = tiles;
      }
    }
    __syncthreads();
    nrows = totals[0];
    ntiles = totals[1];
  } else {
    for (int e = tid; e < E; e += nth) cnt[e] = 0;
    // Local expert of this thread's slots tid + nth * u, read in batches of
    // kIdBatch independent loads (one memory round trip per batch) and kept
    // for the scatter pass.
    constexpr int kIdBatch = 8;
    const int nb = (n + nth * kIdBatch - 1) / (nth * kIdBatch);  // batches (uniform)
    int ev[kIdBatch];
    auto load_ids = [&](int b) {
#pragma unroll
      for (int u = 0; u < kIdBatch; ++u) {
        const int i = (b * kIdBatch + u) * nth + tid;
        ev[u] = i < n ? a.route_ids[i] - a.route_eb : -1;
      }
    };
    load_ids(0);
    __syncthreads();
    for (int b = 0; b < nb; ++b) {
      if (b > 0) load_ids(b);
#pragma unroll
      for (int u = 0; u < kIdBatch; ++u)
        if ((unsigned)ev[u] < (unsigned)E) atomicAdd(&cnt[ev[u]], 1);
    }
    __syncthreads();
    // Exclusive scans of the row and tile counts: each thread owns a
    // contiguous range of experts, one block scan over the thread sums.
    const int per = (E + nth - 1) / nth;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    int v[2] = {0, 0}, tot[2];
    for (int e = lo; e < hi; ++e) {
      v[0] += cnt[e];
      v[1] += (cnt[e] + tok - 1) / tok;
    }
    block_scan_excl_n<2>(v, scan_tmp, tot);
    {
      int r = v[0], t = v[1];
      for (int e = lo; e < hi; ++e) {
        rowoff[e] = r;
        tileoff[e] = t;
        r += cnt[e];
        rowend[e] = r;
        t += (cnt[e] + tok - 1) / tok;
      }
    }
    __syncthreads();
    for (int b = nb - 1; b >= 0; --b) {  // the last batch is still in registers
      if (b < nb - 1) load_ids(b);
#pragma unroll
      for (int u = 0; u < kIdBatch; ++u)
        if ((unsigned)ev[u] < (unsigned)E)
          list[rowoff[ev[u]] + atomicSub(&cnt[ev[u]], 1) - 1] = (b * kIdBatch + u) * nth + tid;
    }
    for (int e = tid; e < E; e += nth) {
      const int t1 = tileoff[e] + (rowend[e] - rowoff[e] + tok - 1) / tok;
      for (int t = tileoff[e]; t < t1; ++t) tile_e[t] = e;
    }
    __syncthreads();
    nrows = tot[0];
    ntiles = tot[1];
  }
  Routes r{rowoff, rowend, tileoff, list, tile_e, ntiles, nrows, tok};
  if (blockIdx.x == 0) {
    for (int i = tid; i < nrows; i += nth) a.route_list[i] = list[i];
    for (int t = tid; t < ntiles; t += nth) a.route_tiles[t] = r.tile(t);
    if (tid == 0) {
      DevStatus* st = const_cast<DevStatus*>(a.status);
      st->ntiles = ntiles;
      st->error = 0;
    }
  }
  return r;
}

// A workgroup of WK waves owns NT 16-row weight tiles of one expert and up to
// MT*16 rows of one token tile; the waves split K and reduce through LDS.
// Per 128-wide K chunk each lane streams 16 bytes of packed codes and one
// scale per weight tile (one scale group of one row); token rows come from
// global memory (L2-resident).  Persistent: workgroups stride over
// (tile, weight-tile group) items.
template <int NT, int MT, int WK, int PF>
__global__ __launch_bounds__(64 * WK) void gemm_stream(GemmArgs a) {
  extern __shared__ float red[];  // [WK][NT*MT][64][4]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar offsets
  const int q = lane >> 4;
  const int col = lane & 15;
  // Routed gate_up: tiles and rows from the LDS tables (after the K
  // reduction area in dynamic LDS).
  const bool routed = a.route_ids != nullptr;
  Routes rt{};
  if (routed)
    rt = build_routes(a, reinterpret_cast<int*>(red + (WK > 1 ? WK * NT * MT * 64 * 4 : 0)),
                      MT * 16);
  const int n_items = (routed ? rt.ntiles : num_tiles(a)) * a.items_per_tile;
  const int c_lo = (a.n_chunks * wave) / WK;
  const int c_hi = (a.n_chunks * (wave + 1)) / WK;
  const uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.bsrc, 0, (int)a.bsrc_bytes, kRsrcWord3);

  // Weight and token rings, kept across items: while a wave streams the
  // last chunks of an item it already loads the first chunks of its next
  // item into the slots they will use (when its chunk count is a multiple of
  // PF, so the slots line up), and that item then skips its prologue loads.
  const int64_t expert_bytes = (int64_t)a.n_tiles * a.n_chunks * kBlockBytes;
  const bool chain = !a.no_chain && c_hi - c_lo >= PF && (c_hi - c_lo) % PF == 0;
  uint4 wq[PF][NT];
  uint32_t sc[PF][NT];
  uint4 xb[2][MT][4];
  bool primed = false;  // the ring holds this item's first PF chunks already

  // Token row offsets of tile td (lane `col` supplies token col of each
  // 16-row token tile), and the output rows.  Lanes without a token get an
  // out-of-range offset and read zeros (no branch around the loads).
  auto row_maps = [&](const TileDesc& td, uint32_t (&xo)[MT], int64_t (&dr)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + col;
      xo[mt] = kNoRow;
      dr[mt] = -1;
      if (m < td.nrows) {
        RowMap rm;
        if (routed) {  // gate_up of a routed call: h row per flat slot
          const int f = rt.list[td.row_begin + m];
          rm = RowMap{f / a.topk, f};
        } else {
          rm = map_row(a, td.expert, (int64_t)td.row_begin + m);
        }
        if (rm.src >= 0) {
          xo[mt] = (uint32_t)((rm.src * (int64_t)a.K + q * kGroup) * 2);
          dr[mt] = rm.dst;
        }
      }
    }
  };

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int ti = item / a.items_per_tile;
    const int ng = item % a.items_per_tile;
    const TileDesc td = routed ? rt.tile(ti) : get_tile(a, ti);
    const int e = td.expert;
    if (e < 0) {  // uniform over the workgroup
      primed = false;
      continue;
    }

    // B operand rows of this item.
    uint32_t xoff[MT];
    int64_t dst[MT];
    row_maps(td, xoff, dst);

    // Weights: one resource over this expert's packed tiles; the chunk and
    // tile offsets are scalar.
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.wpack + (int64_t)e * expert_bytes), 0, (int)expert_bytes, kRsrcWord3);
    const uint32_t tile0 = (uint32_t)(ng * NT) * a.n_chunks * kBlockBytes;

    // The next item of this workgroup, when the ring can run on into it.
    bool nvalid = false;
    __amdgpu_buffer_rsrc_t wres_n = wres;
    uint32_t tile0_n = tile0;
    uint32_t xoff_n[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xoff_n[mt] = xoff[mt];
    if (chain && item + (int)gridDim.x < n_items) {
      const int item_n = item + (int)gridDim.x;
      const TileDesc tn = routed ? rt.tile(item_n / a.items_per_tile)
                                 : get_tile(a, item_n / a.items_per_tile);
      if (tn.expert >= 0) {
        nvalid = true;
        wres_n = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.wpack + (int64_t)tn.expert * expert_bytes), 0, (int)expert_bytes, kRsrcWord3);
        tile0_n = (uint32_t)((item_n % a.items_per_tile) * NT) * a.n_chunks * kBlockBytes;
        int64_t dn[MT];
        row_maps(tn, xoff_n, dn);
      }
    }

    f32x4_t acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = zero4;

    auto load_w = [&](int p, int c) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t blk = tile0 + (uint32_t)(nt * a.n_chunks + c) * kBlockBytes;
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, lane * 16, blk, kStreamAux);
        wq[p][nt] = make_uint4(v[0], v[1], v[2], v[3]);
        sc[p][nt] = __builtin_amdgcn_raw_buffer_load_b16(wres, kBlockWeightBytes + lane * 2, blk, 0);
      }
    };
    // Token fragments of chunk index t of this item (t >= c_hi: chunk
    // c_lo + t - c_hi of the next item, or the last chunk again when there
    // is none: a redundant, in-bounds load).
    auto load_x = [&](int p, int t) {
      const bool cross = t >= c_hi;
      const int c = !cross ? t : (nvalid ? c_lo + (t - c_hi) : c_hi - 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint32_t xo = cross && nvalid ? xoff_n[mt] : xoff[mt];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xres, xo, c * kChunkK * 2 + s * 16, 0);
          xb[p][mt][s] = make_uint4(v[0], v[1], v[2], v[3]);
        }
      }
    };
    // Chunk in weight slot p.  Once tile nt is dequantised its slot
    // registers are free, so the load of tile nt of chunk index `refill`
    // (when do_refill; past c_hi it is the next item's chunk, as in load_x)
    // goes out right there instead of after the whole chunk: half a chunk
    // more latency cover at no register cost.
    auto compute = [&](int p, int xp, int refill, auto do_refill) {
      const bool cross = refill >= c_hi;
      const int rc = !cross ? refill : (nvalid ? c_lo + (refill - c_hi) : c_hi - 1);
      const __amdgpu_buffer_rsrc_t rres = cross && nvalid ? wres_n : wres;
      const uint32_t rt0 = cross && nvalid ? tile0_n : tile0;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8_t av[4];
        dequant_words(wq[p][nt], dq_scale(sc[p][nt]), kMaskLo, kMaskHi, kMagic, av);
        if constexpr (decltype(do_refill)::value) {
          const uint32_t blk = rt0 + (uint32_t)(nt * a.n_chunks + rc) * kBlockBytes;
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rres, lane * 16, blk, kStreamAux);
          wq[p][nt] = make_uint4(v[0], v[1], v[2], v[3]);
          sc[p][nt] = __builtin_amdgcn_raw_buffer_load_b16(rres, kBlockWeightBytes + lane * 2, blk, 0);
          __builtin_amdgcn_sched_barrier(0);  // keep the refill where it is issued
        }
        // No liveness branch around the MFMA: a dead token tile multiplies
        // zeros, which costs less than breaking the instruction stream.
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[st], as_bf16x8(xb[xp][mt][st]),
                                                                  acc[nt][mt], 0, 0, 0);
      }
    };

    // PF is even, so chunk c_lo + i uses weight slot i % PF and token slot
    // i % 2, both compile-time inside the unrolled body.
    // The steady-state body is straight-line: prefetch targets past the last
    // chunk are the next item's first chunks (or the last chunk again, a
    // redundant, in-bounds load), so the compiler can count outstanding
    // loads exactly instead of waiting for all of them.
    static_assert(PF % 2 == 0, "even prefetch depth");
    if (c_lo < c_hi) {
      const int c_last = c_hi - 1;
      if (!primed) {
        load_x(0, c_lo);
#pragma unroll
        for (int p = 0; p < PF; ++p) load_w(p, min(c_lo + p, c_last));
      }
      int c = c_lo;
      for (; c + PF <= c_hi; c += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
          load_x((p + 1) & 1, c + p + 1);
          compute(p, p & 1, c + p + PF, std::true_type{});
        }
      }
#pragma unroll
      for (int p = 0; p < PF - 1; ++p) {
        if (c + p < c_hi) {
          load_x((p + 1) & 1, min(c + p + 1, c_last));
          compute(p, p & 1, 0, std::false_type{});
        }
      }
    }
    primed = nvalid;  // chain holds: the main loop issued the next item's first chunks

    // Cross-wave K reduction: wave w finishes the (nt, mt) pairs with
    // (nt * MT + mt) % WK == w.
    if (WK > 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<f32x4_t*>(red + (((size_t)wave * NT * MT + nt * MT + mt) * 64 + lane) *
                                                4) = acc[nt][mt];
      __syncthreads();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if ((nt * MT + mt) % WK != wave) continue;
          f32x4_t sum = zero4;
          for (int w = 0; w < WK; ++w)
            sum += *reinterpret_cast<const f32x4_t*>(
                red + (((size_t)w * NT * MT + nt * MT + mt) * 64 + lane) * 4);
          acc[nt][mt] = sum;
        }
    }

    // Epilogue: lane holds rows 4q..4q+3 of weight tile nt for token `col`.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int tw = ng * NT + nt;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (WK > 1 && (nt * MT + mt) % WK != wave) continue;
        if (dst[mt] < 0) continue;
        const f32x4_t v = acc[nt][mt];
        if (a.gate_up) {
          const int f0 = tw * 8 + 2 * q;
          *reinterpret_cast<uint32_t*>(a.out + dst[mt] * (int64_t)a.out_ld + f0) =
              pk_bf16(silu_mul(v[0], v[1]), silu_mul(v[2], v[3]));
        } else {
          const int n0 = tw * 16 + 4 * q;
          const float rw = a.row_weights != nullptr ? a.row_weights[dst[mt]] : 1.0f;
          *reinterpret_cast<uint2*>(a.out + dst[mt] * (int64_t)a.out_ld + n0) =
              make_uint2(pk_bf16(v[0] * rw, v[1] * rw), pk_bf16(v[2] * rw, v[3] * rw));
        }
      }
    }
    if (WK > 1) __syncthreads();  // LDS reuse by the next item
  }
}

// Short-K variant (K <= 256, one wave per item, no K split): an item covers
// one token tile and `slices_per_item` consecutive groups of NT weight tiles.
// The token fragments of all K are loaded once per item; the weight loads run
// through a four-slot ring over the item's (group, chunk) steps without a
// break at group boundaries, each group ending with its epilogue.  Row weights
// are read before the loop so no epilogue waits on a global load while
// weight loads are in flight.
template <int NT, int MT, int NC>
__global__ __launch_bounds__(64) void gemm_stream_shortk(GemmArgs a) {
  constexpr int PF = 4;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int col = lane & 15;
  const int n_groups = a.n_tiles / NT;
  const int G = a.slices_per_item;
  const int ipt = a.items_per_tile;
  const int n_items = num_tiles(a) * ipt;
  const uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.bsrc, 0, (int)a.bsrc_bytes, kRsrcWord3);

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int ti = item / ipt;
    const int g0 = (item % ipt) * G;
    const TileDesc td = get_tile(a, ti);
    const int e = td.expert;
    if (e < 0) continue;
    const int ng = n_groups - g0 < G ? n_groups - g0 : G;
    const int nsteps = ng * NC;

    uint32_t xoff[MT];
    int64_t dst[MT];
    float rw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + col;
      xoff[mt] = kNoRow;
      dst[mt] = -1;
      rw[mt] = 1.0f;
      if (m < td.nrows) {
        const RowMap rm = map_row(a, e, (int64_t)td.row_begin + m);
        if (rm.src >= 0) {
          xoff[mt] = (uint32_t)((rm.src * (int64_t)a.K + q * kGroup) * 2);
          dst[mt] = rm.dst;
          if (!a.gate_up && a.row_weights != nullptr) rw[mt] = a.row_weights[rm.dst];
        }
      }
    }
    uint4 xb[NC][MT][4];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4_t v =
              __builtin_amdgcn_raw_buffer_load_b128(xres, xoff[mt], c * kChunkK * 2 + s * 16, 0);
          xb[c][mt][s] = make_uint4(v[0], v[1], v[2], v[3]);
        }

    const int64_t expert_bytes = (int64_t)a.n_tiles * NC * kBlockBytes;
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.wpack + (int64_t)e * expert_bytes), 0, (int)expert_bytes, kRsrcWord3);
    uint4 wq[PF][NT];
    uint32_t sc[PF][NT];
    // Step i: group g0 + i / NC, chunk i % NC (clamped to the last step).
    auto step_blk = [&](int i, int nt) {
      const int ic = i < nsteps ? i : nsteps - 1;
      const int g = g0 + ic / NC, c = ic - (ic / NC) * NC;
      return (uint32_t)(((g * NT + nt) * NC + c) * kBlockBytes);
    };
    auto load_tile = [&](int slot, int i, int nt) {
      const uint32_t blk = step_blk(i, nt);
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, lane * 16, blk, kStreamAux);
      wq[slot][nt] = make_uint4(v[0], v[1], v[2], v[3]);
      sc[slot][nt] = __builtin_amdgcn_raw_buffer_load_b16(wres, kBlockWeightBytes + lane * 2, blk, 0);
    };
#pragma unroll
    for (int slot = 0; slot < PF; ++slot)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) load_tile(slot, slot, nt);

    f32x4_t acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = zero4;

    auto epilogue = [&](int g) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tw = g * NT + nt;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (dst[mt] >= 0) {
            const f32x4_t v = acc[nt][mt];
            if (a.gate_up) {
              const int f0 = tw * 8 + 2 * q;
              *reinterpret_cast<uint32_t*>(a.out + dst[mt] * (int64_t)a.out_ld + f0) =
                  pk_bf16(silu_mul(v[0], v[1]), silu_mul(v[2], v[3]));
            } else {
              const int n0 = tw * 16 + 4 * q;
              const float r = rw[mt];
              *reinterpret_cast<uint2*>(a.out + dst[mt] * (int64_t)a.out_ld + n0) =
                  make_uint2(pk_bf16(v[0] * r, v[1] * r), pk_bf16(v[2] * r, v[3] * r));
            }
          }
          acc[nt][mt] = zero4;
        }
      }
    };

    for (int i0 = 0; i0 < nsteps; i0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int i = i0 + u;
        if (i < nsteps) {
          const int c = u % NC;  // PF is a multiple of NC
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            bf16x8_t av[4];
            dequant_words(wq[u][nt], dq_scale(sc[u][nt]), kMaskLo, kMaskHi, kMagic, av);
            load_tile(u, i + PF, nt);  // refill as soon as the tile is dequantised
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    av[st], as_bf16x8(xb[c][mt][st]), acc[nt][mt], 0, 0, 0);
          }
          if (c == NC - 1) epilogue(g0 + i / NC);
        }
      }
    }
  }
}

// Fused down GEMM + weighted top-k combine of a routed call with at most
// kFusedMaxTokens tokens and kFusedMaxSlots slots (the single-token TP
// slice): one workgroup of W waves per 16-row weight tile of the output.
// Wave w computes, for the local slots j = w, w + W, ... (in ascending flat
// order), the tile's 16 outputs of y = W2_e h[slot] in fp32 (h is stored per
// flat slot by the routed gate_up; the slot's row is MFMA column 0) through a
// PF-deep ring of (slot, K chunk) steps, and leaves them in LDS.  Wave 0 then
// adds w[t,j] * y over the local slots in ascending flat order, which is
// ascending j for every token, and stores the tile's bf16 outputs of every
// token; tokens without a local slot get zero.  y is not rounded to bf16
// before the sum.  Each W2 tile of a slot's expert is read once per slot.
// The slot lists live in registers (lane u holds the u-th entry) and are
// read with readlane at uniform indices, so no load waits on LDS.
template <int W, int PF>
__global__ __launch_bounds__(64 * W) void down_combine_small(GemmArgs a) {
  __shared__ float ys[kFusedMaxSlots][16];
  __shared__ int slot_of[kFusedMaxSlots];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, col = lane & 15;
  const int n = a.route_n, NC = a.n_chunks, T = a.T;
  const uint32_t kMaskLo = 0x000F000Fu, kMaskHi = 0x00F000F0u, kMagic = 0x64006400u;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  // Lane i of every wave holds slot i's local expert and weight.
  const int idv = lane < n ? a.route_ids[lane] - a.route_eb : -1;
  const float wv = lane < n ? a.topk_weights[lane] : 0.f;
  const bool loc = lane < n && (unsigned)idv < (unsigned)a.num_experts;
  const uint64_t mask = __builtin_amdgcn_ballot_w64(loc);
  const int n_local = __builtin_popcountll(mask);
  if (wave == 0 && loc) slot_of[__builtin_popcountll(mask & ((1ull << lane) - 1ull))] = lane;
  __syncthreads();
  // all_v: lane j holds the j-th local slot; mine_v: lane u the slot of this
  // wave's u-th local slot (rank wave + W u).
  const int all_v = lane < n_local ? slot_of[lane] : 0;
  const int mine_v = wave + W * lane < n_local ? slot_of[wave + W * lane] : 0;
  const int my_slots = wave < n_local ? (n_local - wave + W - 1) / W : 0;
  const int nsteps = my_slots * NC;
  const int64_t expert_bytes = (int64_t)a.n_tiles * NC * kBlockBytes;
  const __amdgpu_buffer_rsrc_t hres =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.bsrc, 0, (int)a.bsrc_bytes, kRsrcWord3);

  for (int tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    uint4 wq[PF];
    uint32_t sc[PF];
    uint4 hb[PF][4];
    // Step i of this wave: its slot i / NC, chunk i % NC; steps past the
    // last are clamped to it (a redundant load, in bounds).
    auto load_step = [&](int u, int i) {
      const int ic = i < nsteps ? i : nsteps - 1;
      const int js = ic / NC, c = ic - js * NC;
      const int slot = __builtin_amdgcn_readlane(mine_v, js);
      const int e = __builtin_amdgcn_readlane(idv, slot);
      const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.wpack + (int64_t)e * expert_bytes), 0, (int)expert_bytes, kRsrcWord3);
      const uint32_t blk = (uint32_t)((tile * NC + c) * kBlockBytes);
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(wres, lane * 16, blk, kStreamAux);
      wq[u] = make_uint4(v[0], v[1], v[2], v[3]);
      sc[u] = __builtin_amdgcn_raw_buffer_load_b16(wres, kBlockWeightBytes + lane * 2, blk, 0);
      const uint32_t hoff =
          col == 0 ? (uint32_t)(((int64_t)slot * a.K + q * kGroup) * 2) : kNoRow;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4_t h = __builtin_amdgcn_raw_buffer_load_b128(hres, hoff, c * kChunkK * 2 + st * 16, 0);
        hb[u][st] = make_uint4(h[0], h[1], h[2], h[3]);
      }
    };
    if (nsteps > 0) {
#pragma unroll
      for (int u = 0; u < PF; ++u) load_step(u, u);
    }
    f32x4_t y = zero4;
    for (int i0 = 0; i0 < nsteps; i0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int i = i0 + u;
        if (i < nsteps) {
          bf16x8_t av[4];
          dequant_words(wq[u], dq_scale(sc[u]), kMaskLo, kMaskHi, kMagic, av);
#pragma unroll
          for (int st = 0; st < 4; ++st)
            y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[st], as_bf16x8(hb[u][st]), y, 0, 0, 0);
          if (i + PF < nsteps) load_step(u, i + PF);  // refill the ring slot just consumed
          if (i % NC == NC - 1) {  // slot done: its 16 outputs to LDS
            const int j = wave + W * (i / NC);
            if (col == 0) *reinterpret_cast<f32x4_t*>(&ys[j][4 * q]) = y;
            y = zero4;
          }
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // Lane (r, tq) owns rows r of tokens tq, tq + 4, tq + 8, tq + 12.
      const int r = lane & 15, tq = lane >> 4;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < n_local; j0 += 8) {
        float yv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) yv[u] = j0 + u < n_local ? ys[j0 + u][r] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (j0 + u >= n_local) break;
          const int slot = __builtin_amdgcn_readlane(all_v, j0 + u);
          const int t = slot / a.topk;
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), slot));
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (t == tq + 4 * m) acc[m] = __builtin_fmaf(w, yv[u], acc[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int t = tq + 4 * m;
        if (t < T) a.out[(int64_t)t * a.out_ld + tile * 16 + r] = to_bf16(acc[m]);
      }
    }
    __syncthreads();  // ys is reused by the next tile
  }
}

template <int NT, int MT, int WK, int PF>
hipError_t launch_stream_t(const GemmArgs& a, int grid, hipStream_t stream) {
  const size_t red = WK > 1 ? (size_t)WK * NT * MT * 64 * 4 * sizeof(float) : 0;
  const size_t lds = red + (a.route_ids != nullptr ? route_lds_bytes(a.num_experts, a.route_n) : 0);
  static const int per_cu = blocks_per_cu(gemm_stream<NT, MT, WK, PF>, 64 * WK, red);
  const int cap = per_cu * (a.num_cus > 0 ? a.num_cus : 256);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((gemm_stream<NT, MT, WK, PF>), dim3(grid), dim3(64 * WK), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

template <int NT, int MT, int NC>
hipError_t launch_stream_shortk_t(const GemmArgs& a, int grid, hipStream_t stream) {
  static const int per_cu = blocks_per_cu(gemm_stream_shortk<NT, MT, NC>, 64, 0);
  const int cap = per_cu * (a.num_cus > 0 ? a.num_cus : 256);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((gemm_stream_shortk<NT, MT, NC>), dim3(grid), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_down_combine_small(const GemmArgs& a, hipStream_t stream) {
  if (a.route_n > kFusedMaxSlots || a.T > kFusedMaxTokens) return hipErrorInvalidValue;
  if (a.n_chunks <= 2)  // one ring step per chunk of a slot
    hipLaunchKernelGGL((down_combine_small<8, 2>), dim3(a.n_tiles), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((down_combine_small<8, 4>), dim3(a.n_tiles), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int kernel, int nt, int mt, int wk, int pf, const GemmArgs& a, int grid,
                       hipStream_t stream) {
  (void)kernel;
  if (a.slices_per_item > 0 && a.n_chunks <= 2) {  // short K: several weight-tile groups per item
    if (a.route_ids != nullptr) return hipErrorInvalidValue;  // no routed short-K variant
    const int key = nt * 100 + mt * 10 + a.n_chunks;
    switch (key) {
      case 211: return launch_stream_shortk_t<2, 1, 1>(a, grid, stream);
      case 212: return launch_stream_shortk_t<2, 1, 2>(a, grid, stream);
      case 221: return launch_stream_shortk_t<2, 2, 1>(a, grid, stream);
      case 222: return launch_stream_shortk_t<2, 2, 2>(a, grid, stream);
      case 411: return launch_stream_shortk_t<4, 1, 1>(a, grid, stream);
      case 412: return launch_stream_shortk_t<4, 1, 2>(a, grid, stream);
      case 421: return launch_stream_shortk_t<4, 2, 1>(a, grid, stream);
      case 422: return launch_stream_shortk_t<4, 2, 2>(a, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  const int key = nt * 1000 + mt * 100 + wk * 10 + pf;
  switch (key) {
#define CHORD_STREAM_CASE(NT, MT, WK, PF) \
  case NT * 1000 + MT * 100 + WK * 10 + PF: return launch_stream_t<NT, MT, WK, PF>(a, grid, stream);
#define CHORD_STREAM_WK(NT, MT, WK) CHORD_STREAM_CASE(NT, MT, WK, 2) CHORD_STREAM_CASE(NT, MT, WK, 4)
#define CHORD_STREAM_MT(NT, MT) \
  CHORD_STREAM_WK(NT, MT, 1) CHORD_STREAM_WK(NT, MT, 2) CHORD_STREAM_WK(NT, MT, 4)
    CHORD_STREAM_MT(2, 1)
    CHORD_STREAM_CASE(1, 1, 8, 4)
    CHORD_STREAM_CASE(1, 1, 8, 8)
    CHORD_STREAM_WK(1, 1, 2)
    CHORD_STREAM_WK(1, 1, 4)
    CHORD_STREAM_WK(2, 1, 8)
    CHORD_STREAM_MT(2, 2)
    CHORD_STREAM_MT(4, 1)
    CHORD_STREAM_MT(4, 2)
#undef CHORD_STREAM_MT
#undef CHORD_STREAM_WK
#undef CHORD_STREAM_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace chord
