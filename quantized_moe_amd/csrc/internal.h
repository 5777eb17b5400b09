// Internal declarations shared by the host runtime and the HIP kernels of
// libchord.so.  Not part of the public ABI (see include/chord.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "chord.h"

namespace chord {

// ---------------------------------------------------------------------------
// Packed weight layout (gfx950).
//
// A weight [E, N, K] is cut into 16-row tiles and 128-wide K chunks.  Each
// (expert, tile, chunk) is one 1152-byte block, stored tile-major so that a
// wavefront streaming one tile along K reads contiguous memory:
//
//   bytes [0, 1024):   64 lanes x 16 bytes.  Lane l holds the 32 codes of
//                      tile row r = l % 16 for K range chunk*128 + (l/16)*32
//                      + [0, 32), i.e. exactly one scale group, as 4 words.
//                      Word s covers k = base + 8s .. 8s+7; inside a word the
//                      code of k = 2v sits at bits 4v..4v+3 and the code of
//                      k = 2v+1 at bits 16+4v..16+4v+3, so one shift and one
//                      mask-or give a pair of codes in the two 16-bit halves.
//                      MFMA step s of the chunk takes word s of every lane:
//                      lane group l/16 supplies k = (l/16)*32 + 8s + [0, 8).
//   bytes [1024, 1152): 64 bf16 scales in lane order: lane l's group scale.
//
// Gate_up weights interleave gate and up rows inside each tile so the fused
// SiLU*mul epilogue finds both in one lane: tile t, row r = 4q + w holds
// feature f = 8t + 2q + (w >> 1); w even = gate row f, w odd = up row I + f.
// Down weights keep natural order: tile t, row r = feature 16t + r.
// ---------------------------------------------------------------------------
constexpr int kTileRows = 16;
constexpr int kChunkK = 128;
constexpr int kGroup = 32;
constexpr int kBlockWeightBytes = 1024;
constexpr int kBlockBytes = 1152;

inline size_t packed_bytes(int E, int N, int K) {
  return (size_t)E * (size_t)(N / kTileRows) * (size_t)(K / kChunkK) * (size_t)kBlockBytes;
}

// Tile descriptor produced on the device: local expert, first internal row,
// number of internal rows (<= tile tokens).  Big tiles may be split along K:
// entry kpart of ksplit covers chunks [kpart nc / ksplit, (kpart + 1) nc /
// ksplit); split_id indexes the call's split tiles and pbase is the tile's
// first partial slot (one slot = 256 rows x 16 tokens of fp32).
struct TileDesc {
  int32_t expert;
  int32_t row_begin;
  int32_t nrows;
  int32_t kpart;
  int32_t ksplit;
  int32_t split_id;
  int32_t pbase;
  int32_t pad;
};
constexpr int kMaxSplitTiles = 16;     // tiles split along K per layer call
constexpr int kSplitCapSlots = 4096;   // partial slots (16 KB each: 64 MB)
constexpr int kPartialSlotFloats = 256 * 16;

enum Layout : int { kIndexed = 0, kContiguous = 1, kMasked = 2 };

// Device status words at the start of every layer workspace.
constexpr int kTileGroups = 8;  // tiles are grouped by expert % 8 (one group per XCD)
struct DevStatus {
  int32_t error;                        // nonzero: routing validation failed (bit flags)
  int32_t ntiles;                       // tiles written by the tile builder
  int32_t group_start[kTileGroups + 1]; // tile range of each expert group
  int32_t nsplit;                       // big tiles split along K
  int32_t pad[52];
};

// Arguments of the tile builder (one workgroup).  Each expert segment goes
// either to the small-tile list `tiles` (tiles of <= tile_tokens rows, for the
// weight-streaming kernel; count in status->ntiles) or, when it has at least
// split_rows rows, to the big-tile list `tiles_b` (tiles of <= big_tokens
// rows, grouped by expert % 8, ranges in status->group_start, for the tiled
// kernel).  split_rows = 0 sends every segment to the big list.
struct TileBuildArgs {
  int layout;
  int num_experts;     // E_l
  int tile_tokens;     // max rows per small tile
  int max_tiles;       // capacity of `tiles`
  int big_tokens;      // max rows per big tile
  int max_tiles_b;     // capacity of `tiles_b`
  int split_rows;      // segments with >= split_rows rows go to `tiles_b`
  int validate;
  int split_cap;       // partial slots for K-split big tiles (0: no split)
  int max_ksplit;      // parts per split tile (2..4)
  int max_slices;      // 256-row slices of the wider tiled GEMM
  TileDesc* split_tiles;  // [kMaxSplitTiles]: part-0 entry of each split tile
  // indexed
  const int32_t* expert_ids;
  const int32_t* ntpp;
  int block_m;
  int64_t max_padded;
  // contiguous
  const int32_t* m_indices;
  int64_t M;
  // masked
  const int32_t* masked_m;
  int max_m;
  // out
  TileDesc* tiles;
  TileDesc* tiles_b;
  DevStatus* status;
};

// Arguments of one expert GEMM launch (gate_up or down).
struct GemmArgs {
  const uint8_t* wpack;  // packed weight of this GEMM
  int n_tiles;           // N / 16
  int n_chunks;          // K / 128
  int K;                 // row length of the B source (elements)
  const uint16_t* bsrc;  // B rows: x / a (gate_up) or h (down), bf16 [*, K]
  int64_t bsrc_bytes;    // size of bsrc (bounds of the buffer resource, < 3 GiB)
  int layout;
  int gate_up;           // 1: SiLU*mul epilogue into h; 0: plain store
  // indexed
  const int32_t* sorted_ids;
  int topk;
  int64_t n_flat;        // T * k (sentinel and bound)
  // contiguous
  const int32_t* m_indices;
  // tiles: a device tile list, or (tiles == nullptr, indexed only) one tile
  // per alignment block of block_m rows read from expert_ids / ntpp.
  const TileDesc* tiles;
  const DevStatus* status;  // ntiles
  const int32_t* expert_ids;
  const int32_t* ntpp;
  int block_m;
  int64_t max_padded;
  int num_experts;
  int num_cus;           // compute units (persistent grid clamp)
  int tile_tokens;
  int tiles_per_item;    // 16-row weight tiles per work item
  int items_per_tile;    // n_tiles / tiles_per_item (tiled kernel: 256-row slices)
  int slices_per_item;   // tiled kernel, K <= 256: consecutive slices per work item
  int no_chain;          // streaming kernel: 1 = every item restarts its load ring
  int tile_waves;        // tiled kernel, K > 256: waves per workgroup (4 or 8)
  float* partials;       // tiled kernel: K-split partial slots
  const TileDesc* split_tiles;  // tiled kernel: the split tiles (fixup pass)
  int max_slices;        // slot stride of the tile builder
  // output
  uint16_t* out;         // h [rows, I] (gate_up) or y / out rows [*, H] (down)
  int out_ld;
  int64_t out_rows;      // rows of `out` (bound)
  const float* row_weights;  // grouped down only, may be null
  int64_t n_rows_internal;   // internal row bound (h rows)
  // Routed indexed calls: the rows of each expert come from topk_ids, not
  // from an alignment.  The gate_up launch (route_ids set) builds the tables
  // in LDS in every workgroup; its workgroup 0 also writes them to route_list
  // / route_tiles (+ status->ntiles) for the down launch.  h rows are per
  // flat slot then (h_by_slot: the down GEMM reads h[f], not h[R]).
  const int32_t* route_ids;  // topk_ids [route_n], or null
  int route_eb;              // expert_begin
  int route_n;               // T * k
  int32_t* route_list;       // [route_n]: flat slots grouped by local expert
  TileDesc* route_tiles;     // [route_n]: tiles over route_list
  int h_by_slot;
  // Fused down + combine (routed calls with T <= 16, T * k <= 64): routing
  // weights and the token count of the output [T, H].
  const float* topk_weights;
  int T;
};
constexpr int kRoutedMaxSlots = 2048;  // routed calls: T * k at most
constexpr int kFusedMaxSlots = 64;     // fused down + combine: T * k at most
constexpr int kFusedMaxTokens = 16;    // ... and T at most
// LDS bytes of the routing tables of a routed gate_up launch: per expert a
// first row, an end row, a first tile and a count; per slot a list entry and
// at most one tile.
inline size_t route_lds_bytes(int E, int n) { return (size_t)(4 * E + 2 + 2 * n) * sizeof(int); }
constexpr size_t kRouteLdsMax = 32768;  // routed calls: table bytes at most (planner bound)

struct CombineArgs {
  const uint16_t* rows;     // y [*, H] bf16
  const int32_t* topk_ids;  // indexed: local test via ids; null for contiguous
  const int32_t* flat_to_row;  // contiguous: slot -> row (or -1)
  const float* topk_weights;
  int T, k, H;
  int expert_begin, num_experts;
  int64_t n_rows;
  int64_t read_bytes;  // expected row bytes read (0: the whole row buffer)
  uint16_t* out;
};

struct AlignArgs {
  const int32_t* topk_ids;
  int64_t n;               // T * k
  int expert_begin, num_experts, block_m;
  int64_t max_padded;
  int32_t* sorted_ids;
  int32_t* expert_ids;
  int32_t* ntpp;
  int32_t* chunk_counts;   // workspace [nchunks, E_l] (multi-workgroup path)
  int64_t chunk;           // entries per workgroup (multi-workgroup path)
  int nchunks;
};

// Arguments of the dispatch gathers (grouped layouts built from an
// alignment: sorted_ids / expert_ids / ntpp with block_m-row blocks).
struct DispatchArgs {
  const uint16_t* x;          // token rows [T, H] bf16
  const int32_t* topk_ids;    // [T, k] global expert ids
  int T, k, H;
  int expert_begin, num_experts;
  const int32_t* sorted_ids;  // alignment
  const int32_t* expert_ids;
  const int32_t* ntpp;
  int block_m;
  int64_t max_padded;
  uint16_t* out;              // contiguous a [max_rows, H] / masked a3 [E, max_m, H]
  int64_t max_rows;           // contiguous
  int32_t* m_indices;         // contiguous [max_rows]
  int32_t* num_rows;          // contiguous [1]
  int max_m;                  // masked
  int32_t* masked_m;          // masked [E]
  int32_t* dropped;           // masked [1]
  int32_t* flat_to_row;       // [T * k]
};

// Launchers (defined in the .hip files).  All enqueue on `stream` and return
// hipSuccess or the launch error.
hipError_t launch_pack(const int32_t* q, const uint16_t* s, int E, int N, int K, int gate_up,
                       uint8_t* dst, hipStream_t stream);
hipError_t launch_align(const AlignArgs& a, hipStream_t stream);
hipError_t launch_build_tiles(const TileBuildArgs& a, hipStream_t stream);
// Clears the status words; with a.validate also checks block-derived tiles.
hipError_t launch_check_blocks(const TileBuildArgs& a, hipStream_t stream);
// kernel 1 = weight-streaming GEMM.  nt = 16-row weight tiles per wave, mt =
// 16-row token tiles per work item, wk = waves splitting K, pf = K chunks in
// flight per wave.
hipError_t launch_gemm(int kernel, int nt, int mt, int wk, int pf, const GemmArgs& a, int grid,
                       hipStream_t stream);
// LDS-tiled GEMM (needs a device tile list with tiles of at most 192 rows;
// 4 weight tiles per wave, 256 output rows per workgroup; N a multiple of 64).
hipError_t launch_gemm_tile(const GemmArgs& a, int grid, hipStream_t stream);
hipError_t launch_tile_split_fixup(const GemmArgs& a, hipStream_t stream);
// Fused down GEMM + weighted combine of a routed call with T <= 16 and
// T * k <= 64: out[t] = bf16(sum over local j, ascending, of w[t,j] * y_tj),
// every row of out written.
hipError_t launch_down_combine_small(const GemmArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_gather_contiguous(const DispatchArgs& a, hipStream_t stream);
hipError_t launch_gather_masked(const DispatchArgs& a, hipStream_t stream);
hipError_t launch_zero(uint16_t* p, int64_t n, hipStream_t stream);

constexpr int kAlignSingle = 8192;      // align in one workgroup up to this many entries
constexpr int kAlignMinChunk = 1024;    // entries per align workgroup (at least)
constexpr int kAlignCountCap = 8192;    // chunk x expert counts staged in LDS (about)

// Entries per workgroup of the multi-workgroup alignment: small chunks for
// many workgroups, large enough that the [chunks, experts] count table each
// scatter workgroup stages in LDS stays near kAlignCountCap ints.
inline int64_t align_chunk(int64_t n, int E) {
  int64_t c = (n * E + kAlignCountCap - 1) / kAlignCountCap;
  c = (c + 255) / 256 * 256;
  return c < kAlignMinChunk ? kAlignMinChunk : c;
}
inline int64_t align_nchunks(int64_t n, int E) {
  const int64_t c = align_chunk(n, E);
  const int64_t m = (n + c - 1) / c;
  return m < 1 ? 1 : m;
}
inline bool align_single_workgroup(int64_t n, int E) { return n <= kAlignSingle && E <= 512; }
constexpr int kMaxExperts = 1024;       // E_l limit (LDS tables)
constexpr int kMaxSegments = 16384;     // contiguous 128-row chunks limit

}  // namespace chord
