// Layer plumbing kernels: the device-side tile builder that turns each routing
// layout into a list of (expert, rows) tiles, the block check used when tiles
// are the alignment blocks themselves, and the weighted top-k combine.
#include "device_common.h"

namespace chord {
namespace {

// ---------------------------------------------------------------------------
// Tile builder: one workgroup turns the layout's row map into TileDesc's of at
// most tile_tokens rows, ordered by expert (indexed, masked) or by 128-row
// chunk (contiguous).  With `validate`, routing errors set bits in
// status->error:
//   1 expert id out of range        2 an expert's blocks not contiguous
//   4 bad num_tokens_post_padded    8 m_indices value out of range
//   16 chunk mixes experts          32 masked_m out of [0, max_m]
//   64 tile capacity exceeded
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_tiles(TileBuildArgs a) {
  __shared__ int first[kMaxExperts];
  __shared__ int last[kMaxExperts];
  __shared__ int nblk[kMaxExperts];
  __shared__ int scan_tmp[17 * 11];
  __shared__ int err;
  const int tid = threadIdx.x;
  const int E = a.num_experts;
  const int TOK = a.tile_tokens;
  if (tid == 0) err = 0;
  for (int e = tid; e < E; e += blockDim.x) {
    first[e] = INT32_MAX;
    last[e] = -1;
    nblk[e] = 0;
  }
  __syncthreads();

  // Pass 0: per-expert extents (indexed) / counts (masked), with validation.
  if (a.layout == kIndexed) {
    int64_t ntpp = *a.ntpp;
    const int64_t nb_cap = (a.max_padded + a.block_m - 1) / a.block_m;
    if (ntpp < 0 || ntpp > a.max_padded || ntpp % a.block_m != 0) {
      if (a.validate && tid == 0) atomicOr(&err, 4);
      ntpp = ntpp < 0 ? 0 : (ntpp > a.max_padded ? a.max_padded : ntpp);
    }
    const int64_t nb = min(ntpp / a.block_m, nb_cap);
    // Extents from run boundaries: a block whose left (right) neighbour
    // belongs to another expert starts (ends) a run of its expert.  Only the
    // boundaries touch the LDS tables (a wave of same-expert blocks would
    // otherwise serialise 64 atomics on one address), nblk counts the runs
    // (one per expert in a valid layout), and each thread keeps the ids of
    // kBatch blocks and their neighbours in flight together.  The first batch
    // is read before the padded total is known (inside the buffer's nb_cap
    // blocks), so its loads overlap the load of the total.
    constexpr int kBatch = 4;
    for (int64_t b0 = tid; b0 == tid || b0 < nb; b0 += (int64_t)blockDim.x * kBatch) {
      int ec[kBatch], ep[kBatch], en[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t b = b0 + (int64_t)u * blockDim.x;
        ec[u] = b < nb_cap ? a.expert_ids[b] : -1;
        ep[u] = (b < nb_cap && b > 0) ? a.expert_ids[b - 1] : INT32_MIN;
        en[u] = b + 1 < nb_cap ? a.expert_ids[b + 1] : INT32_MIN;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t b = b0 + (int64_t)u * blockDim.x;
        if (b >= nb) break;
        const int e = ec[u];
        if (e < 0 || e >= E) {
          if (a.validate) atomicOr(&err, 1);
          continue;
        }
        if (b == 0 || ep[u] != e) {
          atomicMin(&first[e], (int)b);
          atomicAdd(&nblk[e], 1);
        }
        if (b + 1 >= nb || en[u] != e) atomicMax(&last[e], (int)b);
      }
    }
    __syncthreads();
    if (tid < E && last[tid] >= 0 && a.validate && nblk[tid] != 1) atomicOr(&err, 2);
  } else if (a.layout == kMasked) {
    if (tid < E) {
      int m = a.masked_m[tid];
      if ((m < 0 || m > a.max_m) && a.validate) atomicOr(&err, 32);
      m = m < 0 ? 0 : (m > a.max_m ? a.max_m : m);
      first[tid] = m;  // rows
    }
  } else {
    // Contiguous: each expert's 128-row chunks; the segment runs from its
    // first chunk to the last valid row of its last chunk (rows of other
    // experts inside it, if the layout is broken, are skipped by the GEMMs'
    // row maps).
    const int nch = (int)(a.M / 128);
    for (int c = tid; c < nch; c += blockDim.x) {
      const int e = a.m_indices[(int64_t)c * 128];
      if (e < 0 || e >= E) {
        if (e != -1 && a.validate) atomicOr(&err, 8);
        continue;
      }
      atomicMin(&first[e], c);
      atomicMax(&last[e], c);
      atomicAdd(&nblk[e], 1);
      if (a.validate)
        for (int r = 1; r < 128; ++r) {
          const int v = a.m_indices[(int64_t)c * 128 + r];
          if (v != e && v != -1) atomicOr(&err, (v < -1 || v >= E) ? 8 : 16);
        }
    }
    __syncthreads();
    if (tid < E && last[tid] >= 0) {
      if (a.validate && last[tid] - first[tid] + 1 != nblk[tid]) atomicOr(&err, 16);
      // Last row of this expert in its last chunk: the chunk's 128 ids are
      // read as 32 independent 16-byte loads, all in flight together (4-byte
      // loads if the caller's m_indices is not 16-byte aligned).
      const int32_t* ids = a.m_indices + (int64_t)last[tid] * 128;
      int lastv = 0;
      if ((reinterpret_cast<uintptr_t>(ids) & 15) == 0) {
        int4 v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = reinterpret_cast<const int4*>(ids)[i];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (v[i].x == tid) lastv = 4 * i + 1;
          if (v[i].y == tid) lastv = 4 * i + 2;
          if (v[i].z == tid) lastv = 4 * i + 3;
          if (v[i].w == tid) lastv = 4 * i + 4;
        }
      } else {
        for (int r = 0; r < 128; ++r)
          if (ids[r] == tid) lastv = r + 1;
      }
      nblk[tid] = (last[tid] - first[tid]) * 128 + lastv;  // segment rows
    }
  }
  __syncthreads();

  // The segment owned by this thread: one expert.  f(expert, row_begin, rows).
  auto for_each_segment = [&](auto&& f) {
    if (tid >= E) return;
    if (a.layout == kIndexed) {
      if (last[tid] >= 0) f(tid, first[tid] * a.block_m, (last[tid] - first[tid] + 1) * a.block_m);
    } else if (a.layout == kMasked) {
      if (first[tid] > 0) f(tid, tid * a.max_m, first[tid]);
    } else {
      if (last[tid] >= 0 && nblk[tid] > 0) f(tid, first[tid] * 128, nblk[tid]);
    }
  };

  // Small tiles (streaming kernel) in expert order.  Big tiles (tiled
  // kernel) are balanced over the 8 groups (one per XCD): ranked by size
  // (rows rounded up to 32, biggest first), rank k goes to group
  // (k / 8 even ? k % 8 : 7 - k % 8) at position k / 8 of that group.  All
  // slices of one big tile stay in one group, so its token rows are read
  // into one XCD's L2.
  //
  // K split: a big tile with g live 16-row groups, well above the mean gm of
  // the call's big tiles, becomes s = round(g / gm) entries (at most 4, and
  // at most one per 8 K chunks of the shorter GEMM), each
  // covering 1/s of K; the parts store fp32 partials and a fixup pass after
  // the GEMM adds them.  One oversized tile (a hot expert) then stops setting
  // the kernel's critical path.  Off when the partial slots or the split-tile
  // list would overflow their caps.
  constexpr int kBuckets = 8;  // 32-row size classes (big tiles <= 256 rows)
  const int TOKB = a.big_tokens;
  auto is_big = [&](int rows) { return rows >= a.split_rows; };
  auto bucket = [&](int rows) { return min(kBuckets - 1, (rows - 1) >> 5); };
  auto groups_of = [](int n) { return (n + 15) >> 4; };

  // Mean live groups of the big tiles.
  int nbig_t = 0, gsum_t = 0;
  for_each_segment([&](int, int, int rows) {
    if (!is_big(rows)) return;
    for (int r = 0; r < rows; r += TOKB) {
      ++nbig_t;
      gsum_t += groups_of(min(TOKB, rows - r));
    }
  });
  int mean_in[2] = {nbig_t, gsum_t}, mean_tot[2];
  block_scan_excl_n<2>(mean_in, scan_tmp, mean_tot);
  bool split_on = a.split_cap > 0 && mean_tot[0] > 0;
  auto ksplit_of = [&](int g) {
    if (!split_on) return 1;
    const int s = (2 * g * mean_tot[0] + mean_tot[1]) / (2 * mean_tot[1]);  // round(g / gm)
    return s < 2 ? 1 : (s > a.max_ksplit ? a.max_ksplit : s);
  };

  // Counters: 8 size classes of big entries, small tiles, split tiles, and
  // split units (sum of s * g over split tiles).
  constexpr int kNC = kBuckets + 3;
  int cnt[kNC], tot[kNC];
  auto count_all = [&]() {
#pragma unroll
    for (int i = 0; i < kNC; ++i) cnt[i] = 0;
    for_each_segment([&](int, int, int rows) {
      if (is_big(rows)) {
        for (int r = 0; r < rows; r += TOKB) {
          const int n = min(TOKB, rows - r), g = groups_of(n), sp = ksplit_of(g);
          for (int p = 0; p < sp; ++p) ++cnt[bucket((n + sp - 1) / sp)];
          if (sp > 1) {
            ++cnt[kBuckets + 1];
            cnt[kBuckets + 2] += sp * g;
          }
        }
      } else {
        cnt[kBuckets] += (rows + TOK - 1) / TOK;
      }
    });
    block_scan_excl_n<kNC>(cnt, scan_tmp, tot);
  };
  count_all();
  if (split_on && (tot[kBuckets + 1] > kMaxSplitTiles ||
                   (int64_t)tot[kBuckets + 2] * a.max_slices > a.split_cap)) {
    split_on = false;  // uniform across the workgroup: the totals are
    count_all();
  }
  const int total_small = tot[kBuckets];
  int base_small = cnt[kBuckets];
  int split_id = cnt[kBuckets + 1];
  int split_units = cnt[kBuckets + 2];
  int rank[kBuckets];
  int total_big = 0;
  for (int b = kBuckets - 1; b >= 0; --b) {  // biggest class first
    rank[b] = total_big + cnt[b];
    total_big += tot[b];
  }
  const bool big_fits = total_big <= a.max_tiles_b;
  if ((total_small > a.max_tiles || !big_fits) && a.validate && tid == 0) atomicOr(&err, 64);
  if (!big_fits) total_big = 0;
  // Group g holds the ranks k with snake(k) == g: one per full round of 8,
  // plus one if g is among the first (or, in an odd round, last) positions
  // of the partial round.
  const int rounds = total_big / kTileGroups, rem = total_big % kTileGroups;
  auto group_count = [&](int g) {
    const bool odd = rounds & 1;
    const bool extra = odd ? g >= kTileGroups - rem : g < rem;
    return rounds + (extra ? 1 : 0);
  };
  if (tid == 0) {
    int gs = 0;
    for (int g = 0; g < kTileGroups; ++g) {
      a.status->group_start[g] = gs;
      gs += group_count(g);
    }
    a.status->group_start[kTileGroups] = gs;
  }
  int gstart[kTileGroups];
  {
    int gs = 0;
#pragma unroll
    for (int g = 0; g < kTileGroups; ++g) {
      gstart[g] = gs;
      gs += group_count(g);
    }
  }
  for_each_segment([&](int e, int row_begin, int rows) {
    if (is_big(rows)) {
      if (!big_fits) return;
      for (int r = 0; r < rows; r += TOKB) {
        const int n = min(TOKB, rows - r), g = groups_of(n), sp = ksplit_of(g);
        const int sid = sp > 1 ? split_id++ : 0;
        const int pbase = sp > 1 ? split_units * a.max_slices : 0;
        if (sp > 1) split_units += sp * g;
        for (int p = 0; p < sp; ++p) {
          const int k = rank[bucket((n + sp - 1) / sp)]++;
          const int pos = k % kTileGroups, rnd = k / kTileGroups;
          const int grp = (rnd & 1) ? kTileGroups - 1 - pos : pos;
          a.tiles_b[gstart[grp] + rnd] = TileDesc{e, row_begin + r, n, p, sp, sid, pbase, 0};
        }
        if (sp > 1) a.split_tiles[sid] = TileDesc{e, row_begin + r, n, 0, sp, sid, pbase, 0};
      }
    } else {
      for (int r = 0; r < rows; r += TOK) {
        if (base_small < a.max_tiles)
          a.tiles[base_small] = TileDesc{e, row_begin + r, min(TOK, rows - r), 0, 1, 0, 0, 0};
        ++base_small;
      }
    }
  });
  __syncthreads();
  if (tid == 0) {
    a.status->ntiles = min(total_small, a.max_tiles);
    a.status->nsplit = split_on && big_fits ? tot[kBuckets + 1] : 0;
    a.status->error = err;
  }
}

// Validation of block-derived tiles (indexed, tile == alignment block): flags
// out-of-range expert ids and a bad padded total in status->error.
__global__ __launch_bounds__(256) void check_blocks(TileBuildArgs a) {
  int64_t ntpp = *a.ntpp;
  int err = 0;
  if (ntpp < 0 || ntpp > a.max_padded || ntpp % a.block_m != 0) err |= 4;
  ntpp = ntpp < 0 ? 0 : (ntpp > a.max_padded ? a.max_padded : ntpp);
  const int64_t nb = ntpp / a.block_m;
  for (int64_t b = threadIdx.x; b < nb; b += blockDim.x) {
    const int e = a.expert_ids[b];
    if (e < 0 || e >= a.num_experts) err |= 1;
  }
  if (err) atomicOr(&a.status->error, err);
}

__global__ void clear_status(DevStatus* s) {
  if (threadIdx.x == 0) {
    s->error = 0;
    s->ntiles = 0;
  }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = bf16(sum over slots j with a row, ascending j, of
// w[t,j] * y_row), fp32 accumulation; tokens without a local slot get 0.
// One wave per (token, span of 64 * 8 * kCombinePieces outputs): the token is
// uniform across the wave, so the slot ids (or the slot -> row map) and the
// weights are scalar loads and the per-batch branch is uniform.  Each lane
// owns kCombinePieces 16-byte pieces (8 outputs each), and the row loads of
// B slots are issued together.  Batches of 2 skip more empty slots on sparse
// routing (one local slot of 8 on the prefill share: 48 -> 45 us) and cost
// nothing measurable when every slot is local (TP slice).  With fewer waves
// than SIMDs the kernel is a chain of memory latencies, so all 8 slots of a
// top-8 token go out in one batch.  B does not change the summation order.
// ---------------------------------------------------------------------------
constexpr int kCombineWaves = 4;
constexpr int kCombinePieces = 2;
// Combines that read more row bytes than this load them with the
// non-temporal cache policy: each row is read once, and a stream bigger than
// the MI355X's 256 MB last-level cache only evicts what later reads would hit
// (TP slice T = 4096, 470 MB of rows: 115 -> 87 us).  Smaller reads may still
// hit rows that cache holds and keep the default policy (grouped combine over
// 117 MB of rows: 34 us with it, 40 without).  The bytes are those the call
// expects to read (the indexed layer's y buffer has a row per slot, of which
// only the local ones are read), else the whole row buffer.
constexpr int64_t kRowsStreamBytes = (int64_t)256 << 20;

template <int B, int AUX>
__global__ __launch_bounds__(64 * kCombineWaves) void combine_kernel(CombineArgs a) {
  constexpr int P = kCombinePieces;
  const int nvec = a.H / 8;
  const int spans = (nvec + 64 * P - 1) / (64 * P);
  // T * spans < 2^31 (host-checked), so 32-bit wave indexing; every value
  // below derived from `wid` is wave-uniform.
  const int wid = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kCombineWaves +
                                                 (int)(threadIdx.x >> 6));
  if (wid >= a.T * spans) return;
  const int t = __builtin_amdgcn_readfirstlane(wid / spans);
  const int vbase = (wid - t * spans) * 64 * P + (int)(threadIdx.x & 63);
  // Rows through a buffer resource (loads past its end return zeros).
  const int64_t row_bytes = (int64_t)a.H * 2;
  const int64_t span = a.n_rows * row_bytes;
  const __amdgpu_buffer_rsrc_t rres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.rows, 0, (int)(span < 0x7FFFFFFF ? span : 0x7FFFFFFF), 0x00020000);
  const int64_t s0 = (int64_t)t * a.k;
  float acc[P][8];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[p][i] = 0.f;
  for (int j0 = 0; j0 < a.k; j0 += B) {
    // Unconditional (index-clamped) metadata loads first, so they batch.
    int32_t raw[B];
    float wj[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int j = j0 + u < a.k ? j0 + u : a.k - 1;
      raw[u] = a.flat_to_row != nullptr ? a.flat_to_row[s0 + j] : a.topk_ids[s0 + j];
      wj[u] = a.topk_weights[s0 + j];
    }
    int64_t row[B];
    bool any = false;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      int64_t r = -1;
      if (j0 + u < a.k) {
        if (a.flat_to_row != nullptr) {
          r = raw[u];
          if (r >= a.n_rows) r = -1;
        } else {
          const int e = raw[u] - a.expert_begin;
          r = (e >= 0 && e < a.num_experts) ? s0 + j0 + u : -1;
        }
      }
      row[u] = r;
      any |= r >= 0;
    }
    if (!any) continue;
    // Slots without a row load from past the buffer's end (zeros) with weight
    // 0: adding those +-0 products leaves every partial sum unchanged, and no
    // load sits behind a branch.
    u32x4_t y[B][P];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (row[u] < 0) wj[u] = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int v = vbase + p * 64;
        const uint32_t off = (row[u] >= 0 && v < nvec) ? (uint32_t)(row[u] * row_bytes + v * 16)
                                                        : 0xFFFFFFF0u;
        y[u][p] = __builtin_amdgcn_raw_buffer_load_b128(rres, off, 0, AUX);
      }
    }
#pragma unroll
    for (int u = 0; u < B; ++u)
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[p][2 * i] += wj[u] * bf16_to_f32(y[u][p][i] & 0xFFFFu);
          acc[p][2 * i + 1] += wj[u] * bf16_to_f32(y[u][p][i] >> 16);
        }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int v = vbase + p * 64;
    if (v >= nvec) continue;
    const uint4 o = make_uint4(pk_bf16(acc[p][0], acc[p][1]), pk_bf16(acc[p][2], acc[p][3]),
                               pk_bf16(acc[p][4], acc[p][5]), pk_bf16(acc[p][6], acc[p][7]));
    *reinterpret_cast<uint4*>(a.out + (int64_t)t * a.H + v * 8) = o;
  }
}

__global__ void zero_kernel(uint16_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

hipError_t launch_build_tiles(const TileBuildArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(build_tiles, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_check_blocks(const TileBuildArgs& a, hipStream_t stream) {
  // Block-derived tiles need no status word unless validating.
  if (!a.validate) return hipSuccess;
  hipLaunchKernelGGL(clear_status, dim3(1), dim3(64), 0, stream, a.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_blocks, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int per_wave = 64 * kCombinePieces;
  const int64_t waves = (int64_t)a.T * ((a.H / 8 + per_wave - 1) / per_wave);
  const dim3 grid((unsigned)((waves + kCombineWaves - 1) / kCombineWaves));
  const dim3 block(64 * kCombineWaves);
  const bool stream_rows = (a.read_bytes > 0 ? a.read_bytes : a.n_rows * a.H * 2) > kRowsStreamBytes;
  if (waves < 1024) {
    if (stream_rows)
      hipLaunchKernelGGL((combine_kernel<8, 2>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((combine_kernel<8, 0>), grid, block, 0, stream, a);
  } else {
    if (stream_rows)
      hipLaunchKernelGGL((combine_kernel<2, 2>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((combine_kernel<2, 0>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_zero(uint16_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace chord
