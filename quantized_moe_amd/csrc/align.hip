// Routing alignment for the indexed layer: a stable counting sort of the flat
// (token, slot) ids by local expert, each expert's group padded to a multiple
// of block_m with the sentinel T*k, plus the per-block expert ids and the
// padded total.  Ranks inside a group come from wavefront ballots (a 10-bit
// match of the expert id) and per-wave counts in LDS, so the order is the
// ascending flat index and the result is deterministic.
//
// Small inputs (<= kAlignSingle entries, <= 512 experts) run in one
// workgroup; larger ones in two launches over chunks of >= kAlignMinChunk
// entries: per-chunk histograms, then per-chunk scatters that derive their
// offsets from the histograms themselves.
#include "device_common.h"

namespace chord {
namespace {

__device__ __forceinline__ int local_expert(const int32_t* ids, int64_t i, int64_t n, int eb,
                                            int E) {
  if (i >= n) return -1;
  const int g = ids[i] - eb;
  return (g >= 0 && g < E) ? g : -1;
}

// Exclusive scan of one int per thread across the workgroup; `tmp` holds
// >= 17 ints of LDS.  Returns the exclusive prefix; *total receives the sum.
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  int x[1] = {v}, t[1];
  block_scan_excl_n<1>(x, tmp, t);
  *total = t[0];
  return x[0];
}

// One round: every thread takes entry i (ascending with the thread index),
// whose local expert e (-1: none) the caller has loaded, and writes it to its
// stable position running[e] + (earlier entries of e in this round).  `wcnt`
// is [waves][E] of zeros on entry and on exit.
__device__ void scatter_round(int e, int64_t i, int E, int* running, int* wcnt,
                              int32_t* __restrict__ sorted_ids) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool valid = e >= 0;
  uint64_t mask = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t m = __ballot(bit);
    mask &= bit ? m : ~m;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(mask & lt);
  const int cnt = __popcll(mask);
  const bool leader = valid && rank == 0;
  if (leader) wcnt[wave * E + e] = cnt;
  __syncthreads();
  if (valid) {
    int off = running[e];
    for (int w = 0; w < wave; ++w) off += wcnt[w * E + e];
    sorted_ids[off + rank] = (int32_t)i;
  }
  __syncthreads();
  if (leader) {
    atomicAdd(&running[e], cnt);
    wcnt[wave * E + e] = 0;
  }
  __syncthreads();
}

// Writes expert_ids for the blocks of expert e and the sentinel into the
// padding of its group.
__device__ void write_segment(int e, int seg, int cnt, int padded, int bm, int32_t sentinel,
                              int32_t* sorted_ids, int32_t* expert_ids) {
  for (int p = seg + cnt; p < seg + padded; ++p) sorted_ids[p] = sentinel;
  for (int b = seg / bm; b < (seg + padded) / bm; ++b) expert_ids[b] = e;
}

__device__ void fill_tail(int64_t ntpp, const AlignArgs& a) {
  const int32_t sentinel = (int32_t)a.n;
  for (int64_t p = ntpp + threadIdx.x; p < a.max_padded; p += blockDim.x) a.sorted_ids[p] = sentinel;
  const int64_t nb = (a.max_padded + a.block_m - 1) / a.block_m;
  for (int64_t b = ntpp / a.block_m + threadIdx.x; b < nb; b += blockDim.x) a.expert_ids[b] = -1;
}

// ---- single workgroup path ------------------------------------------------
__global__ __launch_bounds__(1024) void align_single(AlignArgs a) {
  extern __shared__ int lds[];
  const int E = a.num_experts;
  int* running = lds;              // [E]
  int* wcnt = lds + E;             // [16][E]
  int* tmp = lds + 17 * E;         // [17]
  for (int e = threadIdx.x; e < E; e += blockDim.x) running[e] = 0;
  for (int x = threadIdx.x; x < 16 * E; x += blockDim.x) wcnt[x] = 0;
  // n <= kAlignSingle = 8 x 1024: every thread loads its (up to) 8 entries
  // once, all in flight together, and keeps them for the scatter rounds.
  constexpr int kPer = kAlignSingle / 1024;
  int ev[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    ev[u] = local_expert(a.topk_ids, (int64_t)u * blockDim.x + threadIdx.x, a.n, a.expert_begin, E);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (ev[u] >= 0) atomicAdd(&running[ev[u]], 1);
  __syncthreads();
  // E <= 1024 = blockDim: thread e owns expert e.
  const int e = threadIdx.x;
  const int cnt = e < E ? running[e] : 0;
  const int padded = ((cnt + a.block_m - 1) / a.block_m) * a.block_m;
  int total;
  const int seg = block_exclusive_scan(padded, tmp, &total);
  if (e < E) {
    write_segment(e, seg, cnt, padded, a.block_m, (int32_t)a.n, a.sorted_ids, a.expert_ids);
    running[e] = seg;
  }
  if (threadIdx.x == 0) *a.ntpp = total;
  fill_tail(total, a);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t base = (int64_t)u * blockDim.x;
    if (base >= a.n) break;  // uniform
    scatter_round(ev[u], base + threadIdx.x, E, running, wcnt, a.sorted_ids);
  }
}

// ---- multi-workgroup path -------------------------------------------------
// Two launches: per-chunk expert counts, then per-chunk scatters.  Each
// scatter workgroup stages the whole [chunks, experts] count table in LDS and
// derives from it every expert's padded segment start and its own chunk's
// offset inside each segment, so no offsets launch sits between the two.  The
// padding sentinels, the per-block expert ids, the padded total and the
// buffer tails are written by the scatter workgroups between them.
constexpr int kAlignThreads = 256;
constexpr int kCountBatch = 4;
constexpr int kStageBatch = 8;  // count-table loads in flight per thread
constexpr int kIdBatch = 8;     // scatter rounds whose entries load together

__global__ __launch_bounds__(kAlignThreads) void align_count(AlignArgs a) {
  extern __shared__ int lds[];
  const int E = a.num_experts;
  for (int e = threadIdx.x; e < E; e += blockDim.x) lds[e] = 0;
  __syncthreads();
  const int64_t begin = (int64_t)blockIdx.x * a.chunk;
  const int64_t end = min(a.n, begin + a.chunk);
  for (int64_t base = begin; base < end; base += kAlignThreads * kCountBatch) {
    int e[kCountBatch];
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u)
      e[u] = local_expert(a.topk_ids, base + u * kAlignThreads + threadIdx.x, end,
                          a.expert_begin, E);
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u)
      if (e[u] >= 0) atomicAdd(&lds[e[u]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    a.chunk_counts[(int64_t)blockIdx.x * E + e] = lds[e];
}

__global__ __launch_bounds__(kAlignThreads) void align_scatter(AlignArgs a) {
  extern __shared__ int lds[];
  const int E = a.num_experts, nc = a.nchunks, b = blockIdx.x, bm = a.block_m;
  int* counts = lds;               // [nc][E]
  int* running = counts + nc * E;  // [E]: next slot of each expert for this chunk
  int* seg = running + E;          // [E + 1]: padded segment starts, seg[E] = total
  int* wcnt = seg + E + 1;         // [4][E]
  int* tmp = wcnt + 4 * E;         // [17]
  const int64_t begin = (int64_t)b * a.chunk;
  const int64_t end = min(a.n, begin + a.chunk);
  // The chunk's first kIdBatch rounds of entries load first, in flight while
  // the count table is staged and scanned; the table loads go out
  // kStageBatch at a time (one dependent load per iteration would cost a
  // memory latency per kAlignThreads ints).
  int ev[kIdBatch];
#pragma unroll
  for (int u = 0; u < kIdBatch; ++u)
    ev[u] = local_expert(a.topk_ids, begin + (int64_t)u * blockDim.x + threadIdx.x, end,
                         a.expert_begin, E);
  for (int x0 = threadIdx.x; x0 < nc * E; x0 += blockDim.x * kStageBatch) {
    int v[kStageBatch];
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int x = x0 + u * (int)blockDim.x;
      v[u] = x < nc * E ? a.chunk_counts[x] : 0;
    }
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int x = x0 + u * (int)blockDim.x;
      if (x < nc * E) counts[x] = v[u];
    }
  }
  for (int x = threadIdx.x; x < 4 * E; x += blockDim.x) wcnt[x] = 0;
  __syncthreads();
  // Thread t owns experts [t*per, t*per + per): count over all chunks, count
  // over the chunks before this one, then a workgroup scan of padded sizes.
  const int per = (E + kAlignThreads - 1) / kAlignThreads;
  const int e0 = threadIdx.x * per;
  int mine = 0;
  for (int q = 0; q < per; ++q) {
    const int e = e0 + q;
    if (e >= E) break;
    // Eight independent LDS reads per step (a plain loop waits for each).
    int tot = 0, before = 0;
    for (int c0 = 0; c0 < nc; c0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c0 + u < nc ? counts[(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        before += c0 + u < b ? v[u] : 0;
        tot += v[u];
      }
    }
    running[e] = before;
    seg[e] = tot;
    mine += (tot + bm - 1) / bm * bm;
  }
  int total;
  int start = block_exclusive_scan(mine, tmp, &total);
  const int32_t sentinel = (int32_t)a.n;
  for (int q = 0; q < per; ++q) {
    const int e = e0 + q;
    if (e >= E) break;
    const int cnt = seg[e];
    const int padded = (cnt + bm - 1) / bm * bm;
    if (e % nc == b)
      for (int p = start + cnt; p < start + padded; ++p) a.sorted_ids[p] = sentinel;
    seg[e] = start;
    running[e] += start;
    start += padded;
  }
  if (threadIdx.x == 0) seg[E] = total;
  __syncthreads();
  if (b == 0 && threadIdx.x == 0) *a.ntpp = total;
  const int64_t gt = (int64_t)b * blockDim.x + threadIdx.x;
  const int64_t gs = (int64_t)gridDim.x * blockDim.x;
  const int64_t used_blocks = total / bm;
  for (int64_t blk = gt; blk < used_blocks; blk += gs) {
    // the expert whose segment holds row blk*bm: first i with seg[i] > row, minus one
    const int64_t row = blk * bm;
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (seg[mid] > row) hi = mid;
      else lo = mid + 1;
    }
    a.expert_ids[blk] = lo - 1;
  }
  const int64_t all_blocks = (a.max_padded + bm - 1) / bm;
  for (int64_t blk = used_blocks + gt; blk < all_blocks; blk += gs) a.expert_ids[blk] = -1;
  for (int64_t p = total + gt; p < a.max_padded; p += gs) a.sorted_ids[p] = sentinel;
  for (int64_t base0 = begin; base0 < end; base0 += (int64_t)blockDim.x * kIdBatch) {
    if (base0 != begin) {  // later batches (chunks above kIdBatch rounds)
#pragma unroll
      for (int u = 0; u < kIdBatch; ++u)
        ev[u] = local_expert(a.topk_ids, base0 + (int64_t)u * blockDim.x + threadIdx.x, end,
                             a.expert_begin, E);
    }
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int64_t base = base0 + (int64_t)u * blockDim.x;
      if (base >= end) break;  // uniform
      scatter_round(ev[u], base + threadIdx.x, E, running, wcnt, a.sorted_ids);
    }
  }
}

}  // namespace

hipError_t launch_align(const AlignArgs& a, hipStream_t stream) {
  const int E = a.num_experts;
  if (align_single_workgroup(a.n, E)) {
    const size_t lds = (size_t)(17 * E + 17) * sizeof(int);
    hipLaunchKernelGGL(align_single, dim3(1), dim3(1024), lds, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(align_count, dim3(a.nchunks), dim3(kAlignThreads), (size_t)E * sizeof(int),
                     stream, a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds = ((size_t)a.nchunks * E + 6 * (size_t)E + 18) * sizeof(int);
  hipLaunchKernelGGL(align_scatter, dim3(a.nchunks), dim3(kAlignThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace chord
