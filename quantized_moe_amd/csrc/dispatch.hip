// Dispatch of routed token rows into the grouped layouts: the permute-gather
// in front of the grouped GEMMs ("vLLM x Novita AI: Chord W4A16 INT4 MoE
// Kernel fuer Kimi K2.x", section "Gruppierte SM90-Kernel", Abb. 3).  Both
// layouts start from the stable per-expert alignment (align.hip): the
// contiguous layout is the alignment with 128-row blocks, its blocks becoming
// m_indices and its slots the gathered rows; the masked layout puts each slot
// at its rank inside its expert (ranks from max_m on are dropped and counted).
//
// HBM-bound copies: one workgroup per output row (a row is H*2 bytes, 14 KiB
// for the 7168-wide hidden size), 16-byte loads and stores, grid-stride over
// the rows so the grid does not depend on the device-side row count.
#include "device_common.h"

namespace chord {
namespace {

__device__ __forceinline__ int64_t used_rows(const DispatchArgs& a) {
  const int64_t t = *a.ntpp;
  return t < 0 ? 0 : (t > a.max_padded ? a.max_padded : t);
}

// Block-uniform row copy (or zero fill when src is null).  All loads of a
// thread's pieces (up to 4 per 1024-piece span) are issued before the first
// store, so each thread keeps several 16-byte loads in flight instead of one
// dependent load/store pair at a time.
constexpr int kThreads = 256;
constexpr int kPieces = 4;

__device__ __forceinline__ void copy_row(const uint16_t* __restrict__ src,
                                         uint16_t* __restrict__ dst, int nvec) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int v0 = threadIdx.x; v0 < nvec; v0 += kThreads * kPieces) {
    uint4 buf[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const int v = v0 + u * kThreads;
      buf[u] = make_uint4(0u, 0u, 0u, 0u);
      if (src != nullptr && v < nvec) buf[u] = s[v];
    }
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const int v = v0 + u * kThreads;
      if (v < nvec) d[v] = buf[u];
    }
  }
}

// Slots whose expert is not local map to no row.
__device__ __forceinline__ void mark_nonlocal(const DispatchArgs& a, int64_t gtid, int64_t gsz) {
  const int64_t n = (int64_t)a.T * a.k;
  for (int64_t i = gtid; i < n; i += gsz) {
    const int e = a.topk_ids[i] - a.expert_begin;
    if (e < 0 || e >= a.num_experts) a.flat_to_row[i] = -1;
  }
}

__global__ __launch_bounds__(kThreads) void gather_contiguous(DispatchArgs a) {
  const int nvec = a.H >> 3;
  const int64_t n = (int64_t)a.T * a.k;
  const int64_t used = used_rows(a);
  for (int64_t r = blockIdx.x; r < used; r += gridDim.x) {
    const int64_t f = a.sorted_ids[r];
    const int e = a.expert_ids[r / a.block_m];
    const bool valid = f >= 0 && f < n && e >= 0 && e < a.num_experts;
    copy_row(valid ? a.x + (f / a.k) * a.H : nullptr, a.out + r * a.H, nvec);
    if (threadIdx.x == 0) {
      a.m_indices[r] = valid ? e : -1;
      if (valid) a.flat_to_row[f] = (int32_t)r;
    }
  }
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gsz = (int64_t)gridDim.x * blockDim.x;
  for (int64_t r = used + gtid; r < a.max_rows; r += gsz) a.m_indices[r] = -1;
  mark_nonlocal(a, gtid, gsz);
  if (gtid == 0) *a.num_rows = (int32_t)used;
}

// First alignment block of local expert e among the used blocks [0, nb)
// (their expert ids ascend), or -1 if e has none.
__device__ __forceinline__ int first_block(const int32_t* expert_ids, int nb, int e) {
  int lo = 0, hi = nb;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (expert_ids[mid] < e) lo = mid + 1;
    else hi = mid;
  }
  return lo < nb && expert_ids[lo] == e ? lo : -1;
}

__global__ void clear_counter(int32_t* p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0;
}

__global__ __launch_bounds__(kThreads) void gather_masked(DispatchArgs a) {
  const int nvec = a.H >> 3;
  const int64_t n = (int64_t)a.T * a.k;
  const int64_t used = used_rows(a);
  const int nb = (int)(used / a.block_m);
  for (int64_t r = blockIdx.x; r < used; r += gridDim.x) {
    const int64_t f = a.sorted_ids[r];
    const int e = a.expert_ids[r / a.block_m];
    if (f < 0 || f >= n || e < 0 || e >= a.num_experts) continue;  // padding slot
    const int fb = first_block(a.expert_ids, nb, e);
    if (fb < 0) continue;
    const int64_t rank = r - (int64_t)fb * a.block_m;
    if (rank < a.max_m)
      copy_row(a.x + (f / a.k) * a.H, a.out + ((int64_t)e * a.max_m + rank) * a.H, nvec);
    if (threadIdx.x != 0) continue;
    a.flat_to_row[f] = rank < a.max_m ? (int32_t)((int64_t)e * a.max_m + rank) : -1;
    // The expert's last slot (followed by padding, another expert or the end)
    // writes the row count and adds the overflow.
    const bool last = r + 1 >= used || a.sorted_ids[r + 1] >= n ||
                      a.expert_ids[(r + 1) / a.block_m] != e;
    if (last) {
      const int64_t count = rank + 1;
      a.masked_m[e] = (int32_t)(count < a.max_m ? count : a.max_m);
      if (count > a.max_m) atomicAdd(a.dropped, (int32_t)(count - a.max_m));
    }
  }
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gsz = (int64_t)gridDim.x * blockDim.x;
  mark_nonlocal(a, gtid, gsz);
  for (int64_t e = gtid; e < a.num_experts; e += gsz)
    if (first_block(a.expert_ids, nb, (int)e) < 0) a.masked_m[e] = 0;
}

// Enough workgroups to keep every CU streaming, few enough that the row-count
// independent tails (m_indices fill, non-local slots) stay short.
unsigned dispatch_grid(int64_t rows) {
  const int64_t g = rows < 1 ? 1 : (rows > 2048 ? 2048 : rows);
  return (unsigned)g;
}

}  // namespace

hipError_t launch_gather_contiguous(const DispatchArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(gather_contiguous, dim3(dispatch_grid(a.max_padded)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_gather_masked(const DispatchArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(clear_counter, dim3(1), dim3(64), 0, stream, a.dropped);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gather_masked, dim3(dispatch_grid(a.max_padded)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace chord
