// Expert GEMMs of the W4A16 MoE layer for gfx950, the device-side tile
// builder that turns each routing layout into a list of (expert, rows) tiles,
// and the weighted top-k combine.
//
// Dequantisation keeps the bf16 rounding of (q - 8) * s exactly (the pages'
// subtract-then-scale order, "vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel
// fuer Kimi K2.x", section "H200 und Blackwell indexierter Decode"):
//   * two codes become the fp16 halves 1024 + q of one register with one shift
//     and one mask-or (magic exponent 0x6400);
//   * v_fma_mix_f32 computes (1024 + q) * s - 1032 * s in one rounding, which
//     is exactly (q - 8) * s since that product has at most 11 significant bits;
//   * v_cvt_pk_bf16_f32 rounds two results to bf16, nearest-even.
// The bf16 operands feed v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
#include "internal.h"

namespace chord {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// 8 codes of one packed word -> 8 bf16 weights (q - 8) * s, exact RNE.
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w, float s, float c) {
  uint32_t r[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t m = ((w >> (4 * v)) & 0x000F000Fu) | 0x64006400u;
    const half2_t h = __builtin_bit_cast(half2_t, m);
    const float lo = __builtin_fmaf((float)h[0], s, c);
    const float hi = __builtin_fmaf((float)h[1], s, c);
    r[v] = pk_bf16(lo, hi);
  }
  bf16x8_t out;
  __builtin_memcpy(&out, r, sizeof(out));
  return out;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Row mapping of one tile row: the B source row and the output row, or -1.
struct RowMap {
  int64_t src;  // row index into bsrc
  int64_t dst;  // row index into out
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
      m.src = R;
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

// ---------------------------------------------------------------------------
// Weight-streaming GEMM.  A workgroup of WK waves owns NT 16-row weight tiles
// of one expert and all rows (up to MT*16) of one token tile; the waves split
// K and reduce through LDS.  Each lane streams 16 bytes of packed codes plus
// one scale per 16-row tile and 128-wide K chunk straight from HBM into
// registers (one scale group per lane), dequantises, and issues 4 MFMAs per
// token tile.  The token operand comes straight from global memory (L2).
// Workgroups are persistent: they stride over (tile, weight-tile group) items.
// ---------------------------------------------------------------------------
template <int NT, int MT, int WK, int PF>
__global__ __launch_bounds__(64 * WK) void gemm_skinny(GemmArgs a) {
  extern __shared__ float red[];  // [WK][NT*MT][64][4]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int col = lane & 15;
  const int n_items = a.status->ntiles * a.items_per_tile;
  const int c_lo = (a.n_chunks * wave) / WK;
  const int c_hi = (a.n_chunks * (wave + 1)) / WK;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int ti = item / a.items_per_tile;
    const int ng = item % a.items_per_tile;
    const TileDesc td = a.tiles[ti];
    const int e = td.expert;

    // Token operand rows of this lane (one column per 16-row token tile).
    const uint16_t* src[MT];
    int64_t dst[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + col;
      src[mt] = nullptr;
      dst[mt] = -1;
      if (m < td.nrows) {
        const RowMap rm = map_row(a, e, (int64_t)td.row_begin + m);
        if (rm.src >= 0) {
          src[mt] = a.bsrc + rm.src * (int64_t)a.K + q * kGroup;
          dst[mt] = rm.dst;
        }
      }
    }
    bool mt_live[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) mt_live[mt] = mt * 16 < td.nrows;

    const uint8_t* wbase[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      wbase[nt] = a.wpack +
                  ((int64_t)e * a.n_tiles + (int64_t)ng * NT + nt) * a.n_chunks * kBlockBytes;

    f32x4_t acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 wq[PF][NT];
    uint32_t sc[PF][NT];
    uint4 xb[PF][MT][4];

    auto load = [&](int p, int c) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint8_t* b = wbase[nt] + (int64_t)c * kBlockBytes;
        wq[p][nt] = *reinterpret_cast<const uint4*>(b + lane * 16);
        sc[p][nt] = *reinterpret_cast<const uint16_t*>(b + kBlockWeightBytes + lane * 2);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (src[mt] != nullptr)
            xb[p][mt][s] = *reinterpret_cast<const uint4*>(src[mt] + c * kChunkK + s * 8);
          else
            xb[p][mt][s] = make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto compute = [&](int p) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float s = bf16_to_f32(sc[p][nt]);
        const float cc = -1032.0f * s;
        const uint32_t wv[4] = {wq[p][nt].x, wq[p][nt].y, wq[p][nt].z, wq[p][nt].w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8_t av = dequant_word(wv[st], s, cc);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if (mt_live[mt])
              acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(xb[p][mt][st]),
                                                                    acc[nt][mt], 0, 0, 0);
          }
        }
      }
    };

#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (c_lo + p < c_hi) load(p, c_lo + p);
    for (int c = c_lo; c < c_hi; c += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        if (c + p < c_hi) {
          compute(p);
          if (c + p + PF < c_hi) load(p, c + p + PF);
        }
      }
    }

    // Cross-wave K reduction.
    if (WK > 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          float* r = red + (((size_t)wave * NT * MT + nt * MT + mt) * 64 + lane) * 4;
          *reinterpret_cast<f32x4_t*>(r) = acc[nt][mt];
        }
      __syncthreads();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if ((nt * MT + mt) % WK != wave) continue;
          f32x4_t sum = f32x4_t{0.f, 0.f, 0.f, 0.f};
          for (int w = 0; w < WK; ++w)
            sum += *reinterpret_cast<const f32x4_t*>(
                red + (((size_t)w * NT * MT + nt * MT + mt) * 64 + lane) * 4);
          acc[nt][mt] = sum;
        }
    }

    // Epilogue.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int tw = ng * NT + nt;  // weight tile index inside the expert
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (WK > 1 && (nt * MT + mt) % WK != wave) continue;
        if (dst[mt] < 0) continue;
        const f32x4_t v = acc[nt][mt];
        if (a.gate_up) {
          const int f0 = tw * 8 + 2 * q;
          const uint32_t hv = pk_bf16(silu_mul(v[0], v[1]), silu_mul(v[2], v[3]));
          *reinterpret_cast<uint32_t*>(a.out + dst[mt] * (int64_t)a.out_ld + f0) = hv;
        } else {
          const int n0 = tw * 16 + 4 * q;
          float rw = 1.0f;
          if (a.row_weights != nullptr) rw = a.row_weights[dst[mt]];
          const uint2 o = make_uint2(pk_bf16(v[0] * rw, v[1] * rw), pk_bf16(v[2] * rw, v[3] * rw));
          *reinterpret_cast<uint2*>(a.out + dst[mt] * (int64_t)a.out_ld + n0) = o;
        }
      }
    }
    if (WK > 1) __syncthreads();  // LDS reuse by the next item
  }
}

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
__device__ int block_scan_excl(int v, int* tmp, int* total) {
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

__global__ __launch_bounds__(1024) void build_tiles(TileBuildArgs a) {
  __shared__ int first[kMaxExperts];
  __shared__ int last[kMaxExperts];
  __shared__ int nblk[kMaxExperts];
  __shared__ int tmp[16];
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

  // Segments owned by this thread: (start row, rows) pairs, enumerated twice.
  int my_tiles = 0;
  if (a.layout == kIndexed) {
    int64_t ntpp = *a.ntpp;
    const int64_t nb_cap = (a.max_padded + a.block_m - 1) / a.block_m;
    if (ntpp < 0 || ntpp > a.max_padded || ntpp % a.block_m != 0) {
      if (a.validate) atomicOr(&err, 4);
      ntpp = ntpp < 0 ? 0 : (ntpp > a.max_padded ? a.max_padded : ntpp);
    }
    const int64_t nb = min(ntpp / a.block_m, nb_cap);
    for (int64_t b = tid; b < nb; b += blockDim.x) {
      const int e = a.expert_ids[b];
      if (e < 0 || e >= E) {
        if (a.validate) atomicOr(&err, 1);
        continue;
      }
      atomicMin(&first[e], (int)b);
      atomicMax(&last[e], (int)b);
      atomicAdd(&nblk[e], 1);
    }
    __syncthreads();
    if (tid < E && last[tid] >= 0) {
      const int nbk = last[tid] - first[tid] + 1;
      if (nbk != nblk[tid] && a.validate) atomicOr(&err, 2);
      my_tiles = (nbk * a.block_m + TOK - 1) / TOK;
    }
  } else if (a.layout == kMasked) {
    if (tid < E) {
      int m = a.masked_m[tid];
      if ((m < 0 || m > a.max_m) && a.validate) atomicOr(&err, 32);
      m = m < 0 ? 0 : (m > a.max_m ? a.max_m : m);
      first[tid] = m;  // rows
      my_tiles = (m + TOK - 1) / TOK;
    }
  } else {
    // contiguous: thread handles chunks [c0, c1)
    const int nch = (int)(a.M / 128);
    const int per = (nch + blockDim.x - 1) / blockDim.x;
    const int c0 = tid * per, c1 = min(nch, c0 + per);
    for (int c = c0; c < c1; ++c) {
      const int e = a.m_indices[(int64_t)c * 128];
      if (e < 0 || e >= E) {
        if (e != -1 && a.validate) atomicOr(&err, 8);
        continue;
      }
      int lastv = 0;
      for (int r = 0; r < 128; ++r) {
        const int v = a.m_indices[(int64_t)c * 128 + r];
        if (v == e) lastv = r + 1;
        else if (a.validate && v != -1) atomicOr(&err, (v < -1 || v >= E) ? 8 : 16);
      }
      my_tiles += (lastv + TOK - 1) / TOK;
    }
  }
  int total;
  int base = block_scan_excl(my_tiles, tmp, &total);
  if (total > a.max_tiles && a.validate) atomicOr(&err, 64);

  auto emit = [&](int expert, int row_begin, int rows) {
    for (int r = 0; r < rows; r += TOK) {
      if (base < a.max_tiles) a.tiles[base] = TileDesc{expert, row_begin + r, min(TOK, rows - r), 0};
      ++base;
    }
  };
  if (a.layout == kIndexed) {
    if (tid < E && last[tid] >= 0)
      emit(tid, first[tid] * a.block_m, (last[tid] - first[tid] + 1) * a.block_m);
  } else if (a.layout == kMasked) {
    if (tid < E && first[tid] > 0) emit(tid, tid * a.max_m, first[tid]);
  } else {
    const int nch = (int)(a.M / 128);
    const int per = (nch + blockDim.x - 1) / blockDim.x;
    const int c0 = tid * per, c1 = min(nch, c0 + per);
    for (int c = c0; c < c1; ++c) {
      const int e = a.m_indices[(int64_t)c * 128];
      if (e < 0 || e >= E) continue;
      int lastv = 0;
      for (int r = 0; r < 128; ++r)
        if (a.m_indices[(int64_t)c * 128 + r] == e) lastv = r + 1;
      emit(e, c * 128, lastv);
    }
  }
  __syncthreads();
  if (tid == 0) {
    a.status->ntiles = min(total, a.max_tiles);
    a.status->error = err;
  }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = bf16(sum over slots j with a row, ascending j, of
// w[t,j] * y_row), fp32 accumulation; tokens without a local slot get 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const int nvec = a.H / 8;
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.k; ++j) {
      int64_t row;
      if (a.flat_to_row != nullptr) {
        row = a.flat_to_row[(int64_t)t * a.k + j];
        if (row < 0 || row >= a.n_rows) continue;
      } else {
        const int e = a.topk_ids[(int64_t)t * a.k + j] - a.expert_begin;
        if (e < 0 || e >= a.num_experts) continue;
        row = (int64_t)t * a.k + j;
      }
      const float w = a.topk_weights[(int64_t)t * a.k + j];
      const uint4 y = *reinterpret_cast<const uint4*>(a.rows + row * a.H + v * 8);
      const uint32_t yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w * bf16_to_f32(yw[i] & 0xFFFFu);
        acc[2 * i + 1] += w * bf16_to_f32(yw[i] >> 16);
      }
    }
    const uint4 o = make_uint4(pk_bf16(acc[0], acc[1]), pk_bf16(acc[2], acc[3]),
                               pk_bf16(acc[4], acc[5]), pk_bf16(acc[6], acc[7]));
    *reinterpret_cast<uint4*>(a.out + (int64_t)t * a.H + v * 8) = o;
  }
}

__global__ void zero_kernel(uint16_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

template <int NT, int MT, int WK, int PF>
hipError_t launch_skinny_t(const GemmArgs& a, int grid, hipStream_t stream) {
  const size_t lds = WK > 1 ? (size_t)WK * NT * MT * 64 * 4 * sizeof(float) : 0;
  hipLaunchKernelGGL((gemm_skinny<NT, MT, WK, PF>), dim3(grid), dim3(64 * WK), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_tiles(const TileBuildArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(build_tiles, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

// kernel 1 = skinny.  mt = token tiles of 16 per workgroup; the caller sets
// a.tiles_per_item to the NT of the instance (2).
hipError_t launch_gemm(int kernel, int mt, const GemmArgs& a, int grid, hipStream_t stream) {
  (void)kernel;
  switch (mt) {
    case 1: return launch_skinny_t<2, 1, 4, 2>(a, grid, stream);
    case 2: return launch_skinny_t<2, 2, 4, 2>(a, grid, stream);
    case 3: return launch_skinny_t<2, 3, 4, 2>(a, grid, stream);
    case 4: return launch_skinny_t<2, 4, 4, 2>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_zero(uint16_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace chord
