/*
 * chord.h -- C ABI of libchord.so, a W4A16 mixture-of-experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer: BF16 activations, unsigned 4-bit weight codes with one BF16 scale
 * per group of 32 along K, dequantised as (q - 8) * s.  Each routed row goes
 * through its expert's gate_up GEMM, SiLU(gate) * up, and the down GEMM; the
 * rows of a token are then combined with its top-k routing weights.
 *
 * Sources (cited by page title and section):
 *   [Novita]  "vLLM x Novita AI: Chord W4A16 INT4 MoE Kernel fuer Kimi K2.x"
 *   [aihirek] "A Novita AI uj INT4 MoE-kernelt nyilt forraskodova tett a Kimi
 *             K2.x-hez"
 *   [picx]    "vLLM and Novita AI Announce Chord, an INT4 MoE Backend for
 *             Kimi K2.x"
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates device memory on the layer path and never frees caller
 *     memory.  Scratch memory is a caller-provided workspace whose size is
 *     given by the matching *_workspace_bytes query.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*, NULL = default stream).  Results are valid after the stream
 *     synchronises.  There is no host synchronisation unless
 *     CHORD_FLAG_VALIDATE is set, so the default path can be captured into a
 *     hipGraph.
 *   - chord_bf16 is the raw bit pattern of a bfloat16.  Index tensors are
 *     int32.  Routing weights are fp32.  All tensors are row-major and
 *     contiguous.
 *   - Every call returns a chord_status.  Errors that the host can detect
 *     (null pointers, bad sizes, wrong weight mode, small workspace) are
 *     returned BEFORE anything is enqueued; chord_last_error() then describes
 *     the failure (thread-local).  Calls are thread-safe.
 *   - Only gfx950 devices are supported; other devices give
 *     CHORD_ERR_UNSUPPORTED.
 */
#ifndef CHORD_H_
#define CHORD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t chord_bf16;

typedef enum {
  CHORD_OK = 0,
  CHORD_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, expected_m <= 0, override on a grouped call */
  CHORD_ERR_UNSUPPORTED = 2,      /* group size != 32, K % 128 != 0, odd shapes, non-gfx950 device */
  CHORD_ERR_LAYOUT_MISMATCH = 3,  /* weight packed for another mode or role */
  CHORD_ERR_WORKSPACE = 4,        /* workspace missing or too small */
  CHORD_ERR_ROUTING = 5,          /* CHORD_FLAG_VALIDATE found bad routing tensors */
  CHORD_ERR_HIP = 6               /* a HIP runtime call or launch failed */
} chord_status;

/* Entry-point modes.  The mode a weight was packed for is recorded in its
 * handle and checked at dispatch: feeding a weight packed for one mode to
 * another mode's entry point fails loudly ([Novita] §"Gruppierte SM90-Kernel"). */
typedef enum {
  CHORD_MODE_INDEXED = 0,
  CHORD_MODE_CONTIGUOUS = 1,
  CHORD_MODE_MASKED = 2
} chord_mode;

/* Role of a packed weight inside the layer. */
typedef enum {
  CHORD_ROLE_GATE_UP = 0, /* W13: N = 2*I rows, gate rows [0,I) then up rows [I,2I); K = H */
  CHORD_ROLE_DOWN = 1     /* W2:  N = H rows; K = I */
} chord_role;

/* Flags (bitmask). */
#define CHORD_FLAG_VALIDATE 1u /* check routing tensors on the device and read back one error word
                                  ("trusted routing validation" on, [Novita] §"vLLM-Integration") */

#define CHORD_WEIGHT_MAGIC 0x43573441u /* "CW4A" */
#define CHORD_WEIGHT_VERSION 1u

/* Host handle of a packed weight.  `data` is caller-owned device memory of
 * `bytes` bytes written by chord_w4a16_pack. */
typedef struct {
  uint32_t magic;
  uint32_t version;
  int32_t mode;       /* chord_mode */
  int32_t role;       /* chord_role */
  int32_t num_experts;
  int32_t n;          /* output rows per expert */
  int32_t k;          /* reduction length */
  int32_t group_size; /* always 32 */
  void* data;
  size_t bytes;
} chord_w4a16_weight;

/* Optional schedule override for the indexed entry point (NULL = planner).
 * Grouped entry points reject any override ([Novita] §"Gruppierte SM90-Kernel":
 * the grouped dispatch does not accept indexed block_m / tuning overrides). */
typedef struct {
  int32_t kernel;      /* 0 auto, 1 weight-streaming GEMMs, 2 LDS-tiled GEMMs (needs
                          I a multiple of 32, else kernel 1 runs; tiles of up to
                          192 token rows; the nt/wk/prefetch/tokens fields are
                          then ignored), 3 both: experts with >= 48 rows take the
                          tiled GEMMs (on an internal side stream, joined back
                          to the caller's stream), the others the streaming
                          GEMMs; 4 / 5: the LDS-tiled GEMMs in their single-role
                          form (every wave dequantises and multiplies) / their
                          producer-consumer form (K > 256: 8 waves only issue
                          MFMAs on LDS operands, 4 waves load and dequantise;
                          tiles of up to 176 rows), where kernel 2 lets the
                          planner choose; both forms give bit-identical results */
  int32_t tokens;      /* rows per token tile of kernel 1: 16 or 32; 0 auto */
  int32_t gate_up_nt;  /* 16-row weight tiles per wave in the gate_up GEMM: 2 or 4; 0 auto */
  int32_t gate_up_wk;  /* waves splitting K in the gate_up GEMM: 1, 2 or 4; 0 auto */
  int32_t down_nt;     /* as above for the down GEMM */
  int32_t down_wk;
  int32_t prefetch;    /* K chunks in flight per wave: 2 or 4; 0 auto */
  int32_t tile_split;  /* 1: no K split of outsized tiles in the tiled GEMMs (each output is
                          then summed over K in one pass, in chunk order); 0 auto: a tile
                          with far more rows than the call's mean is split along K into up
                          to 4 parts whose fp32 partials the last part adds in part order */
} chord_schedule;

/* ---------------------------------------------------------------------------
 * Status and diagnostics
 * ------------------------------------------------------------------------- */

/* Static name of a status code. */
const char* chord_status_string(chord_status s);

/* Details of the last error on the calling thread ("" if none). */
const char* chord_last_error(void);

/* Writes a NUL-terminated description of the last schedule chosen on this
 * thread (kernel, tile sizes, grid) into buf[0..n).  Returns CHORD_OK, or
 * CHORD_ERR_INVALID_ARGUMENT if buf is NULL or n == 0. */
chord_status chord_last_plan(char* buf, size_t n);

/* The schedule a layer call would choose, computed on the host alone: no GPU,
 * no HIP call.  Describes a call by its mode (CHORD_MODE_*), T and k (indexed
 * and contiguous; ignored for masked), the global expert count (indexed), the
 * local expert count E_l, H, I, a size hint (indexed: block_m; contiguous:
 * valid_m_hint; masked: expected_m), its internal rows (indexed: max_padded;
 * contiguous: M; masked: E_l * max_m) and the compute units to plan for
 * (0: the MI355X's 256).  An override (indexed only, may be NULL) is applied
 * as the layer call applies it.  Writes "<mode>: <plan>" in the format of
 * chord_last_plan into buf[0..n).  Returns CHORD_OK or
 * CHORD_ERR_INVALID_ARGUMENT (bad descriptor, override out of range, NULL
 * buf or n == 0). */
chord_status chord_w4a16_moe_plan(int mode, int T, int k, int num_global_experts, int E_l, int H,
                                  int I, int hint, int64_t rows, int num_cus,
                                  const chord_schedule* override, char* buf, size_t n);

/* Library version string. */
const char* chord_version(void);

/* Kernel timing for diagnostics and benchmarks.  While enabled, every layer
 * call records HIP events on its own stream around its four kernel stages:
 * [0] tile builder, [1] gate_up GEMM (+SiLU*mul), [2] down GEMM, [3] combine
 * (zero time for grouped calls without a token combine).  chord_profile_read
 * synchronises the recorded events and returns the summed milliseconds per
 * stage and the number of calls since the last reset.  Enabling adds four
 * event records per call; it never synchronises inside a layer call. */
chord_status chord_profile_enable(int on);
chord_status chord_profile_reset(void);
chord_status chord_profile_read(double* stage_ms /* [4] */, int64_t* calls);

/* ---------------------------------------------------------------------------
 * Weight packing (load time, not on the layer path)
 * ------------------------------------------------------------------------- */

/* Bytes of device memory chord_w4a16_pack writes for E experts of an [N, K]
 * weight; 0 if the shape is unsupported. */
size_t chord_w4a16_packed_bytes(int mode, int role, int E, int N, int K);

/*
 * Repacks a W4A16 weight into the library's gfx950 layout.
 *
 * qweight: device, int32 [E, N, K/8]; code k of a row is bits 4*(k%8)..+3 of
 *          word k/8 (low nibble first, 8 codes per int32 along K).
 * scales:  device, bf16 [E, N, K/32]; weight = (code - 8) * scale.
 * role:    CHORD_ROLE_GATE_UP (N = 2*I, gate rows first) or CHORD_ROLE_DOWN.
 * dst:     device buffer of at least chord_w4a16_packed_bytes(...) bytes,
 *          caller-owned; it must outlive every layer call that uses `handle`.
 * handle:  host struct filled on success.
 *
 * Supported: group_size == 32, K % 128 == 0, N % 16 == 0 (GATE_UP: I % 8 == 0),
 * E >= 1.  Other quantisation schemes fail here instead of selecting a wrong
 * kernel ([picx]; [Novita] §"vLLM-Integration").  Enqueued on `stream`.
 */
chord_status chord_w4a16_pack(int mode, int role, const int32_t* qweight, const chord_bf16* scales,
                              int E, int N, int K, int group_size, void* dst, size_t dst_bytes,
                              chord_w4a16_weight* handle, void* stream);

/* ---------------------------------------------------------------------------
 * Routing alignment (indexed layout)
 * ------------------------------------------------------------------------- */

/* Minimum sorted_ids length: T*k + E_l*(block_m - 1), a bound that holds for
 * any routing (every slot local, every expert ending in a partial block).  The
 * indexed layer consumes buffers of this oversize length as they are, without
 * reading the routed count back to the host ([Novita] §"vLLM-Integration":
 * the indexed fast path takes the oversize alignment buffers with trusted
 * routing validation off and stays graph-capturable).  Returns 0 for bad
 * arguments (T < 0, k < 1, num_local_experts < 1, block_m < 1). */
int64_t chord_moe_align_max_padded(int T, int k, int num_local_experts, int block_m);

/* Workspace bytes chord_moe_align needs for these sizes. */
size_t chord_moe_align_workspace_bytes(int T, int k, int num_local_experts, int block_m);

/*
 * Aligns routed (token, slot) pairs per local expert for the indexed layer
 * ([Novita] §"Zwei Kernel-Familien" and Abb. 3: activations stay unpadded, the
 * index list carries a padding sentinel; [aihirek] §"Ket kulon kernelcsalad").
 *
 * topk_ids:  device int32 [T, k], global expert ids.  Ids outside
 *            [expert_begin, expert_begin + num_local_experts) are not local
 *            and are left out.
 * sorted_ids: device int32 [max_padded] out.  Local flat ids i = t*k + j,
 *            grouped by local expert in ascending order, ascending i inside a
 *            group, each group padded to a multiple of block_m with the
 *            sentinel T*k; the rest of the buffer is the sentinel too.
 * expert_ids: device int32 [ceil(max_padded / block_m)] out: local expert
 *            index (0..E_l-1) of each block, -1 past the padded total.
 * num_tokens_post_padded: device int32 [1] out: the padded total.
 * max_padded: >= chord_moe_align_max_padded(T, k, E_l, block_m); larger
 *            (oversize) buffers are fine and need no host readback
 *            ([Novita] §"vLLM-Integration").
 * block_m:   16, 32, 64 or 128.
 * Output is deterministic and bit-identical to a stable counting sort.
 */
chord_status chord_moe_align(const int32_t* topk_ids, int T, int k, int expert_begin,
                             int num_local_experts, int block_m, int32_t* sorted_ids,
                             int32_t* expert_ids, int32_t* num_tokens_post_padded,
                             int64_t max_padded, void* workspace, size_t ws_bytes, uint32_t flags,
                             void* stream);

/* ---------------------------------------------------------------------------
 * Dispatch into the grouped layouts, and the combine back to tokens
 * ([Novita] §"Gruppierte SM90-Kernel" and Abb. 3: the grouped kernels take
 * activations already permuted per expert; [aihirek] §"Ket kulon
 * kernelcsalad").  Rows keep the alignment's stable order: ascending local
 * expert, ascending flat slot id i = t*k + j inside an expert.
 * ------------------------------------------------------------------------- */

/* Rows the contiguous dispatch needs: T*k + E_l*127 rounded up to 128. */
int64_t chord_moe_dispatch_contiguous_rows(int T, int k, int num_local_experts);

/* Workspace bytes of chord_moe_dispatch_contiguous (mode
 * CHORD_MODE_CONTIGUOUS) or chord_moe_dispatch_masked (CHORD_MODE_MASKED);
 * 0 for bad arguments. */
size_t chord_moe_dispatch_workspace_bytes(int mode, int T, int k, int num_local_experts);

/*
 * Permute-gather into the contiguous grouped layout: each local expert's
 * slots become a segment of rows padded to a multiple of 128 (the GEMM's
 * M-tile), segments in ascending expert order.
 *
 * x:          device bf16 [T, H], 16-byte aligned; H % 8 == 0.
 * topk_ids:   device int32 [T, k], global expert ids; local ones lie in
 *             [expert_begin, expert_begin + num_local_experts).
 * a:          device bf16 [max_rows, H] out, 16-byte aligned.  Rows below
 *             *num_rows hold x[t] of their slot, padding rows are 0; rows from
 *             *num_rows on are not written.
 * m_indices:  device int32 [max_rows] out: local expert of each row, -1 for
 *             padding and for every row from *num_rows on.
 * max_rows:   multiple of 128, >= chord_moe_dispatch_contiguous_rows(T, k,
 *             E_l) (a bound that holds for any routing, so the call needs no
 *             host readback).
 * flat_to_row: device int32 [T*k] out: row of each local slot, -1 for the
 *             others (the combine contract of chord_w4a16_moe_grouped_contiguous
 *             and chord_moe_combine).
 * num_rows:   device int32 [1] out: rows used, a multiple of 128.
 * workspace:  device, chord_moe_dispatch_workspace_bytes(CHORD_MODE_CONTIGUOUS,
 *             ...) bytes, caller-owned; holds the alignment between calls.
 * Enqueued on `stream`; outputs are deterministic.
 */
chord_status chord_moe_dispatch_contiguous(const chord_bf16* x, int T, int H,
                                           const int32_t* topk_ids, int k, int expert_begin,
                                           int num_local_experts, chord_bf16* a,
                                           int32_t* m_indices, int64_t max_rows,
                                           int32_t* flat_to_row, int32_t* num_rows,
                                           void* workspace, size_t ws_bytes, void* stream);

/*
 * Permute-gather into the masked grouped layout: slot number r (in the stable
 * order) of local expert e goes to a3[e, r] while r < max_m; later slots of a
 * hot expert are dropped, counted, and map to no row.
 *
 * x, topk_ids, H, expert_begin: as for the contiguous dispatch.
 * a3:         device bf16 [num_local_experts, max_m, H] out, 16-byte aligned;
 *             rows from masked_m[e] on are not written.
 * masked_m:   device int32 [num_local_experts] out: min(slots of e, max_m).
 * flat_to_row: device int32 [T*k] out: e*max_m + r for a kept slot, -1 for a
 *             dropped or non-local one.
 * dropped:    device int32 [1] out: slots dropped over all experts.
 * workspace:  chord_moe_dispatch_workspace_bytes(CHORD_MODE_MASKED, ...) bytes.
 * max_m >= 1; num_local_experts * max_m < 2^31.  Enqueued on `stream`.
 */
chord_status chord_moe_dispatch_masked(const chord_bf16* x, int T, int H, const int32_t* topk_ids,
                                       int k, int expert_begin, int num_local_experts, int max_m,
                                       chord_bf16* a3, int32_t* masked_m, int32_t* flat_to_row,
                                       int32_t* dropped, void* workspace, size_t ws_bytes,
                                       void* stream);

/*
 * Unpermute-combine: out[t] = bf16( sum over j with flat_to_row[t*k+j] in
 * [0, n_rows) of topk_weights[t,j] * rows[flat_to_row[t*k+j]] ), fp32
 * accumulation in ascending j: the weighted top-k sum that ends the MoE
 * layer, for the grouped layouts whose GEMMs stop at per-row outputs
 * ([Novita] §"Gruppierte SM90-Kernel").  Tokens with no such slot get 0.
 *
 * rows:       device bf16 [n_rows, H] (e.g. the masked layer's flat output),
 *             16-byte aligned; n_rows * H * 2 < 2^31.
 * flat_to_row: device int32 [T*k]; topk_weights: device fp32 [T, k].
 * out:        device bf16 [T, H], every row written.  Enqueued on `stream`.
 */
chord_status chord_moe_combine(const chord_bf16* rows, int64_t n_rows, int H,
                               const int32_t* flat_to_row, const float* topk_weights, int T,
                               int k, chord_bf16* out, void* stream);

/* ---------------------------------------------------------------------------
 * The layer
 * ------------------------------------------------------------------------- */

/* block_m the planner wants for an indexed call with these shapes (the caller
 * aligns with it before the layer call).  Token counts per expert, not total
 * tokens, decide the schedule ([Novita] TL;DR and §"H200 Prefill und TP8").
 *
 * Returns 0 when the call needs no alignment: the planner routes it inside
 * the GEMM (the weight-streaming kernels at T*k <= 2048 slots whose routing
 * tables, (4 E_l + 2 + 2 T*k) ints, fit 32 KB of LDS, e.g. decode and the
 * small TP slices): every workgroup of the gate_up launch derives
 * the rows of its expert from topk_ids itself, so the caller may skip
 * chord_moe_align and pass NULL alignment pointers (max_padded 0, block_m 0)
 * to chord_w4a16_moe_indexed.  This keeps the pages' contract of an indexed
 * path that needs no host readback ([Novita] §"vLLM-Integration") and drops
 * the alignment launch and its dependent index loads from the critical path
 * of the small calls. */
int chord_w4a16_moe_indexed_block_m(int T, int k, int E_g, int E_l, int H, int I);

/* Workspace bytes for a layer call.  rows = max_padded (indexed; 0 for a
 * call without alignment), M (contiguous) or E*max_m (masked); T and k are
 * used by the indexed mode.
 * The pages define no workspace; it exists so that a layer call allocates
 * nothing and reads nothing back, which keeps the default indexed path
 * capturable in a graph ([Novita] §"vLLM-Integration").  It holds the device
 * status words and tile list, h [rows, I] bf16 and, for the indexed mode, the
 * per-slot down outputs; the caller owns it and may reuse it across calls on
 * one stream.  Returns 0 for bad arguments. */
size_t chord_w4a16_moe_workspace_bytes(int mode, int T, int k, int E_l, int H, int I,
                                       int64_t rows);

/*
 * Indexed layer: out[t] = bf16( sum over local j of topk_weights[t,j] * y_tj ),
 * y_tj = W2_e( bf16( silu(W1_e x_t) * (W3_e x_t) ) ), e = topk_ids[t,j] - expert_begin.
 *
 * The indexed family ([Novita] §"Zwei Kernel-Familien": the path that takes
 * vLLM's sorted_ids / expert_ids / num_tokens_padded routing; §"Kernel-
 * Optimierungen / Indizierte Kernel": one family serving EP8 prefill, TP8
 * single-instance and EP8 decode, its schedule tuned by tokens per expert;
 * [aihirek] §"Ket kulon kernelcsalad").  Activations stay unpadded: padding
 * lives in the index list as the sentinel T*k (Abb. 3 of [Novita]).  The
 * alignment is consumed on the device, oversize buffers included, with no
 * host readback unless CHORD_FLAG_VALIDATE asks for the trusted-routing check
 * ([Novita] §"vLLM-Integration").
 *
 * x:        device bf16 [T, H].
 * w13, w2:  handles packed with CHORD_MODE_INDEXED, roles GATE_UP (N=2I, K=H)
 *           and DOWN (N=H, K=I), same number of experts E_l.
 * topk_ids, topk_weights: device [T, k] int32 / fp32.
 * num_global_experts: experts the router chooses from (E_g >= E_l; <= 0
 *           means E_l).  Host-side hint: T*k/E_g is the expected number of
 *           rows per expert that picks the schedule.
 * sorted_ids, expert_ids, num_tokens_post_padded, max_padded, block_m: the
 *           alignment (chord_moe_align's output contract); oversize buffers
 *           are consumed on the device without host readback.  Not read, and
 *           may be NULL / 0, when chord_w4a16_moe_indexed_block_m returns 0
 *           for these shapes and no schedule override is given (a routed
 *           call: the gate_up launch builds each expert's row list from
 *           topk_ids in LDS; with T <= 16 and T*k <= 64, and no down
 *           override, the down GEMM and the combine also run as one launch,
 *           summing w * y in fp32 without rounding y to bf16 first).
 * out:      device bf16 [T, H]; every row is written (rows of tokens with no
 *           local expert are 0).
 * override: NULL or a schedule override.
 * T == 0 is a no-op.  With CHORD_FLAG_VALIDATE the routing tensors are
 * checked on the device and CHORD_ERR_ROUTING is returned if any is invalid;
 * without it, invalid entries are skipped and never written out of bounds.
 */
chord_status chord_w4a16_moe_indexed(const chord_bf16* x, int T, int H, int I,
                                     const chord_w4a16_weight* w13, const chord_w4a16_weight* w2,
                                     const int32_t* topk_ids, const float* topk_weights, int k,
                                     int expert_begin, int num_global_experts,
                                     const int32_t* sorted_ids,
                                     const int32_t* expert_ids,
                                     const int32_t* num_tokens_post_padded, int64_t max_padded,
                                     int block_m, chord_bf16* out, void* workspace,
                                     size_t ws_bytes, const chord_schedule* override,
                                     uint32_t flags, void* stream);

/* Scratch bytes the allocation-free indexed entry point holds per GPU. */
#define CHORD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * Allocation-free variant of chord_w4a16_moe_indexed, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and error behaviour as chord_w4a16_moe_indexed, minus the
 * workspace: the call's scratch (status words, tile list, h and the per-slot
 * down outputs) lives in a static device array of CHORD_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that the library holds on each GPU it runs on, from the first such
 * call on that GPU until the process ends.  It calls no hipMalloc / hipFree
 * and creates no stream or event (the stage profiler is not recorded; a
 * kernel-3 schedule, which needs a side stream, is rejected).
 *
 * Limit: calls whose workspace (chord_w4a16_moe_workspace_bytes) exceeds
 * CHORD_NOALLOC_SCRATCH_BYTES return CHORD_ERR_WORKSPACE before anything is
 * enqueued; the decode EP share (T = 64, 48 of 384 experts, H = 7168,
 * I = 2048) and the TP slices up to T = 512 fit.
 *
 * Every allocation-free call on a GPU shares that GPU's array, and each call
 * rewrites what it reads (nothing has to start at zero): calls that overlap
 * on one GPU, from other streams or threads, race on it and must be
 * serialised by the caller.
 */
chord_status chord_w4a16_moe_indexed_noalloc(const chord_bf16* x, int T, int H, int I,
                                             const chord_w4a16_weight* w13,
                                             const chord_w4a16_weight* w2,
                                             const int32_t* topk_ids, const float* topk_weights,
                                             int k, int expert_begin, int num_global_experts,
                                             const int32_t* sorted_ids, const int32_t* expert_ids,
                                             const int32_t* num_tokens_post_padded,
                                             int64_t max_padded, int block_m, chord_bf16* out,
                                             const chord_schedule* override, uint32_t flags,
                                             void* stream);

/*
 * Grouped contiguous layer ([Novita] §"Gruppierte SM90-Kernel", Abb. 3): rows
 * concatenated per expert in segments padded to 128-row boundaries.
 *
 * a:          device bf16 [M, H]; M % 128 == 0.
 * m_indices:  device int32 [M]: local expert of each row, -1 for padding.
 *             Each 128-row chunk holds rows of one expert (padding at its end).
 * valid_m_hint: host heuristic (number of valid rows, or <= 0 if unknown).
 * row_weights: NULL or device fp32 [M]; multiplies each row's output.
 * out_rows:   device bf16 [M, H]: y of each valid row (times row_weights);
 *             padding rows are unspecified.
 * flat_to_row, topk_weights, out_tokens: NULL, or (device int32 [T*k],
 *             device fp32 [T, k], device bf16 [T, H]): also combine rows to
 *             tokens, out_tokens[t] = bf16(sum_j topk_weights[t,j] *
 *             out_rows[flat_to_row[t*k+j]]) over the slots with a row (>= 0).
 * override:   must be NULL.
 */
chord_status chord_w4a16_moe_grouped_contiguous(
    const chord_bf16* a, int64_t M, const int32_t* m_indices, int64_t valid_m_hint,
    const chord_w4a16_weight* w13, const chord_w4a16_weight* w2, int H, int I,
    const float* row_weights, const int32_t* flat_to_row, int T, int k, const float* topk_weights,
    chord_bf16* out_rows, chord_bf16* out_tokens, void* workspace, size_t ws_bytes,
    const chord_schedule* override, uint32_t flags, void* stream);

/*
 * Grouped masked layer ([Novita] §"Gruppierte SM90-Kernel", Abb. 3): a fixed
 * budget of max_m rows per expert.
 *
 * a:          device bf16 [E, max_m, H].
 * masked_m:   device int32 [E]: valid rows of each expert (authoritative).
 *             Values above max_m are clamped (CHORD_FLAG_VALIDATE: ROUTING).
 * expected_m: positive host hint used only to pick the launch; outputs do not
 *             depend on it.
 * row_weights: NULL or device fp32 [E, max_m].
 * out:        device bf16 [E*max_m, H], flat; rows past an expert's valid
 *             count are unspecified and must be ignored by the consumer.
 * override:   must be NULL.
 */
chord_status chord_w4a16_moe_grouped_masked(const chord_bf16* a, int E, int max_m,
                                            const int32_t* masked_m, int expected_m,
                                            const chord_w4a16_weight* w13,
                                            const chord_w4a16_weight* w2, int H, int I,
                                            const float* row_weights, chord_bf16* out,
                                            void* workspace, size_t ws_bytes,
                                            const chord_schedule* override, uint32_t flags,
                                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CHORD_H_ */
