// Host runtime of libchord.so: argument validation (before any HIP call, so
// misuse is reported without touching the device), the per-call schedule
// planner with its memoised plan cache, workspace layout, and the launch
// sequences of the three layer entry points.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "internal.h"

using namespace chord;

namespace {

thread_local std::string g_last_error;
thread_local std::string g_last_plan;

chord_status fail(chord_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

chord_status hip_fail(hipError_t e, const char* what) {
  return fail(CHORD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define CHORD_CHECK(expr)                    \
  do {                                       \
    chord_status _s = (expr);                \
    if (_s != CHORD_OK) return _s;           \
  } while (0)

#define HIP_TRY(expr, what)                       \
  do {                                            \
    hipError_t _e = (expr);                       \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// ---- device check ---------------------------------------------------------
struct DeviceInfo {
  bool checked = false;
  bool ok = false;
  int cus = 0;
  char arch[64] = {0};
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

chord_status check_device(int* cus) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(CHORD_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t p;
    HIP_TRY(hipGetDeviceProperties(&p, dev), "hipGetDeviceProperties");
    snprintf(d.arch, sizeof(d.arch), "%s", p.gcnArchName);
    d.ok = strncmp(p.gcnArchName, "gfx950", 6) == 0;
    d.cus = p.multiProcessorCount;
    d.checked = true;
  }
  if (!d.ok)
    return fail(CHORD_ERR_UNSUPPORTED, "device %d is %s; only gfx950 (MI355X) is supported", dev,
                d.arch);
  if (cus) *cus = d.cus;
  return CHORD_OK;
}

// ---- environment overrides (parsed once) ----------------------------------
struct EnvOverrides {
  int kernel = 0;
  int tokens = 0;
  int gu_nt = 0, gu_wk = 0, dn_nt = 0, dn_wk = 0;  // "nt,wk" per GEMM
  int tile_wgs = 0;  // tiled kernel: workgroups per CU
  int tile_waves = 0;  // tiled kernel (K > 256): waves per workgroup, 4 or 8
  int tile_pc = 0;     // tiled kernel (K > 256): 1 producer/consumer form, 0 off
  int tile_split = 0;  // tiled kernel: 1 turns the K split of outsized tiles off
  int stream_wgs = 0;  // streaming kernel: workgroups per CU (0: balanced default)
  int prefetch = 0;
  int routed = 1;  // 0: routed indexed calls off (every indexed call reads the alignment)
  int fused = 1;   // 0: routed calls of a few tokens keep a separate combine launch
  int stream_chain = 1;  // 0: streaming kernel restarts its load ring at every item
  bool log = false;
};
const EnvOverrides& env() {
  static EnvOverrides e = [] {
    EnvOverrides o;
    if (const char* s = getenv("CHORD_W4A16_KERNEL")) o.kernel = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_TOKENS")) o.tokens = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_GATE_UP")) sscanf(s, "%d,%d", &o.gu_nt, &o.gu_wk);
    if (const char* s = getenv("CHORD_W4A16_DOWN")) sscanf(s, "%d,%d", &o.dn_nt, &o.dn_wk);
    if (const char* s = getenv("CHORD_W4A16_TILE_WGS")) o.tile_wgs = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_TILE_WAVES")) o.tile_waves = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_TILE_PC")) o.tile_pc = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_TILE_SPLIT")) o.tile_split = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_STREAM_WGS")) o.stream_wgs = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_PREFETCH")) o.prefetch = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_ROUTED")) o.routed = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_FUSED")) o.fused = atoi(s);
    if (const char* s = getenv("CHORD_W4A16_STREAM_CHAIN")) o.stream_chain = atoi(s);
    if (const char* s = getenv("CHORD_LOG")) o.log = atoi(s) != 0;
    return o;
  }();
  return e;
}

// ---- planner and plan cache ------------------------------------------------
// Every byte of a key is a named field (the explicit `pad` keeps the int64
// aligned without compiler padding), so hashing and comparing the raw bytes
// is well defined; keys are only built by make_key, which zero-fills first.
struct PlanKey {
  int32_t mode, T, k, E_g, E_l, H, I, hint, cus;
  int32_t ov[8];  // schedule override fields (kernel, tokens, gu_nt, gu_wk, dn_nt, dn_wk,
                  // prefetch, tile_split)
  int32_t pad;
  int64_t rows;
  bool operator==(const PlanKey& o) const { return memcmp(this, &o, sizeof(*this)) == 0; }
};
static_assert(sizeof(PlanKey) == 18 * 4 + 8 && offsetof(PlanKey, rows) == 18 * 4,
              "PlanKey must have no padding bytes");
PlanKey make_key(int mode, int T, int k, int E_g, int E_l, int H, int I, int hint, int cus,
                 int64_t rows) {
  PlanKey key;
  memset(&key, 0, sizeof(key));
  key.mode = mode;
  key.T = T;
  key.k = k;
  key.E_g = E_g;
  key.E_l = E_l;
  key.H = H;
  key.I = I;
  key.hint = hint;
  key.cus = cus;
  key.rows = rows;
  return key;
}
void fill_override(PlanKey& key, const chord_schedule* s) {
  if (!s) return;
  key.ov[0] = s->kernel;
  key.ov[1] = s->tokens;
  key.ov[2] = s->gate_up_nt;
  key.ov[3] = s->gate_up_wk;
  key.ov[4] = s->down_nt;
  key.ov[5] = s->down_wk;
  key.ov[6] = s->prefetch;
  key.ov[7] = s->tile_split;
}
struct PlanKeyHash {
  size_t operator()(const PlanKey& k) const {
    const unsigned char* p = reinterpret_cast<const unsigned char*>(&k);
    size_t h = 1469598103934665603ull;
    for (size_t i = 0; i < sizeof(k); ++i) h = (h ^ p[i]) * 1099511628211ull;
    return h;
  }
};
struct GemmPlan {
  int slices;  // tiled kernel with K <= 256: 256-row slices per work item
  int nt;      // 16-row weight tiles per wave (streaming kernel)
  int wk;      // waves splitting K (streaming kernel)
  int pf;      // K chunks in flight per wave (streaming kernel)
  int grid;    // persistent workgroups
  int waves;   // tiled kernel with K > 256: waves per workgroup (4 or 8)
};
// kernel: 1 = weight-streaming GEMMs on small tiles, 2 = LDS-tiled GEMMs on
// big tiles, 3 = both, each expert going to one of them by its row count.
struct Plan {
  int kernel;
  int mt;            // streaming kernel: 16-row token groups per tile
  int tile_tokens;   // streaming kernel: rows per small tile
  bool block_tiles;  // indexed: small tiles are the alignment blocks (no tile builder)
  int max_tiles;     // small-tile list capacity
  int max_tiles_b;   // big-tile list capacity
  int split_rows;    // kernel 3: experts with >= split_rows rows take the tiled kernel
  bool tile_ksplit;  // tiled kernel: outsized tiles may be split along K
  bool tile_pc;      // tiled GEMMs with K > 256 in the producer/consumer form
  int big_tokens;    // rows per big tile
  bool routed;       // indexed: rows from topk_ids inside the gate_up launch (no alignment read)
  bool fused;        // routed: down GEMM and combine in one launch
  int cus;
  GemmPlan gu, dn;    // streaming GEMMs
  GemmPlan gut, dnt;  // tiled GEMMs
  char text[240];
};
std::mutex g_plan_mu;
std::unordered_map<PlanKey, Plan, PlanKeyHash> g_plans;

constexpr int kTileSlice = 256;    // output rows per workgroup of the tiled kernel
constexpr int kTileTokens = 192;   // token rows per big tile (tiled kernel)
constexpr int kTileTokensPc = 176; // ... in the producer/consumer form (11 token groups)
constexpr double kPcMinRows = 64.0;  // producer/consumer form from this many rows per expert
constexpr double kTileMinRows = 24.0;        // auto choice of the tiled family
constexpr double kTileMinRowsShortK = 8.0;   // same, when the down GEMM is short-K
constexpr double kSplitRows = 48.0;          // kernel 3: experts with this many rows go tiled

int max_tiles_for(int64_t rows, int E_l, int tile_tokens) {
  return (int)((rows + tile_tokens - 1) / tile_tokens) + E_l + 1;
}

// tok_e = expected rows per local expert; the schedule follows it, not the
// total token count.  Kernel family: the LDS-tiled kernel once an expert's
// rows amortise the in-register dequantisation over many MFMAs; the
// weight-streaming kernel below that.  Kernel 3 (both, each expert by its row
// count, the tiled part on a side stream) is available as an override.
Plan make_plan(const PlanKey& key) {
  Plan p{};
  double tok_e;
  if (key.mode == kIndexed) {
    const int eg = key.E_g > 0 ? key.E_g : key.E_l;
    tok_e = (double)key.T * key.k / eg;
  } else if (key.mode == kMasked) {
    tok_e = key.hint;
  } else {
    tok_e = 128.0;
  }
  p.cus = key.cus;
  const bool tile_ok = (2 * key.I) % 64 == 0 && key.H % 64 == 0;  // 4 tiles per wave
  int kernel = key.ov[0] ? key.ov[0] : env().kernel;
  // Kernel 4 / 5: the LDS-tiled family in its single-role / producer-
  // consumer form (kernel 2 lets the planner choose the form).
  int tile_form = 0;  // 0 planner, 1 single-role, 2 producer/consumer
  if (kernel == 4 || kernel == 5) {
    tile_form = kernel - 3;
    kernel = 2;
  }
  if (kernel < 1 || kernel > 3) {
    // Expected rows per expert decide the family (measured crossovers on
    // MI355X at steady clocks): the tiled kernel from 24 rows, or from 8 when
    // the down GEMM is short-K (I <= 256: token tile resident in LDS, several
    // slices per item; TP slice T = 512: 328 -> 294 us; masked Zipf with
    // the K split: E = 24 246 -> ~227, E = 48 389 -> ~331, E = 96 547 -> ~509).
    // Masked calls split outsized tiles along K (below), which removes the
    // hot-expert tail that made the tiled family lose on skewed counts.
    const double cross =
        (key.I <= 256 || key.mode == kMasked) ? kTileMinRowsShortK : kTileMinRows;
    kernel = tok_e >= cross ? 2 : 1;
  }
  if (!tile_ok) kernel = 1;
  p.kernel = kernel;
  p.split_rows = kernel == 3 ? (int)kSplitRows : (kernel == 2 ? 0 : INT32_MAX);
  p.max_tiles_b = kernel & 2 ? max_tiles_for(key.rows, key.E_l, kTileTokensPc) : 0;
  // K split of outsized big tiles (masked layout: budgets per expert with
  // skewed counts): both tiled GEMMs must run the general tiled kernel
  // (K > 256; the short-K kernel has no split), and no override or
  // environment switch may have turned it off.  It costs a fixup launch
  // after each tiled GEMM, so near-uniform layouts do without.
  // (The workspace holds partial slots for masked calls only.)
  p.tile_ksplit = (kernel & 2) && key.mode == kMasked && key.H / kChunkK > 2 &&
                  key.I / kChunkK > 2 && key.ov[7] != 1 && env().tile_split != 1;
  // Producer/consumer form of the tiled GEMMs with K > 256: waves that only
  // issue MFMAs and waves that only load and dequantise (no K split; tiles of
  // at most 176 rows).  It pays once tiles hold many token groups.
  if (tile_form == 0)
    tile_form = (env().tile_pc == 1 && tok_e >= kPcMinRows) ? 2 : 1;
  p.tile_pc = kernel == 2 && tile_form == 2 && !p.tile_ksplit;
  p.big_tokens = p.tile_pc ? kTileTokensPc : kTileTokens;

  // Tiled GEMMs: one workgroup per CU (registers, ~150 KB of LDS); the
  // launcher clamps to the occupancy it measures.
  // With K <= 256 the token tile stays in LDS and a work item covers several
  // 256-row slices: as many as keep about three items per CU of expected
  // tiles (experts x 192-row tiles each).
  const double tiles_est = std::max(1.0, (double)key.E_l * std::ceil(std::max(tok_e, 1.0) / kTileTokens));
  auto tgemm = [&](int N, int K) {
    GemmPlan g{};
    const int nslices = (N + kTileSlice - 1) / kTileSlice;
    int S = 1;
    if (K / kChunkK <= 2) {
      S = nslices;
      while (S > 1 && tiles_est * ((nslices + S - 1) / S) < 3.0 * key.cus) S = (S + 1) / 2;
    }
    g.slices = S;
    // Two waves per SIMD (8 per workgroup, 2 weight tiles each): one wave
    // cannot keep the MFMA pipe busy (prefill gate_up 486 -> 434 us).  Or
    // the producer/consumer form (marked waves = 2).
    g.waves = env().tile_waves == 4 ? 4 : 8;
    if (p.tile_pc && K / kChunkK > 2) g.waves = 2;
    const int64_t items = (int64_t)p.max_tiles_b * ((nslices + S - 1) / S);
    const int per_cu = env().tile_wgs > 0 ? env().tile_wgs : 1;
    g.grid = (int)std::max<int64_t>(1, std::min<int64_t>(items, (int64_t)per_cu * key.cus));
    return g;
  };
  if (kernel & 2) {
    p.gut = tgemm(2 * key.I, key.H);
    p.dnt = tgemm(key.H, key.I);
  }

  // Routed indexed calls (weight-streaming family chosen by the planner, a
  // few thousand slots at most): every gate_up workgroup builds the
  // per-expert row lists from topk_ids in LDS, so no alignment launch and no
  // dependent chain of index loads precede the weight stream; h and y are
  // stored per flat slot.  With at most 16 tokens and 64 slots the down GEMM
  // and the combine run as one launch.
  const int64_t slots = (int64_t)key.T * key.k;
  // The gate_up K must span more than 2 chunks: with K <= 256 the streaming
  // GEMM runs its short-K variant, which takes its tiles from the alignment.
  // The routing tables share the launch's 64 KB of dynamic LDS with the K
  // reduction area (at most 32 KB), so they get the other 32 KB: up to about
  // a thousand local experts at the 2,048-slot maximum.
  p.routed = kernel == 1 && key.mode == kIndexed && key.ov[0] == 0 && env().kernel == 0 &&
             env().routed != 0 && slots >= 1 && slots <= kRoutedMaxSlots &&
             key.H / kChunkK > 2 && route_lds_bytes(key.E_l, (int)slots) <= kRouteLdsMax;

  // Streaming GEMMs.
  const double tok_small = kernel == 3 ? std::min(tok_e, kSplitRows - 1) : tok_e;
  int mt = (int)((tok_small + 15.0) / 16.0);
  mt = std::max(1, std::min(2, mt));
  const int tokens = key.ov[1] ? key.ov[1] : env().tokens;
  if (tokens == 16 || tokens == 32) mt = tokens / 16;
  p.mt = mt;
  p.tile_tokens = mt * 16;
  // Fused down + combine for a handful of tokens (one launch, y never leaves
  // the workgroup).  A down GEMM override asks for the separate down launch.
  p.fused = p.routed && env().fused != 0 && key.ov[4] == 0 && key.ov[5] == 0 &&
            slots <= kFusedMaxSlots && key.T <= kFusedMaxTokens;
  // key.hint carries block_m for indexed calls.
  p.block_tiles = !p.routed && kernel == 1 && key.mode == kIndexed && key.hint == p.tile_tokens;
  p.max_tiles = kernel == 2 ? 0
                : p.routed ? (int)std::min<int64_t>(slots, slots / p.tile_tokens + key.E_l)
                : p.block_tiles ? (int)((key.rows + key.hint - 1) / key.hint)
                                : max_tiles_for(key.rows, key.E_l, p.tile_tokens);
  const int ov_pf = key.ov[6] ? key.ov[6] : env().prefetch;
  auto gemm = [&](int N, int K, int ov_nt, int ov_wk, int env_nt, int env_wk) {
    GemmPlan g{};
    // Defaults measured on MI355X at the decode / TP-slice shapes: deep-K
    // gate_up splits K over two waves; the short-K down GEMM runs one wave per
    // item with 4 weight tiles; very short K (<= 512) keeps 4 chunks in flight.
    const int chunks = K / kChunkK;
    g.nt = 4;
    g.wk = chunks >= 24 ? 2 : 1;
    g.pf = chunks <= 4 ? 4 : 2;
    // Too few work items to cover the CUs (a handful of routed rows): narrower
    // items (2 weight tiles) and, for deep K, a 4-way K split.
    const double tiles_guess = std::max(1.0, std::min((double)key.E_l, key.mode == kIndexed
                                                                          ? (double)key.T * key.k
                                                                          : (double)key.rows));
    if (tiles_guess * (N / 16 / 4) < key.cus) {
      g.nt = 2;
      if (chunks >= 16) g.wk = 4;
    }
    // Nearly empty token tiles (a few rows per expert) on a wide, deep-K GEMM:
    // the token loads of an item are mostly out-of-range zeros, so 2 weight
    // tiles per item cost little extra and the smaller register set fits a
    // fourth wave per SIMD (decode gate_up, N = 4096: 128 -> 121 us at steady
    // clocks).  With denser tiles the doubled token loads per weight byte make
    // it slower, and on the narrow TP-slice gate_up (N = 512) the doubled
    // item count does (T = 32: 123 -> 128 us).
    if (tok_e <= 4.0 && chunks >= 24 && N >= 2048) g.nt = 2;
    const int nt = ov_nt ? ov_nt : env_nt;
    const int wk = ov_wk ? ov_wk : env_wk;
    if (nt == 1 || nt == 2 || nt == 4) g.nt = nt;
    if (wk == 1 || wk == 2 || wk == 4) g.wk = wk;
    if (ov_pf == 2 || ov_pf == 4) g.pf = ov_pf;
    if ((N / 16) % g.nt != 0) g.nt = 2;
    // A handful of routed rows on a deep-K GEMM (the TP slice at T = 1): the
    // 4-way split leaves half the CUs idle and each wave a serial chain of 14
    // chunk loads, so K splits over 8 waves (2 weight tiles, one token tile;
    // not selectable by overrides).
    if (nt == 0 && wk == 0 && g.nt == 2 && mt == 1 && chunks >= 32 &&
        tiles_guess * (N / 16 / 2) <= key.cus / 2)
      g.wk = 8;
    // Still no more single-tile items than CUs: one weight tile per item, so
    // every CU holds a workgroup, and 4 chunks in flight per wave (T = 1
    // gate_up: 11.9 -> 10.3 us).
    if (g.wk == 8 && tiles_guess * (N / 16) <= key.cus) {
      g.nt = 1;
      g.pf = env().prefetch == 8 ? 8 : 4;
    }
    // Short K (<= 2 chunks): an item covers several groups of weight tiles of
    // one token tile (token fragments loaded once, weight loads pipelined
    // across the groups), about 8 items per CU of expected tiles.
    g.slices = 0;
    const int n_groups = (N / 16) / g.nt;
    if (chunks <= 2 && g.wk == 1) {
      const double per = tiles_guess * n_groups / (8.0 * key.cus);
      g.slices = (int)std::max(1.0, std::min((double)n_groups, std::ceil(per)));
    }
    const int64_t items = (int64_t)p.max_tiles *
                          (g.slices > 0 ? (n_groups + g.slices - 1) / g.slices : n_groups);
    g.grid = (int)std::max<int64_t>(1, std::min<int64_t>(items, (int64_t)key.cus * 64));
    if (env().stream_wgs > 0)
      g.grid = (int)std::max<int64_t>(1, std::min<int64_t>(items, (int64_t)key.cus * env().stream_wgs));
    return g;
  };
  if (kernel & 1) {
    p.gu = gemm(2 * key.I, key.H, key.ov[2], key.ov[3], env().gu_nt, env().gu_wk);
    p.dn = gemm(key.H, key.I, key.ov[4], key.ov[5], env().dn_nt, env().dn_wk);
  }

  const int cap = (int)sizeof(p.text);
  int n = std::min(cap, snprintf(p.text, sizeof(p.text), "tok_e=%.1f", tok_e));
  if (kernel & 1)
    n += snprintf(p.text + n, sizeof(p.text) - n,
                  " | stream tiles=%s of %d rows: gate_up nt=%d wk=%d pf=%d, %s nt=%d wk=%d pf=%d"
                  " groups/item %d",
                  p.routed ? "routed" : p.block_tiles ? "blocks" : "list", p.tile_tokens, p.gu.nt,
                  p.gu.wk, p.gu.pf, p.fused ? "down+combine" : "down", p.dn.nt, p.dn.wk, p.dn.pf,
                  p.dn.slices);
  n = std::min(cap, n);
  if (kernel & 2)
    snprintf(p.text + n, sizeof(p.text) - n, " | tile 256x%d, %s (slices/item %d, %d)%s",
             p.big_tokens,
             p.tile_pc ? (p.dnt.waves == 2 ? "producer/consumer" : "producer/consumer gate_up")
                       : (p.gut.waves == 4 ? "4 waves" : "8 waves"),
             p.gut.slices, p.dnt.slices, kernel == 3 ? " for experts with >= 48 rows" : "");
  return p;
}

Plan get_plan(const PlanKey& key) {
  std::lock_guard<std::mutex> lk(g_plan_mu);
  auto it = g_plans.find(key);
  if (it != g_plans.end()) return it->second;
  Plan p = make_plan(key);
  g_plans.emplace(key, p);
  if (env().log) fprintf(stderr, "[chord] plan mode=%d T=%d E_l=%d: %s\n", key.mode, key.T, key.E_l,
                         p.text);
  return p;
}

// Whether an indexed call with these shapes (and override) is routed: the
// planner's choice of the weight-streaming family at <= kRoutedMaxSlots
// slots, which depends on neither block_m, the buffer sizes nor the CU count.
bool routed_call(int T, int k, int E_g, int E_l, int H, int I, const chord_schedule* ov) {
  if (T < 1 || k < 1 || E_l < 1 || E_l > kMaxExperts || H <= 0 || I <= 0) return false;
  PlanKey key = make_key(kIndexed, T, k, E_g, E_l, H, I, 0, 256, 0);
  fill_override(key, ov);
  return get_plan(key).routed;
}

// ---- kernel-stage profiling (HIP events on the caller's stream) -----------
struct ProfRecord {
  hipEvent_t ev[5];
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof_pending;
std::vector<hipEvent_t> g_ev_pool;
double g_prof_ms[4] = {0, 0, 0, 0};
int64_t g_prof_calls = 0;

// Records the event for stage boundary `i` (0..4) of the current call.
struct StageTimer {
  bool on = false;
  ProfRecord rec{};
  hipStream_t stream = nullptr;
  explicit StageTimer(hipStream_t s, bool allowed = true) : stream(s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    on = g_prof_on && allowed;
    if (!on) return;
    for (int i = 0; i < 5; ++i) {
      if (!g_ev_pool.empty()) {
        rec.ev[i] = g_ev_pool.back();
        g_ev_pool.pop_back();
      } else if (hipEventCreate(&rec.ev[i]) != hipSuccess) {
        on = false;
        return;
      }
    }
  }
  void mark(int i) {
    if (on) (void)hipEventRecord(rec.ev[i], stream);
  }
  void finish() {
    if (!on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pending.push_back(rec);
    on = false;
  }
};

// ---- workspace layout -----------------------------------------------------
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t status, tiles, tiles_b, split_tiles, partials, route_list, h, y, total;
  int max_tiles, max_tiles_b, max_slices;
};

// rows: the alignment's max_padded (indexed; 0 when the call is routed and
// passes no alignment), M (contiguous) or E*max_m (masked).  Indexed layouts
// also fit a routed call: h and the tile list hold at least T*k rows, and the
// routed slot list takes T*k ints.
WsLayout layer_ws(int mode, int T, int k, int E_l, int H, int I, int64_t rows) {
  WsLayout w{};
  const int64_t slots = mode == kIndexed ? (int64_t)T * k : 0;
  rows = std::max(rows, slots);
  w.max_tiles = max_tiles_for(rows, E_l, 16);
  // Big tiles, plus up to 3 extra entries per K-split tile.
  w.max_tiles_b = max_tiles_for(rows, E_l, kTileTokensPc) + 3 * kMaxSplitTiles;
  w.max_slices = (std::max(2 * I, H) + kTileSlice - 1) / kTileSlice;
  size_t off = 0;
  w.status = off;
  off = align_up(off + sizeof(DevStatus), 256);
  w.tiles = off;
  off = align_up(off + (size_t)w.max_tiles * sizeof(TileDesc), 256);
  w.tiles_b = off;
  off = align_up(off + (size_t)w.max_tiles_b * sizeof(TileDesc), 256);
  w.split_tiles = off;
  off = align_up(off + (size_t)kMaxSplitTiles * sizeof(TileDesc), 256);
  // K-split partial slots: only masked calls split outsized tiles along K.
  w.partials = off;
  if (mode == kMasked)
    off = align_up(off + (size_t)kSplitCapSlots * kPartialSlotFloats * sizeof(float), 256);
  w.route_list = off;
  off = align_up(off + (size_t)slots * sizeof(int32_t), 256);
  w.h = off;
  off = align_up(off + (size_t)rows * I * 2, 256);
  w.y = off;
  if (mode == kIndexed) off = align_up(off + (size_t)T * k * H * 2, 256);
  w.total = off;
  return w;
}

// ---- weight handle checks -------------------------------------------------
chord_status check_weight(const chord_w4a16_weight* w, const char* name, int mode, int role) {
  if (!w) return fail(CHORD_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (w->magic != CHORD_WEIGHT_MAGIC || w->version != CHORD_WEIGHT_VERSION)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "%s is not a packed chord weight handle", name);
  if (!w->data) return fail(CHORD_ERR_INVALID_ARGUMENT, "%s has no data", name);
  if (w->mode != mode)
    return fail(CHORD_ERR_LAYOUT_MISMATCH, "%s was packed for mode %d, this entry point is mode %d",
                name, w->mode, mode);
  if (w->role != role)
    return fail(CHORD_ERR_LAYOUT_MISMATCH, "%s has role %d, expected %d", name, w->role, role);
  if (w->group_size != kGroup) return fail(CHORD_ERR_UNSUPPORTED, "%s group size", name);
  if (w->bytes < packed_bytes(w->num_experts, w->n, w->k))
    return fail(CHORD_ERR_INVALID_ARGUMENT, "%s byte count too small", name);
  return CHORD_OK;
}

chord_status check_pair(const chord_w4a16_weight* w13, const chord_w4a16_weight* w2, int mode,
                        int H, int I) {
  CHORD_CHECK(check_weight(w13, "w13", mode, CHORD_ROLE_GATE_UP));
  CHORD_CHECK(check_weight(w2, "w2", mode, CHORD_ROLE_DOWN));
  if (H <= 0 || I <= 0) return fail(CHORD_ERR_INVALID_ARGUMENT, "H=%d I=%d", H, I);
  if (w13->n != 2 * I || w13->k != H)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "w13 is [%d,%d], expected [2I=%d, H=%d]", w13->n,
                w13->k, 2 * I, H);
  if (w2->n != H || w2->k != I)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "w2 is [%d,%d], expected [H=%d, I=%d]", w2->n, w2->k,
                H, I);
  if (w13->num_experts != w2->num_experts)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "w13 has %d experts, w2 %d", w13->num_experts,
                w2->num_experts);
  if (w13->num_experts > kMaxExperts)
    return fail(CHORD_ERR_UNSUPPORTED, "more than %d local experts", kMaxExperts);
  if ((2 * I / 16) % 2 != 0 || (H / 16) % 2 != 0)
    return fail(CHORD_ERR_UNSUPPORTED, "H and 2I must be multiples of 32");
  return CHORD_OK;
}

bool valid_bm(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }

void set_plan_text(const char* mode, const Plan& p) {
  char b[256];
  snprintf(b, sizeof(b), "%s: %s", mode, p.text);
  g_last_plan = b;
}

// Side stream (one per device, default priority) on which the tiled kernel
// runs next to the streaming kernel when both are planned (kernel 3): the
// caller's stream forks to it and joins back through two events, so the two
// kernels share the GPU instead of running one after the other.  Calls on one
// device serialise on the side stream (the fork-launch-join sequence holds a
// lock), which keeps the event reuse safe.
struct SideStream {
  bool ready = false;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];

hipError_t get_side(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (!ss.ready) {
    if ((e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
    ss.ready = true;
  }
  *out = &ss;
  return hipSuccess;
}

// Launches one expert GEMM with the planned kernel(s): the streaming kernel
// over the small-tile list, the tiled kernel over the big-tile list.
hipError_t launch_planned(const Plan& plan, bool gate_up, GemmArgs g, TileDesc* tiles_b,
                          hipStream_t stream) {
  GemmArgs gs = g, gt = g;
  const GemmPlan& sp = gate_up ? plan.gu : plan.dn;
  const GemmPlan& tp = gate_up ? plan.gut : plan.dnt;
  gs.tiles_per_item = sp.nt;
  gs.items_per_tile = sp.nt > 0 ? g.n_tiles / sp.nt : 0;
  gs.slices_per_item = sp.slices;
  gs.no_chain = env().stream_chain == 0;
  if (sp.slices > 0) gs.items_per_tile = (gs.items_per_tile + sp.slices - 1) / sp.slices;
  gt.tiles = tiles_b;
  gt.tiles_per_item = kTileSlice / kTileRows;
  gt.items_per_tile = (g.n_tiles + gt.tiles_per_item - 1) / gt.tiles_per_item;
  gt.tile_tokens = plan.big_tokens;
  gt.slices_per_item = std::max(1, std::min(tp.slices, gt.items_per_tile));
  gt.tile_waves = tp.waves;
  if (plan.kernel == 1) return launch_gemm(1, sp.nt, plan.mt, sp.wk, sp.pf, gs, sp.grid, stream);
  // The tiled GEMM, then (K split on) the pass that completes split tiles.
  auto tiled = [&](hipStream_t st) {
    hipError_t e = launch_gemm_tile(gt, tp.grid, st);
    if (e == hipSuccess && plan.tile_ksplit && gt.n_chunks > 2) e = launch_tile_split_fixup(gt, st);
    return e;
  };
  if (plan.kernel == 2) return tiled(stream);
  std::lock_guard<std::mutex> lk(g_side_mu);
  SideStream* ss = nullptr;
  hipError_t e;
  if ((e = get_side(&ss)) != hipSuccess) return e;
  if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess) return e;
  if ((e = tiled(ss->s)) != hipSuccess) return e;
  if ((e = launch_gemm(1, sp.nt, plan.mt, sp.wk, sp.pf, gs, sp.grid, stream)) != hipSuccess)
    return e;
  if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess) return e;
  return hipStreamWaitEvent(stream, ss->join, 0);
}

// The routing of a routed indexed call (plan.routed): what the gate_up launch
// derives its rows from, and for the fused down + combine its output.
struct RouteCall {
  const int32_t* topk_ids = nullptr;
  const float* topk_weights = nullptr;
  int expert_begin = 0;
  int T = 0;
  uint16_t* out = nullptr;  // [T, H] (fused only)
};

// Shared GEMM sequence: tiles -> gate_up -> down.
chord_status run_expert_gemms(int layout, const Plan& plan, const WsLayout& ws, uint8_t* wsp,
                              const chord_w4a16_weight* w13, const chord_w4a16_weight* w2, int H,
                              int I, const uint16_t* bsrc, int64_t bsrc_rows,
                              int64_t rows_internal, const int32_t* sorted_ids, int topk,
                              int64_t n_flat, const int32_t* m_indices, uint16_t* down_out,
                              int64_t down_rows, const float* row_weights, TileBuildArgs tb,
                              hipStream_t stream, StageTimer& timer,
                              const RouteCall* route = nullptr) {
  // Buffer resources address their source with 32-bit offsets.
  const int64_t kMaxBuf = ((int64_t)1 << 31) - 1;
  if (bsrc_rows * H * 2 > kMaxBuf || rows_internal * I * 2 > kMaxBuf ||
      (int64_t)(2 * I / kTileRows) * (H / kChunkK) * kBlockBytes > kMaxBuf ||
      (int64_t)(H / kTileRows) * (I / kChunkK) * kBlockBytes > kMaxBuf)
    return fail(CHORD_ERR_UNSUPPORTED, "a layer operand exceeds 2 GiB");
  DevStatus* status = reinterpret_cast<DevStatus*>(wsp + ws.status);
  TileDesc* tiles = reinterpret_cast<TileDesc*>(wsp + ws.tiles);
  TileDesc* tiles_b = reinterpret_cast<TileDesc*>(wsp + ws.tiles_b);
  uint16_t* h = reinterpret_cast<uint16_t*>(wsp + ws.h);
  tb.layout = layout;
  tb.tile_tokens = plan.tile_tokens;
  tb.max_tiles = std::min(plan.max_tiles, ws.max_tiles);
  tb.big_tokens = plan.big_tokens;
  tb.max_tiles_b = plan.tile_ksplit ? ws.max_tiles_b : std::min(plan.max_tiles_b, ws.max_tiles_b);
  tb.split_cap = plan.tile_ksplit ? kSplitCapSlots : 0;
  // Parts of at least 8 K chunks in the shorter GEMM (shorter parts spend
  // more on their prologue than they gain), 2..4; the environment (2..4)
  // overrides for experiments.
  tb.max_ksplit = env().tile_split >= 2 && env().tile_split <= 4
                      ? env().tile_split
                      : std::max(2, std::min(4, std::min(H, I) / kChunkK / 8));
  tb.max_slices = ws.max_slices;
  tb.split_tiles = reinterpret_cast<TileDesc*>(wsp + ws.split_tiles);
  tb.split_rows = plan.split_rows;
  tb.tiles = tiles;
  tb.tiles_b = tiles_b;
  tb.status = status;
  timer.mark(0);
  if (plan.routed) {
    // no tile builder: the gate_up launch routes itself
  } else if (plan.block_tiles) {
    HIP_TRY(launch_check_blocks(tb, stream), "block check launch");
  } else {
    HIP_TRY(launch_build_tiles(tb, stream), "tile builder launch");
  }
  timer.mark(1);

  GemmArgs g{};
  g.layout = layout;
  g.sorted_ids = sorted_ids;
  g.topk = topk;
  g.n_flat = n_flat;
  g.m_indices = m_indices;
  g.tiles = plan.block_tiles ? nullptr : tiles;
  g.status = status;
  g.expert_ids = tb.expert_ids;
  g.ntpp = tb.ntpp;
  g.block_m = tb.block_m;
  g.max_padded = tb.max_padded;
  g.num_experts = tb.num_experts;
  g.num_cus = plan.cus;
  g.partials = reinterpret_cast<float*>(wsp + ws.partials);
  g.split_tiles = tb.split_tiles;
  g.max_slices = ws.max_slices;
  g.tile_tokens = plan.tile_tokens;
  g.n_rows_internal = rows_internal;

  // gate_up: B = activations rows, out = h [rows_internal, I]
  g.wpack = static_cast<const uint8_t*>(w13->data);
  g.n_tiles = 2 * I / kTileRows;
  g.n_chunks = H / kChunkK;
  g.K = H;
  g.bsrc = bsrc;
  g.bsrc_bytes = bsrc_rows * H * 2;
  g.gate_up = 1;
  g.out = h;
  g.out_ld = I;
  g.out_rows = rows_internal;
  g.row_weights = nullptr;
  if (plan.routed) {
    // Rows from topk_ids; h per flat slot.  Workgroup 0 leaves the slot
    // list and the tiles in the workspace for the down launch.
    g.tiles = nullptr;
    g.route_ids = route->topk_ids;
    g.route_eb = route->expert_begin;
    g.route_n = (int)n_flat;
    g.route_list = reinterpret_cast<int32_t*>(wsp + ws.route_list);
    g.route_tiles = tiles;
  }
  HIP_TRY(launch_planned(plan, true, g, tiles_b, stream), "gate_up launch");
  timer.mark(2);

  // down: B = h, out = y / out rows
  g.wpack = static_cast<const uint8_t*>(w2->data);
  g.n_tiles = H / kTileRows;
  g.n_chunks = I / kChunkK;
  g.K = I;
  g.bsrc = h;
  g.bsrc_bytes = rows_internal * I * 2;
  g.gate_up = 0;
  g.out = down_out;
  g.out_ld = H;
  g.out_rows = down_rows;
  g.row_weights = row_weights;
  if (plan.routed) {
    g.route_ids = nullptr;
    g.tiles = tiles;                       // written by the gate_up launch
    g.sorted_ids = g.route_list;
    g.h_by_slot = 1;
    if (plan.fused) {
      g.route_ids = route->topk_ids;
      g.topk_weights = route->topk_weights;
      g.T = route->T;
      g.out = route->out;
      HIP_TRY(launch_down_combine_small(g, stream), "down+combine launch");
      timer.mark(3);
      return CHORD_OK;
    }
  }
  HIP_TRY(launch_planned(plan, false, g, tiles_b, stream), "down launch");
  timer.mark(3);
  return CHORD_OK;
}

chord_status finish_validate(uint32_t flags, const WsLayout& ws, uint8_t* wsp, hipStream_t stream) {
  if (!(flags & CHORD_FLAG_VALIDATE)) return CHORD_OK;
  int32_t err = 0;
  HIP_TRY(hipMemcpyAsync(&err, wsp + ws.status, sizeof(err), hipMemcpyDeviceToHost, stream),
          "status readback");
  HIP_TRY(hipStreamSynchronize(stream), "stream sync");
  if (err != 0) return fail(CHORD_ERR_ROUTING, "routing validation failed (flags 0x%x)", err);
  return CHORD_OK;
}

// ---- scratch of the allocation-free indexed entry point --------------------
// A file-scope device array: each GPU the library runs on holds its own copy
// from the first allocation-free call until the process ends.  In host code
// the array's name is a host-side stand-in, not a device address, so it is
// never passed to a kernel or a copy: the device address is looked up once
// per device (with that device current) and kept in g_scratch.  Every
// allocation-free call on a GPU shares that GPU's array; calls that overlap
// on one GPU (other streams, other threads) race on it.
constexpr size_t kNoAllocScratchBytes = CHORD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch[64];

chord_status noalloc_scratch(void** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(CHORD_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(CHORD_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CHORD_OK;
}

}  // namespace

// Dispatch into the grouped layouts: shared checks, workspace layout and the
// alignment step both layouts start from.
namespace {

constexpr int kContigBlock = 128;  // contiguous segments pad to the M-tile
constexpr int kMaskedBlock = 16;   // masked dispatch: smallest alignment block

struct DispatchWs {
  size_t align_off, sorted_off, experts_off, ntpp_off, total;
  int64_t max_padded;
};

DispatchWs dispatch_ws(int T, int k, int E_l, int block_m) {
  DispatchWs w{};
  w.max_padded = chord_moe_align_max_padded(T, k, E_l, block_m);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  w.align_off = take(chord_moe_align_workspace_bytes(T, k, E_l, block_m));
  w.sorted_off = take((size_t)w.max_padded * sizeof(int32_t));
  w.experts_off = take((size_t)((w.max_padded + block_m - 1) / block_m) * sizeof(int32_t));
  w.ntpp_off = take(sizeof(int32_t));
  w.total = off;
  return w;
}

// Shared argument checks and the alignment step of both dispatch layouts.
chord_status dispatch_prepare(const chord_bf16* x, int T, int H, const int32_t* topk_ids, int k,
                              int expert_begin, int E_l, int block_m, int32_t* flat_to_row,
                              void* workspace, size_t ws_bytes, hipStream_t st, DispatchArgs* d) {
  if (T < 0 || k < 1 || H <= 0) return fail(CHORD_ERR_INVALID_ARGUMENT, "T=%d k=%d H=%d", T, k, H);
  if (H % 8 != 0) return fail(CHORD_ERR_UNSUPPORTED, "H=%d must be a multiple of 8", H);
  if (E_l < 1 || E_l > kMaxExperts)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "num_local_experts=%d (1..%d)", E_l, kMaxExperts);
  if ((int64_t)T * k >= ((int64_t)1 << 30)) return fail(CHORD_ERR_UNSUPPORTED, "T*k too large");
  if (T > 0 && (!x || !topk_ids || !flat_to_row))
    return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "x must be 16-byte aligned");
  const DispatchWs w = dispatch_ws(T, k, E_l, block_m);
  if (!workspace || ws_bytes < w.total)
    return fail(CHORD_ERR_WORKSPACE, "dispatch workspace %zu bytes, %zu needed", ws_bytes,
                w.total);
  // Host checks are done; chord_moe_align checks the device before launching.
  uint8_t* wsp = static_cast<uint8_t*>(workspace);
  int32_t* sorted = reinterpret_cast<int32_t*>(wsp + w.sorted_off);
  int32_t* experts = reinterpret_cast<int32_t*>(wsp + w.experts_off);
  int32_t* ntpp = reinterpret_cast<int32_t*>(wsp + w.ntpp_off);
  const chord_status s =
      chord_moe_align(topk_ids, T, k, expert_begin, E_l, block_m, sorted, experts, ntpp,
                      w.max_padded, wsp + w.align_off,
                      chord_moe_align_workspace_bytes(T, k, E_l, block_m), 0, st);
  if (s != CHORD_OK) return s;
  *d = DispatchArgs{};
  d->x = reinterpret_cast<const uint16_t*>(x);
  d->topk_ids = topk_ids;
  d->T = T;
  d->k = k;
  d->H = H;
  d->expert_begin = expert_begin;
  d->num_experts = E_l;
  d->sorted_ids = sorted;
  d->expert_ids = experts;
  d->ntpp = ntpp;
  d->block_m = block_m;
  d->max_padded = w.max_padded;
  d->flat_to_row = flat_to_row;
  return CHORD_OK;
}

// Every field of a schedule override within the values the kernels are
// instantiated for (0 = automatic).
bool override_in_range(const chord_schedule* o) {
  auto in = [](int v, std::initializer_list<int> ok) {
    for (int x : ok)
      if (v == x) return true;
    return false;
  };
  return in(o->kernel, {0, 1, 2, 3, 4, 5}) && in(o->tokens, {0, 16, 32}) &&
         in(o->gate_up_nt, {0, 2, 4}) && in(o->down_nt, {0, 2, 4}) &&
         in(o->gate_up_wk, {0, 1, 2, 4}) && in(o->down_wk, {0, 1, 2, 4}) &&
         in(o->prefetch, {0, 2, 4}) && in(o->tile_split, {0, 1});
}

}  // namespace

// ===========================================================================
// Public C ABI
// ===========================================================================
extern "C" {

const char* chord_status_string(chord_status s) {
  switch (s) {
    case CHORD_OK: return "CHORD_OK";
    case CHORD_ERR_INVALID_ARGUMENT: return "CHORD_ERR_INVALID_ARGUMENT";
    case CHORD_ERR_UNSUPPORTED: return "CHORD_ERR_UNSUPPORTED";
    case CHORD_ERR_LAYOUT_MISMATCH: return "CHORD_ERR_LAYOUT_MISMATCH";
    case CHORD_ERR_WORKSPACE: return "CHORD_ERR_WORKSPACE";
    case CHORD_ERR_ROUTING: return "CHORD_ERR_ROUTING";
    case CHORD_ERR_HIP: return "CHORD_ERR_HIP";
  }
  return "CHORD_ERR_UNKNOWN";
}

const char* chord_last_error(void) { return g_last_error.c_str(); }

chord_status chord_last_plan(char* buf, size_t n) {
  if (!buf || n == 0) return CHORD_ERR_INVALID_ARGUMENT;
  snprintf(buf, n, "%s", g_last_plan.c_str());
  return CHORD_OK;
}

chord_status chord_w4a16_moe_plan(int mode, int T, int k, int num_global_experts, int E_l, int H,
                                  int I, int hint, int64_t rows, int num_cus,
                                  const chord_schedule* override, char* buf, size_t n) {
  if (!buf || n == 0) return fail(CHORD_ERR_INVALID_ARGUMENT, "null or empty output buffer");
  if (mode != kIndexed && mode != kContiguous && mode != kMasked)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "mode %d", mode);
  if (E_l < 1 || E_l > kMaxExperts || H <= 0 || I <= 0 || H % kChunkK != 0 || I % kChunkK != 0 ||
      rows < 0 || num_cus < 0 || hint < 0 || T < 0 || k < 0 || num_global_experts < 0)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "bad call descriptor");
  if (mode == kIndexed && (T < 1 || k < 1 || (hint != 0 && !valid_bm(hint))))
    return fail(CHORD_ERR_INVALID_ARGUMENT,
                "indexed plans need T, k and a block_m of 16..128 (0: no alignment)");
  if (mode != kIndexed && override)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "grouped calls take no schedule override");
  if (override && !override_in_range(override))
    return fail(CHORD_ERR_INVALID_ARGUMENT, "schedule override out of range");
  PlanKey key = make_key(mode, mode == kMasked ? 0 : T, mode == kMasked ? 0 : k,
                         mode == kIndexed ? num_global_experts : 0, E_l, H, I, hint,
                         num_cus > 0 ? num_cus : 256, rows);
  fill_override(key, override);
  const Plan plan = get_plan(key);
  snprintf(buf, n, "%s: %s", mode == kIndexed ? "indexed" : mode == kContiguous ? "contiguous" : "masked",
           plan.text);
  return CHORD_OK;
}

const char* chord_version(void) { return "chord-mi355x 0.1 (gfx950)"; }

chord_status chord_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return CHORD_OK;
}

chord_status chord_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_pending)
    for (auto e : r.ev) g_ev_pool.push_back(e);
  g_prof_pending.clear();
  for (double& m : g_prof_ms) m = 0;
  g_prof_calls = 0;
  return CHORD_OK;
}

chord_status chord_profile_read(double* stage_ms, int64_t* calls) {
  g_last_error.clear();
  if (!stage_ms || !calls) return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_pending) {
    HIP_TRY(hipEventSynchronize(r.ev[4]), "hipEventSynchronize");
    for (int i = 0; i < 4; ++i) {
      float ms = 0.f;
      HIP_TRY(hipEventElapsedTime(&ms, r.ev[i], r.ev[i + 1]), "hipEventElapsedTime");
      g_prof_ms[i] += ms;
    }
    ++g_prof_calls;
    for (auto e : r.ev) g_ev_pool.push_back(e);
  }
  g_prof_pending.clear();
  for (int i = 0; i < 4; ++i) stage_ms[i] = g_prof_ms[i];
  *calls = g_prof_calls;
  return CHORD_OK;
}

size_t chord_w4a16_packed_bytes(int mode, int role, int E, int N, int K) {
  if (mode < 0 || mode > 2 || role < 0 || role > 1) return 0;
  if (E < 1 || N <= 0 || K <= 0 || K % kChunkK != 0 || N % kTileRows != 0) return 0;
  if (role == CHORD_ROLE_GATE_UP && ((N / 2) % 8 != 0 || N % 2 != 0)) return 0;
  return packed_bytes(E, N, K);
}

chord_status chord_w4a16_pack(int mode, int role, const int32_t* qweight, const chord_bf16* scales,
                              int E, int N, int K, int group_size, void* dst, size_t dst_bytes,
                              chord_w4a16_weight* handle, void* stream) {
  g_last_error.clear();
  if (mode < 0 || mode > 2) return fail(CHORD_ERR_INVALID_ARGUMENT, "mode %d", mode);
  if (role < 0 || role > 1) return fail(CHORD_ERR_INVALID_ARGUMENT, "role %d", role);
  if (!qweight || !scales || !dst || !handle)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (group_size != kGroup)
    return fail(CHORD_ERR_UNSUPPORTED, "group size %d (only 32 is supported)", group_size);
  if (E < 1 || N <= 0 || K <= 0) return fail(CHORD_ERR_INVALID_ARGUMENT, "E=%d N=%d K=%d", E, N, K);
  if (K % kChunkK != 0) return fail(CHORD_ERR_UNSUPPORTED, "K=%d must be a multiple of 128", K);
  if (N % kTileRows != 0) return fail(CHORD_ERR_UNSUPPORTED, "N=%d must be a multiple of 16", N);
  if (role == CHORD_ROLE_GATE_UP && (N / 2) % 8 != 0)
    return fail(CHORD_ERR_UNSUPPORTED, "gate_up N=%d: I must be a multiple of 8", N);
  const size_t need = packed_bytes(E, N, K);
  if (dst_bytes < need)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "dst has %zu bytes, %zu needed", dst_bytes, need);
  CHORD_CHECK(check_device(nullptr));
  HIP_TRY(launch_pack(qweight, scales, E, N, K, role == CHORD_ROLE_GATE_UP ? 1 : 0,
                      static_cast<uint8_t*>(dst), static_cast<hipStream_t>(stream)),
          "pack launch");
  handle->magic = CHORD_WEIGHT_MAGIC;
  handle->version = CHORD_WEIGHT_VERSION;
  handle->mode = mode;
  handle->role = role;
  handle->num_experts = E;
  handle->n = N;
  handle->k = K;
  handle->group_size = kGroup;
  handle->data = dst;
  handle->bytes = need;
  return CHORD_OK;
}

int64_t chord_moe_align_max_padded(int T, int k, int num_local_experts, int block_m) {
  if (T < 0 || k < 1 || num_local_experts < 1 || block_m < 1) return 0;
  return (int64_t)T * k + (int64_t)num_local_experts * (block_m - 1);
}

size_t chord_moe_align_workspace_bytes(int T, int k, int num_local_experts, int block_m) {
  (void)block_m;
  if (T < 0 || k < 1 || num_local_experts < 1) return 0;
  const int64_t n = (int64_t)T * k;
  return (size_t)align_nchunks(n, num_local_experts) * num_local_experts * sizeof(int32_t) + 256;
}

chord_status chord_moe_align(const int32_t* topk_ids, int T, int k, int expert_begin,
                             int num_local_experts, int block_m, int32_t* sorted_ids,
                             int32_t* expert_ids, int32_t* num_tokens_post_padded,
                             int64_t max_padded, void* workspace, size_t ws_bytes, uint32_t flags,
                             void* stream) {
  g_last_error.clear();
  (void)flags;
  if (T < 0 || k < 1) return fail(CHORD_ERR_INVALID_ARGUMENT, "T=%d k=%d", T, k);
  if (num_local_experts < 1 || num_local_experts > kMaxExperts)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "num_local_experts=%d (1..%d)", num_local_experts,
                kMaxExperts);
  if (!valid_bm(block_m))
    return fail(CHORD_ERR_INVALID_ARGUMENT, "block_m=%d (16, 32, 64 or 128)", block_m);
  if ((T > 0 && !topk_ids) || !sorted_ids || !expert_ids || !num_tokens_post_padded)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  const int64_t n = (int64_t)T * k;
  if (n >= (int64_t)1 << 30) return fail(CHORD_ERR_UNSUPPORTED, "T*k too large");
  if (max_padded < chord_moe_align_max_padded(T, k, num_local_experts, block_m))
    return fail(CHORD_ERR_INVALID_ARGUMENT, "max_padded=%lld below T*k + E_l*(block_m-1)=%lld",
                (long long)max_padded,
                (long long)chord_moe_align_max_padded(T, k, num_local_experts, block_m));
  const size_t need = chord_moe_align_workspace_bytes(T, k, num_local_experts, block_m);
  const bool single = align_single_workgroup(n, num_local_experts);
  if (!single && (!workspace || ws_bytes < need))
    return fail(CHORD_ERR_WORKSPACE, "align workspace %zu bytes, %zu needed", ws_bytes, need);
  CHORD_CHECK(check_device(nullptr));
  AlignArgs a{};
  a.topk_ids = topk_ids;
  a.n = n;
  a.expert_begin = expert_begin;
  a.num_experts = num_local_experts;
  a.block_m = block_m;
  a.max_padded = max_padded;
  a.sorted_ids = sorted_ids;
  a.expert_ids = expert_ids;
  a.ntpp = num_tokens_post_padded;
  a.chunk = align_chunk(n, num_local_experts);
  a.nchunks = (int)align_nchunks(n, num_local_experts);
  if (!single) a.chunk_counts = static_cast<int32_t*>(workspace);
  const hipError_t e = launch_align(a, static_cast<hipStream_t>(stream));
  HIP_TRY(e, "align launch");
  g_last_plan = single ? "align: single workgroup" : "align: count/scatter";
  return CHORD_OK;
}

// ---------------------------------------------------------------------------
// Dispatch into the grouped layouts and the standalone combine.
// ---------------------------------------------------------------------------

int64_t chord_moe_dispatch_contiguous_rows(int T, int k, int num_local_experts) {
  const int64_t b = chord_moe_align_max_padded(T, k, num_local_experts, kContigBlock);
  if (b <= 0) return 0;
  return (b + kContigBlock - 1) / kContigBlock * kContigBlock;
}

size_t chord_moe_dispatch_workspace_bytes(int mode, int T, int k, int num_local_experts) {
  if (T < 0 || k < 1 || num_local_experts < 1) return 0;
  if (mode == CHORD_MODE_CONTIGUOUS) return dispatch_ws(T, k, num_local_experts, kContigBlock).total;
  if (mode == CHORD_MODE_MASKED) return dispatch_ws(T, k, num_local_experts, kMaskedBlock).total;
  return 0;
}

chord_status chord_moe_dispatch_contiguous(const chord_bf16* x, int T, int H,
                                           const int32_t* topk_ids, int k, int expert_begin,
                                           int num_local_experts, chord_bf16* a,
                                           int32_t* m_indices, int64_t max_rows,
                                           int32_t* flat_to_row, int32_t* num_rows,
                                           void* workspace, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!a || !m_indices || !num_rows) return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(a) % 16 != 0)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "a must be 16-byte aligned");
  const int64_t need = chord_moe_dispatch_contiguous_rows(T, k, num_local_experts);
  if (max_rows < need || max_rows % kContigBlock != 0)
    return fail(CHORD_ERR_INVALID_ARGUMENT,
                "max_rows=%lld: needs a multiple of 128 of at least %lld", (long long)max_rows,
                (long long)need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  DispatchArgs d{};
  CHORD_CHECK(dispatch_prepare(x, T, H, topk_ids, k, expert_begin, num_local_experts,
                               kContigBlock, flat_to_row, workspace, ws_bytes, st, &d));
  d.out = reinterpret_cast<uint16_t*>(a);
  d.max_rows = max_rows;
  d.m_indices = m_indices;
  d.num_rows = num_rows;
  HIP_TRY(launch_gather_contiguous(d, st), "dispatch launch");
  g_last_plan = "dispatch: align (128-row blocks) + contiguous gather";
  return CHORD_OK;
}

chord_status chord_moe_dispatch_masked(const chord_bf16* x, int T, int H, const int32_t* topk_ids,
                                       int k, int expert_begin, int num_local_experts, int max_m,
                                       chord_bf16* a3, int32_t* masked_m, int32_t* flat_to_row,
                                       int32_t* dropped, void* workspace, size_t ws_bytes,
                                       void* stream) {
  g_last_error.clear();
  if (max_m < 1) return fail(CHORD_ERR_INVALID_ARGUMENT, "max_m=%d must be positive", max_m);
  if (!a3 || !masked_m || !dropped) return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(a3) % 16 != 0)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "a3 must be 16-byte aligned");
  if ((int64_t)num_local_experts * max_m >= ((int64_t)1 << 31))
    return fail(CHORD_ERR_UNSUPPORTED, "E*max_m too large");
  hipStream_t st = static_cast<hipStream_t>(stream);
  DispatchArgs d{};
  CHORD_CHECK(dispatch_prepare(x, T, H, topk_ids, k, expert_begin, num_local_experts,
                               kMaskedBlock, flat_to_row, workspace, ws_bytes, st, &d));
  d.out = reinterpret_cast<uint16_t*>(a3);
  d.max_m = max_m;
  d.masked_m = masked_m;
  d.dropped = dropped;
  HIP_TRY(launch_gather_masked(d, st), "dispatch launch");
  g_last_plan = "dispatch: align (16-row blocks) + masked gather";
  return CHORD_OK;
}

chord_status chord_moe_combine(const chord_bf16* rows, int64_t n_rows, int H,
                               const int32_t* flat_to_row, const float* topk_weights, int T,
                               int k, chord_bf16* out, void* stream) {
  g_last_error.clear();
  if (T < 0 || k < 1 || H <= 0 || n_rows < 0)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "T=%d k=%d H=%d n_rows=%lld", T, k, H,
                (long long)n_rows);
  if (H % 8 != 0) return fail(CHORD_ERR_UNSUPPORTED, "H=%d must be a multiple of 8", H);
  if (T == 0) return CHORD_OK;
  if (!flat_to_row || !topk_weights || !out || (n_rows > 0 && !rows))
    return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(rows) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "rows and out must be 16-byte aligned");
  if (n_rows * H * 2 > INT32_MAX)
    return fail(CHORD_ERR_UNSUPPORTED, "rows span more than 2 GiB");
  CHORD_CHECK(check_device(nullptr));
  CombineArgs c{};
  c.rows = reinterpret_cast<const uint16_t*>(rows);
  c.topk_ids = nullptr;
  c.flat_to_row = flat_to_row;
  c.topk_weights = topk_weights;
  c.T = T;
  c.k = k;
  c.H = H;
  c.n_rows = n_rows;
  c.out = reinterpret_cast<uint16_t*>(out);
  HIP_TRY(launch_combine(c, static_cast<hipStream_t>(stream)), "combine launch");
  g_last_plan = "combine";
  return CHORD_OK;
}

int chord_w4a16_moe_indexed_block_m(int T, int k, int E_g, int E_l, int H, int I) {
  if (routed_call(T, k, E_g, E_l, H, I, nullptr)) return 0;  // no alignment needed
  // Expected rows per expert under uniform routing; a block of 16 or 32 rows
  // is then one tile of the weight-streaming GEMM.
  const int eg = E_g > 0 ? E_g : (E_l > 0 ? E_l : 1);
  const double tok_e = (double)std::max(T, 0) * std::max(k, 0) / eg;
  return (tok_e > 16.0 && tok_e <= 32.0) ? 32 : 16;
}

size_t chord_w4a16_moe_workspace_bytes(int mode, int T, int k, int E_l, int H, int I,
                                       int64_t rows) {
  if (mode < 0 || mode > 2 || T < 0 || k < 0 || E_l < 1 || H <= 0 || I <= 0 || rows < 0) return 0;
  return layer_ws(mode, T, k, E_l, H, I, rows).total;
}

}  // extern "C"

namespace {

// The indexed layer on a given workspace.  no_alloc: the call may not create
// HIP objects (no profiling events, no side stream for kernel 3).
chord_status indexed_impl(const chord_bf16* x, int T, int H, int I, const chord_w4a16_weight* w13,
                          const chord_w4a16_weight* w2, const int32_t* topk_ids,
                          const float* topk_weights, int k, int expert_begin,
                          int num_global_experts, const int32_t* sorted_ids,
                          const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                          int64_t max_padded, int block_m, chord_bf16* out, void* workspace,
                          size_t ws_bytes, const chord_schedule* override, uint32_t flags,
                          void* stream, bool no_alloc) {
  if (T < 0 || k < 1) return fail(CHORD_ERR_INVALID_ARGUMENT, "T=%d k=%d", T, k);
  CHORD_CHECK(check_pair(w13, w2, CHORD_MODE_INDEXED, H, I));
  const int E_l = w13->num_experts;
  if (T == 0) return CHORD_OK;
  if (!x || !topk_ids || !topk_weights || !out)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  if ((int64_t)T * k >= ((int64_t)1 << 30))
    return fail(CHORD_ERR_UNSUPPORTED, "routing tensors too large");
  if (override && !override_in_range(override))
    return fail(CHORD_ERR_INVALID_ARGUMENT, "schedule override out of range");
  // A routed call derives its rows from topk_ids and reads no alignment.
  const bool routed = routed_call(T, k, num_global_experts, E_l, H, I, override);
  if (routed) {
    max_padded = 0;
    block_m = 0;
  } else {
    if (!sorted_ids || !expert_ids || !num_tokens_post_padded)
      return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument (this call reads the alignment)");
    if (!valid_bm(block_m))
      return fail(CHORD_ERR_INVALID_ARGUMENT, "block_m=%d (16, 32, 64 or 128)", block_m);
    if (max_padded < chord_moe_align_max_padded(T, k, E_l, block_m))
      return fail(CHORD_ERR_INVALID_ARGUMENT, "max_padded=%lld below T*k + E_l*(block_m-1)",
                  (long long)max_padded);
    if (max_padded >= ((int64_t)1 << 31))
      return fail(CHORD_ERR_UNSUPPORTED, "routing tensors too large");
  }
  if ((int64_t)T * k * H * 2 > INT32_MAX)  // y rows are read through a 32-bit buffer offset
    return fail(CHORD_ERR_UNSUPPORTED, "T*k*H*2 exceeds 2 GiB");
  if (no_alloc && override && override->kernel == 3)
    return fail(CHORD_ERR_INVALID_ARGUMENT,
                "kernel 3 needs a side stream, which the allocation-free call does not create");
  const WsLayout ws = layer_ws(kIndexed, T, k, E_l, H, I, max_padded);
  if (no_alloc && ws.total > kNoAllocScratchBytes)
    return fail(CHORD_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu",
                ws.total, kNoAllocScratchBytes);
  if (no_alloc) {
    CHORD_CHECK(check_device(nullptr));
    CHORD_CHECK(noalloc_scratch(&workspace));
    ws_bytes = kNoAllocScratchBytes;
  }
  if (!workspace || ws_bytes < ws.total)
    return fail(CHORD_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, ws.total);
  int cus = 0;
  CHORD_CHECK(check_device(&cus));
  PlanKey key = make_key(kIndexed, T, k, num_global_experts, E_l, H, I, block_m, cus, max_padded);
  fill_override(key, override);
  const Plan plan = get_plan(key);
  if (no_alloc && plan.kernel == 3)
    return fail(CHORD_ERR_INVALID_ARGUMENT,
                "kernel 3 needs a side stream, which the allocation-free call does not create");
  set_plan_text("indexed", plan);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* wsp = static_cast<uint8_t*>(workspace);
  if (plan.routed != routed)
    return fail(CHORD_ERR_HIP, "internal: routed plan mismatch");
  TileBuildArgs tb{};
  tb.num_experts = E_l;
  tb.validate = (flags & CHORD_FLAG_VALIDATE) ? 1 : 0;
  tb.expert_ids = expert_ids;
  tb.ntpp = num_tokens_post_padded;
  tb.block_m = block_m;
  tb.max_padded = max_padded;
  uint16_t* y = reinterpret_cast<uint16_t*>(wsp + ws.y);
  StageTimer timer(st, !no_alloc);
  RouteCall rc;
  rc.topk_ids = topk_ids;
  rc.topk_weights = topk_weights;
  rc.expert_begin = expert_begin;
  rc.T = T;
  rc.out = reinterpret_cast<uint16_t*>(out);
  CHORD_CHECK(run_expert_gemms(kIndexed, plan, ws, wsp, w13, w2, H, I, x, T,
                               std::max<int64_t>(max_padded, (int64_t)T * k), sorted_ids, k,
                               (int64_t)T * k, nullptr, y, (int64_t)T * k, nullptr, tb, st, timer,
                               &rc));
  if (plan.fused) {  // the down launch already combined into out
    timer.mark(4);
    timer.finish();
    return finish_validate(flags, ws, wsp, st);
  }
  CombineArgs c{};
  c.rows = y;
  c.topk_ids = topk_ids;
  c.flat_to_row = nullptr;
  c.topk_weights = topk_weights;
  c.T = T;
  c.k = k;
  c.H = H;
  c.expert_begin = expert_begin;
  c.num_experts = E_l;
  c.n_rows = (int64_t)T * k;
  c.out = out;
  // The rows actually read are the local slots, about T*k*E_l/E_g of the
  // T*k the buffer is sized for.
  {
    const int eg = num_global_experts > E_l ? num_global_experts : E_l;
    c.read_bytes = (int64_t)((double)T * k * E_l / eg * H * 2);
  }
  HIP_TRY(launch_combine(c, st), "combine launch");
  timer.mark(4);
  timer.finish();
  return finish_validate(flags, ws, wsp, st);
}

}  // namespace

extern "C" {

chord_status chord_w4a16_moe_indexed(const chord_bf16* x, int T, int H, int I,
                                     const chord_w4a16_weight* w13, const chord_w4a16_weight* w2,
                                     const int32_t* topk_ids, const float* topk_weights, int k,
                                     int expert_begin, int num_global_experts,
                                     const int32_t* sorted_ids, const int32_t* expert_ids,
                                     const int32_t* num_tokens_post_padded, int64_t max_padded,
                                     int block_m, chord_bf16* out, void* workspace,
                                     size_t ws_bytes, const chord_schedule* override,
                                     uint32_t flags, void* stream) {
  g_last_error.clear();
  return indexed_impl(x, T, H, I, w13, w2, topk_ids, topk_weights, k, expert_begin,
                      num_global_experts, sorted_ids, expert_ids, num_tokens_post_padded,
                      max_padded, block_m, out, workspace, ws_bytes, override, flags, stream,
                      false);
}

chord_status chord_w4a16_moe_indexed_noalloc(const chord_bf16* x, int T, int H, int I,
                                             const chord_w4a16_weight* w13,
                                             const chord_w4a16_weight* w2,
                                             const int32_t* topk_ids, const float* topk_weights,
                                             int k, int expert_begin, int num_global_experts,
                                             const int32_t* sorted_ids, const int32_t* expert_ids,
                                             const int32_t* num_tokens_post_padded,
                                             int64_t max_padded, int block_m, chord_bf16* out,
                                             const chord_schedule* override, uint32_t flags,
                                             void* stream) {
  g_last_error.clear();
  return indexed_impl(x, T, H, I, w13, w2, topk_ids, topk_weights, k, expert_begin,
                      num_global_experts, sorted_ids, expert_ids, num_tokens_post_padded,
                      max_padded, block_m, out, nullptr, 0, override, flags, stream, true);
}

chord_status chord_w4a16_moe_grouped_contiguous(
    const chord_bf16* a, int64_t M, const int32_t* m_indices, int64_t valid_m_hint,
    const chord_w4a16_weight* w13, const chord_w4a16_weight* w2, int H, int I,
    const float* row_weights, const int32_t* flat_to_row, int T, int k, const float* topk_weights,
    chord_bf16* out_rows, chord_bf16* out_tokens, void* workspace, size_t ws_bytes,
    const chord_schedule* override, uint32_t flags, void* stream) {
  g_last_error.clear();
  if (override)
    return fail(CHORD_ERR_INVALID_ARGUMENT,
                "grouped dispatch chooses its own schedule; overrides are rejected");
  CHORD_CHECK(check_pair(w13, w2, CHORD_MODE_CONTIGUOUS, H, I));
  const int E_l = w13->num_experts;
  if (M < 0 || M % 128 != 0) return fail(CHORD_ERR_INVALID_ARGUMENT, "M=%lld must be a multiple of 128", (long long)M);
  if (M / 128 > kMaxSegments) return fail(CHORD_ERR_UNSUPPORTED, "M too large");
  const bool want_tokens = out_tokens != nullptr;
  if (want_tokens && (!flat_to_row || !topk_weights || T < 0 || k < 1))
    return fail(CHORD_ERR_INVALID_ARGUMENT, "token combine needs flat_to_row, topk_weights, T, k");
  if (want_tokens && M * H * 2 > INT32_MAX)  // rows are read through a 32-bit buffer offset
    return fail(CHORD_ERR_UNSUPPORTED, "M*H*2 exceeds 2 GiB for the token combine");
  if (M == 0) {
    if (want_tokens && T > 0) {
      CHORD_CHECK(check_device(nullptr));
      HIP_TRY(launch_zero(out_tokens, (int64_t)T * H, static_cast<hipStream_t>(stream)), "zero");
    }
    return CHORD_OK;
  }
  if (!a || !m_indices || !out_rows) return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  const WsLayout ws = layer_ws(kContiguous, T, k, E_l, H, I, M);
  if (!workspace || ws_bytes < ws.total)
    return fail(CHORD_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, ws.total);
  int cus = 0;
  CHORD_CHECK(check_device(&cus));
  const PlanKey key = make_key(kContiguous, T, k, 0, E_l, H, I,
                               (int)std::min<int64_t>(valid_m_hint, 1 << 30), cus, M);
  const Plan plan = get_plan(key);
  set_plan_text("contiguous", plan);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* wsp = static_cast<uint8_t*>(workspace);
  TileBuildArgs tb{};
  tb.num_experts = E_l;
  tb.validate = (flags & CHORD_FLAG_VALIDATE) ? 1 : 0;
  tb.m_indices = m_indices;
  tb.M = M;
  StageTimer timer(st);
  CHORD_CHECK(run_expert_gemms(kContiguous, plan, ws, wsp, w13, w2, H, I, a, M, M, nullptr, 1, 0,
                               m_indices, out_rows, M, row_weights, tb, st, timer));
  if (want_tokens && T > 0) {
    CombineArgs c{};
    c.rows = out_rows;
    c.topk_ids = nullptr;
    c.flat_to_row = flat_to_row;
    c.topk_weights = topk_weights;
    c.T = T;
    c.k = k;
    c.H = H;
    c.num_experts = E_l;
    c.n_rows = M;
    c.out = out_tokens;
    HIP_TRY(launch_combine(c, st), "combine launch");
  }
  timer.mark(4);
  timer.finish();
  return finish_validate(flags, ws, wsp, st);
}

chord_status chord_w4a16_moe_grouped_masked(const chord_bf16* a, int E, int max_m,
                                            const int32_t* masked_m, int expected_m,
                                            const chord_w4a16_weight* w13,
                                            const chord_w4a16_weight* w2, int H, int I,
                                            const float* row_weights, chord_bf16* out,
                                            void* workspace, size_t ws_bytes,
                                            const chord_schedule* override, uint32_t flags,
                                            void* stream) {
  g_last_error.clear();
  if (override)
    return fail(CHORD_ERR_INVALID_ARGUMENT,
                "grouped dispatch chooses its own schedule; overrides are rejected");
  if (expected_m <= 0)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "expected_m=%d must be positive", expected_m);
  CHORD_CHECK(check_pair(w13, w2, CHORD_MODE_MASKED, H, I));
  if (E != w13->num_experts)
    return fail(CHORD_ERR_INVALID_ARGUMENT, "E=%d but the weights hold %d experts", E,
                w13->num_experts);
  if (max_m < 0) return fail(CHORD_ERR_INVALID_ARGUMENT, "max_m=%d", max_m);
  if (max_m == 0) return CHORD_OK;
  if (!a || !masked_m || !out) return fail(CHORD_ERR_INVALID_ARGUMENT, "null pointer argument");
  const int64_t rows = (int64_t)E * max_m;
  if (rows >= ((int64_t)1 << 31)) return fail(CHORD_ERR_UNSUPPORTED, "E*max_m too large");
  const WsLayout ws = layer_ws(kMasked, 0, 0, E, H, I, rows);
  if (!workspace || ws_bytes < ws.total)
    return fail(CHORD_ERR_WORKSPACE, "workspace %zu bytes, %zu needed", ws_bytes, ws.total);
  int cus = 0;
  CHORD_CHECK(check_device(&cus));
  const PlanKey key = make_key(kMasked, 0, 0, 0, E, H, I, expected_m, cus, rows);
  const Plan plan = get_plan(key);
  set_plan_text("masked", plan);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* wsp = static_cast<uint8_t*>(workspace);
  TileBuildArgs tb{};
  tb.num_experts = E;
  tb.validate = (flags & CHORD_FLAG_VALIDATE) ? 1 : 0;
  tb.masked_m = masked_m;
  tb.max_m = max_m;
  StageTimer timer(st);
  CHORD_CHECK(run_expert_gemms(kMasked, plan, ws, wsp, w13, w2, H, I, a, rows, rows, nullptr, 1,
                               0, nullptr, out, rows, row_weights, tb, st, timer));
  timer.mark(4);
  timer.finish();
  return finish_validate(flags, ws, wsp, st);
}

}  // extern "C"
