// C ABI of the TriAttention pruning pass (declared in include/tria.h):
// host-side validation, workspace layout, launch sequencing and kernel timing.
// All arithmetic of the pass runs in the kernels of tria_kernels.hip.
#include "tria.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <vector>

#include "tria_kernels.h"
#include "tria_host.h"

namespace {

// ------------------------------------------------------------------ log
// The host's decisions (tile sizes, grids, kernel variants, strategies) and every
// error an entry point returns, one line each on stderr, prefixed "[tria] ".  On when
// the environment variable TRIA_LOG holds anything but "" or "0" at the first call
// that logs, or after tria_log(1).
std::atomic<int> g_log{-1};

bool log_on() {
  int v = g_log.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("TRIA_LOG");
    int want = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    g_log.compare_exchange_strong(v, want);
    v = g_log.load(std::memory_order_relaxed);
  }
  return v > 0;
}

void tlog(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[768];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[tria] %s\n", buf);
}

thread_local char g_err[512] = "";

tria_status fail(tria_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  tlog("error %d (%s): %s", (int)s, tria_strerror(s), g_err);
  return s;
}

const char* pairing_name(int p) { return p == TRIA_PAIR_NEOX ? "NEOX" : "interleaved"; }
const char* layout_name(const tria_kv_view* v) { return v->block_table ? "paged" : "dense"; }

}  // namespace

void tria::set_last_error(const char* msg) { snprintf(g_err, sizeof g_err, "%s", msg); }

namespace {

// ------------------------------------------------------------------ timing
enum { kIdCoef = 0, kIdScore, kIdSelect, kIdCompact, kIdCalib, kNumIds };
const char* const kNames[kNumIds] = {"k_coef", "k_score", "k_select", "k_compact", "k_calib"};

struct Rec {
  int id;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<Rec> g_recs;
// set while tria_pass_noalloc runs on this thread: no timing events are created
thread_local bool t_no_events = false;

// Runs `launch` on `stream`, bracketed by HIP events on the same stream when
// timing is on.  The events skip the system-scope fence (an L2 writeback and
// invalidate) a default event performs on record; each recorded event still idles
// the GPU for several microseconds between kernels.
template <class Fn>
hipError_t timed(int id, hipStream_t stream, Fn&& launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    on = g_timing && !t_no_events;
  }
  if (!on) return launch();
  Rec r{id, nullptr, nullptr};
  hipError_t e = hipEventCreateWithFlags(&r.a, hipEventDisableSystemFence);
  if (e != hipSuccess) return e;
  e = hipEventCreateWithFlags(&r.b, hipEventDisableSystemFence);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(r.a, stream)) != hipSuccess) return e;
  if ((e = launch()) != hipSuccess) return e;
  if ((e = hipEventRecord(r.b, stream)) != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_tmu);
  g_recs.push_back(r);
  return hipSuccess;
}

tria_status launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TRIA_OK;
  return fail(TRIA_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

// cap on tria_score's persistent grid (0: the device's resident capacity)
std::atomic<int32_t> g_score_wg_cap{0};
// polls of the score kernel's bounded wait for a group's moments (< 0: none)
std::atomic<int32_t> g_wait_polls{tria::kPollLimit};
// tria_select's work distribution (tria_select_strategy_t)
std::atomic<int32_t> g_select_strategy{TRIA_SELECT_AUTO};

// ------------------------------------------------------------------ validation
tria_status check_params(const tria_params* p) {
  if (!p) return fail(TRIA_EINVAL, "params is NULL");
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(TRIA_ESHAPE, "head_dim %d not in {64, 128, 256}", p->head_dim);
  if (p->n_kv_heads < 1) return fail(TRIA_ESHAPE, "n_kv_heads %d < 1", p->n_kv_heads);
  if (p->group < 1 || p->group > tria::kMaxGroup)
    return fail(TRIA_ESHAPE, "group %d not in [1, %d]", p->group, tria::kMaxGroup);
  if (p->n_layers < 1) return fail(TRIA_ESHAPE, "n_layers %d < 1", p->n_layers);
  if (p->pairing != TRIA_PAIR_NEOX && p->pairing != TRIA_PAIR_INTERLEAVED)
    return fail(TRIA_EINVAL, "unknown pairing %d", p->pairing);
  if (p->agg != TRIA_AGG_MEAN && p->agg != TRIA_AGG_MAX) return fail(TRIA_EINVAL, "unknown agg %d", p->agg);
  if (!(p->rope_base > 1.0) || !std::isfinite(p->rope_base))
    return fail(TRIA_EINVAL, "rope_base must be a finite value > 1");
  if (!p->offsets) return fail(TRIA_EINVAL, "offsets is NULL");
  if (p->n_offsets < 1 || p->n_offsets > tria::kMaxOffsets)
    return fail(TRIA_EINVAL, "n_offsets %d not in [1, %d]", p->n_offsets, tria::kMaxOffsets);
  for (int i = 0; i < p->n_offsets; ++i)
    if (p->offsets[i] < 0 || p->offsets[i] > (int64_t(1) << 40))
      return fail(TRIA_EINVAL, "offset[%d] = %lld outside [0, 2^40]", i, (long long)p->offsets[i]);
  if (p->sink < 0 || p->window < 0) return fail(TRIA_EINVAL, "sink and window must be >= 0");
  if (p->offset_reduce != TRIA_OFFSETS_MEAN && p->offset_reduce != TRIA_OFFSETS_MAX)
    return fail(TRIA_EINVAL, "unknown offset_reduce %d", p->offset_reduce);
  return TRIA_OK;
}

tria_status check_view(const tria_kv_view* v, const char* name, int head_dim, int32_t n_slots) {
  if (!v) return fail(TRIA_EINVAL, "%s view is NULL", name);
  if (!v->base) return fail(TRIA_EINVAL, "%s base is NULL", name);
  if (reinterpret_cast<uintptr_t>(v->base) % 16 != 0) return fail(TRIA_ESHAPE, "%s base not 16-byte aligned", name);
  if (v->stride_head < 0 || v->stride_slot < 0 || v->stride_unit < 0)
    return fail(TRIA_ESHAPE, "%s has a negative stride", name);
  if (v->stride_head % 8 || v->stride_slot % 8 || v->stride_unit % 8)
    return fail(TRIA_ESHAPE, "%s strides must be multiples of 8 elements", name);
  if (v->block_table) {
    if (v->block_size < 1 || v->max_blocks < 1 || v->n_pool_blocks < 1)
      return fail(TRIA_ESHAPE, "%s: paged view needs block_size, max_blocks, n_pool_blocks >= 1", name);
    if ((int64_t)v->max_blocks * v->block_size < n_slots)
      return fail(TRIA_ESHAPE, "%s: block table covers %lld slots < %d", name,
                  (long long)v->max_blocks * v->block_size, n_slots);
  }
  (void)head_dim;
  return TRIA_OK;
}

tria::KView kview(const tria_kv_view* v) {
  return tria::KView{static_cast<const uint16_t*>(v->base), v->stride_unit, v->stride_head, v->stride_slot,
                     v->block_table, v->block_size, v->max_blocks, v->n_pool_blocks};
}

tria::MutKView mkview(const tria_kv_view* v) {
  return tria::MutKView{static_cast<uint16_t*>(v->base), v->stride_unit, v->stride_head, v->stride_slot,
                        v->block_table, v->block_size, v->max_blocks, v->n_pool_blocks};
}

// Byte interval [lo, hi) covered by a dense view of `units` x Hkv x `slots` rows.
void dense_range(const tria_kv_view* v, int32_t units, int32_t hkv, int32_t slots, int d, uintptr_t& lo,
                 uintptr_t& hi) {
  lo = reinterpret_cast<uintptr_t>(v->base);
  const int64_t last = (int64_t)(units - 1) * v->stride_unit + (int64_t)(hkv - 1) * v->stride_head +
                       (int64_t)(slots - 1) * v->stride_slot + d;
  hi = lo + 2 * (uintptr_t)last;
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

// ------------------------------------------------------------------ workspace
struct Layout {
  size_t B, Bmax, nconst, part, gstat, arrive, claim, hist, st, tiles, list, masks, total;
  int32_t tile, n_tiles, n_st;   // keys per score tile, score tiles and selection tiles per row
  tria::OffsetBlocks ob;
};

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: [flag word | MFMA B operands and reference magnitudes | (maximum over
// offsets) offset-block B operands | norm constants | tile moments | merged moments |
// tile arrival counts | tile claim counter | aggregate histograms | selection state |
// per-tile counts | candidates | per-tile slot masks]
Layout layout(const tria_params* p, int32_t n_units, int32_t n_max) {
  Layout L{};
  const size_t U = (size_t)n_units, hq = (size_t)p->n_kv_heads * p->group, d = (size_t)p->head_dim;
  L.tile = tria::score_tile_keys(p->group, p->offset_reduce == TRIA_OFFSETS_MAX, n_max);
  L.n_tiles = (n_max + L.tile - 1) / L.tile;
  size_t off = 256;  // flag word
  L.B = off;
  off += al256(U * (size_t)p->n_kv_heads * (d / 16 + d / 64) * 64 * 16);  // B operands, reference magnitudes
  L.ob = tria::offset_blocks(p->n_offsets, p->group);
  L.Bmax = off;
  if (p->offset_reduce == TRIA_OFFSETS_MAX)
    off += al256(U * (size_t)p->n_kv_heads * L.ob.nblk * (d / 32) * 64 * 16);
  L.nconst = off;
  off += al256(U * hq * 4);
  L.part = off;
  off += al256(U * hq * (size_t)L.n_tiles * 3 * 8);
  L.gstat = off;
  off += al256(U * hq * 8);
  L.arrive = off;
  off += al256(U * (size_t)p->n_kv_heads * 4);
  L.claim = off;
  off += 256;  // the tile claim counter
  L.hist = off;
  off += al256(U * (size_t)p->n_kv_heads * tria::kBins * 4);
  // selection: per-group state, per-tile counts, candidate lists
  const size_t ug = U * (size_t)p->n_kv_heads;
  L.n_st = (n_max + tria::kSelTile - 1) / tria::kSelTile;
  L.st = off;
  off += al256(ug * sizeof(tria::SelState));
  L.tiles = off;
  off += al256(ug * (size_t)L.n_st * 3 * 4);  // above-b1 counts, offsets, candidates
  L.list = off;
  off += al256(ug * (size_t)n_max * 4);
  L.masks = off;  // per tile and thread: slots above the threshold bin, slots in it
  off += al256(ug * (size_t)L.n_st * 256 * sizeof(tria::SelMask) * 2);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t tria_workspace_size(const tria_params* p, int32_t n_units, int32_t n_max) {
  if (check_params(p) != TRIA_OK || n_units < 0 || n_max < 0) return 0;
  return layout(p, n_units, n_max).total;
}

}  // extern "C"

namespace {

// The bodies of the entry points: every check first; with dry = true nothing is
// launched (tria_pass_noalloc validates all three steps before it launches any).
tria_status score_impl(const tria_params* p, const tria_kv_view* k, int32_t n_units, int32_t n_max,
                       const int32_t* len, const int32_t* unit_layer, const int32_t* q_pos,
                       const float* q_mean_re, const float* q_mean_im, const float* q_abs_mean, float* raw,
                       float* agg, void* ws, size_t ws_bytes, void* stream, bool dry) {
  tria_status st = check_params(p);
  if (st != TRIA_OK) return st;
  if (n_units < 0 || n_max < 0) return fail(TRIA_EINVAL, "n_units and n_max must be >= 0");
  if (n_max % 16 != 0) return fail(TRIA_ESHAPE, "n_max %d must be a multiple of 16", n_max);
  if ((st = check_view(k, "k", p->head_dim, n_max)) != TRIA_OK) return st;
  if (!len || !unit_layer || !q_pos || !q_mean_re || !q_mean_im || !q_abs_mean || !agg)
    return fail(TRIA_EINVAL, "a required device pointer is NULL");
  if (reinterpret_cast<uintptr_t>(agg) % 16 || (raw && reinterpret_cast<uintptr_t>(raw) % 16))
    return fail(TRIA_ESHAPE, "raw and agg must be 16-byte aligned");
  if (!ws) return fail(TRIA_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(TRIA_EWORKSPACE, "workspace must be 256-byte aligned");
  const Layout L = layout(p, n_units, n_max);
  if (ws_bytes < L.total)
    return fail(TRIA_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  if (n_units == 0 || n_max == 0) return TRIA_OK;
  const int omax = p->offset_reduce == TRIA_OFFSETS_MAX ? 1 : 0;
  const bool paged = k->block_table != nullptr;
  if (omax && tria::score_lds(p->head_dim, p->group, paged, 1, L.ob.nblk, L.tile, k->block_size, 0) > 160 * 1024)
    return fail(TRIA_ESHAPE, "maximum over %d offsets: %d coefficient blocks of head_dim %d do not fit in LDS",
                p->n_offsets, L.ob.nblk, p->head_dim);
  const int wg_cap = g_score_wg_cap.load();
  // The mean over offsets with G > 4 keeps two score buffers of 1024-key tiles; for
  // a dense cache whose tiles all fit on the device at once with one buffer of twice
  // as long tiles, that mode (k_score_single) runs instead: no tile waits on another
  // round, and half as many tiles pay the per-tile exchange (e.g. 8 KV heads x
  // 131072 keys, G = 8: one round of 512 tiles instead of two of 512).  The choice
  // depends on the device's resident capacity only, not on
  // tria_score_max_workgroups: the tiles, and so the rounding of the merged moments,
  // do not change with the grid (a capped grid runs the single-buffer mode in
  // several rounds; its waits still end, since a workgroup waits only once its own
  // tile is published)
  int tile = L.tile, n_tiles = L.n_tiles, single = 0;
  if (!omax && !paged && p->group > 4) {
    const int t1 = tria::single_tile_keys(n_max);
    const int nt1 = (n_max + t1 - 1) / t1;
    const int cap1 =
        tria::score_capacity(p->head_dim, p->pairing, paged, p->group, 0, L.ob.nblk, t1, k->block_size, 1);
    if (cap1 > 0 && (long)n_units * p->n_kv_heads * nt1 <= (long)cap1) {
      tile = t1;
      n_tiles = nt1;
      single = 1;
    }
  }
  // the tiles of one (unit, KV head) wait for each other: they must all fit at once
  const int cap = tria::score_capacity(p->head_dim, p->pairing, paged, p->group, omax, L.ob.nblk, tile,
                                       k->block_size, single);
  if (cap < 0) return fail(TRIA_ELAUNCH, "k_score occupancy query failed");
  if (n_tiles > cap)
    return fail(TRIA_ESHAPE, "n_max %d needs %d concurrent score tiles per (unit, KV head); the device holds %d",
                n_max, n_tiles, cap);
  if (wg_cap > 0 && n_tiles > wg_cap)
    return fail(TRIA_ESHAPE, "n_max %d needs %d concurrent score tiles per (unit, KV head); the workgroup cap is %d",
                n_max, n_tiles, wg_cap);
  if (log_on()) {
    const long tiles = (long)n_units * p->n_kv_heads * n_tiles;
    const int grid_cap = wg_cap > 0 && wg_cap < cap ? wg_cap : cap;
    tlog("score: %d units x %d KV heads x n_max %d, d %d, G %d, %s, %s K, %d offsets (%s), %s aggregation: "
         "%s, tiles of %d keys (%d per (unit, KV head), %ld in all), %s, grid %ld (resident capacity %d, cap %d), "
         "LDS %zu B, moment wait %d polls, workspace %zu of %zu B",
         n_units, p->n_kv_heads, n_max, p->head_dim, p->group, pairing_name(p->pairing), layout_name(k),
         p->n_offsets, omax ? "maximum" : "mean", p->agg == TRIA_AGG_MAX ? "max" : "mean",
         omax ? "k_score_max" : single ? "k_score_single" : "k_score", tile, n_tiles, tiles,
         single ? "one score buffer" : "two score buffers",
         tiles < grid_cap ? tiles : (long)grid_cap, cap, wg_cap,
         tria::score_lds(p->head_dim, p->group, paged, omax, L.ob.nblk, tile, k->block_size, single),
         g_wait_polls.load(), L.total, ws_bytes);
  }
  if (dry) return TRIA_OK;

  char* w = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* flags = reinterpret_cast<int32_t*>(w);
  uint32_t* B = reinterpret_cast<uint32_t*>(w + L.B);
  double* part = reinterpret_cast<double*>(w + L.part);
  int32_t* next_tile = reinterpret_cast<int32_t*>(w + L.claim);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + L.hist);

  tria::Offsets offs{};
  offs.n = p->n_offsets;
  for (int i = 0; i < p->n_offsets; ++i) offs.v[i] = (double)p->offsets[i];

  float* nconst = reinterpret_cast<float*>(w + L.nconst);
  tria::CoefArgs ca{kview(k), n_units, p->n_kv_heads * p->group, p->n_kv_heads, p->head_dim, p->n_layers,
                    p->pairing, std::log(p->rope_base), len, unit_layer, q_pos, q_mean_re, q_mean_im, q_abs_mean,
                    p->group, n_tiles, tile, n_max, B, nconst,
                    reinterpret_cast<uint64_t*>(part), next_tile, hist, flags, omax,
                    reinterpret_cast<uint32_t*>(w + L.Bmax), L.ob, reinterpret_cast<uint64_t*>(w + L.gstat),
                    reinterpret_cast<int32_t*>(w + L.arrive)};
  hipError_t e = timed(kIdCoef, s, [&] { return tria::launch_coef(ca, offs, s); });
  if ((st = launch_status(e, "k_coef")) != TRIA_OK) return st;

  tria::ScoreArgs sa{kview(k), n_units, n_max, p->n_kv_heads, p->group, p->sink, p->window,
                     tile, n_tiles, p->agg,
                     len, B, nconst, raw, part, agg, next_tile, hist, flags, omax,
                     reinterpret_cast<const uint32_t*>(w + L.Bmax), L.ob, g_wait_polls.load(),
                     reinterpret_cast<uint64_t*>(w + L.gstat), reinterpret_cast<int32_t*>(w + L.arrive), single};
  e = timed(kIdScore, s, [&] { return tria::launch_score(sa, p->head_dim, p->pairing, wg_cap, s); });
  return launch_status(e, "k_score");
}

tria_status select_impl(const tria_params* p, int32_t n_units, int32_t n_max, int32_t b_max, const int32_t* len,
                        const int32_t* budget, const float* agg, int32_t* idx, int32_t* cnt, void* ws,
                        size_t ws_bytes, void* stream, bool dry) {
  tria_status st = check_params(p);
  if (st != TRIA_OK) return st;
  if (n_units < 0 || n_max < 0 || b_max < 0) return fail(TRIA_EINVAL, "n_units, n_max and b_max must be >= 0");
  if (!len || !budget || !agg || !idx || !cnt) return fail(TRIA_EINVAL, "a required device pointer is NULL");
  if (n_max % 16 != 0) return fail(TRIA_ESHAPE, "n_max %d must be a multiple of 16", n_max);
  if (reinterpret_cast<uintptr_t>(agg) % 16) return fail(TRIA_ESHAPE, "agg must be 16-byte aligned");
  if (!ws) return fail(TRIA_EWORKSPACE, "workspace is NULL (tria_select reads tria_score's histograms from it)");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(TRIA_EWORKSPACE, "workspace must be 256-byte aligned");
  const Layout L = layout(p, n_units, n_max);
  if (ws_bytes < L.total)
    return fail(TRIA_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  if (n_units == 0) return TRIA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (L.n_st > tria::kMaxSelTiles)
    return fail(TRIA_ESHAPE, "n_max %d exceeds the selection's %d tiles", n_max, tria::kMaxSelTiles);
  if (log_on()) {
    const int strategy = g_select_strategy.load();
    const bool per_group = strategy == TRIA_SELECT_PER_GROUP && n_max <= tria::kSelGroupMax;
    if (per_group)
      tlog("select: %d units x %d KV heads, n_max %d, b_max %d: k_sel_group (one workgroup per (unit, KV head))",
           n_units, p->n_kv_heads, n_max, b_max);
    else
      tlog("select: %d units x %d KV heads, n_max %d, b_max %d: k_sel_thresh, k_sel_collect, k_sel_refine "
           "(ranks up to %d candidates, else radix passes), k_sel_emit; %d selection tiles of %d slots per row%s",
           n_units, p->n_kv_heads, n_max, b_max, tria::kSelRankMax, L.n_st, tria::kSelTile,
           strategy == TRIA_SELECT_PER_GROUP ? " (per-group requested; the row exceeds its limit)" : "");
  }
  if (dry) return TRIA_OK;
  int32_t* tiles = reinterpret_cast<int32_t*>(w + L.tiles);
  const size_t nt = (size_t)n_units * p->n_kv_heads * L.n_st;
  tria::SelectArgs sa{n_units, n_max, b_max, p->n_kv_heads, p->sink, p->window, L.n_st, len, budget, agg,
                      reinterpret_cast<const uint32_t*>(w + L.hist), reinterpret_cast<tria::SelState*>(w + L.st),
                      tiles, tiles + nt, tiles + 2 * nt, reinterpret_cast<int32_t*>(w + L.list),
                      reinterpret_cast<tria::SelMask*>(w + L.masks),
                      reinterpret_cast<tria::SelMask*>(w + L.masks) + nt * 256, idx, cnt,
                      reinterpret_cast<int32_t*>(w)};
  const int strategy = g_select_strategy.load();
  hipError_t e = timed(kIdSelect, s, [&] { return tria::launch_select(sa, strategy, s); });
  return launch_status(e, "k_select");
}

tria_status compact_impl(const tria_params* p, const tria_kv_view* k_src, const tria_kv_view* v_src,
                         const int32_t* pos_src, int32_t pos_heads, int32_t n_units, int32_t n_max, int32_t b_max,
                         const int32_t* len, const int32_t* idx, const int32_t* cnt, const tria_kv_view* k_dst,
                         const tria_kv_view* v_dst, int32_t* pos_dst, void* stream, bool dry) {
  tria_status st = check_params(p);
  if (st != TRIA_OK) return st;
  if (n_units < 0 || n_max < 0 || b_max < 0) return fail(TRIA_EINVAL, "n_units, n_max and b_max must be >= 0");
  if ((st = check_view(k_src, "k_src", p->head_dim, n_max)) != TRIA_OK) return st;
  if ((st = check_view(v_src, "v_src", p->head_dim, n_max)) != TRIA_OK) return st;
  if ((st = check_view(k_dst, "k_dst", p->head_dim, b_max)) != TRIA_OK) return st;
  if ((st = check_view(v_dst, "v_dst", p->head_dim, b_max)) != TRIA_OK) return st;
  if (!len || !idx || !cnt) return fail(TRIA_EINVAL, "a required device pointer is NULL");
  if (pos_src && pos_heads != 1 && pos_heads != p->n_kv_heads)
    return fail(TRIA_ESHAPE, "pos_heads %d must be 1 or n_kv_heads", pos_heads);
  // with no source slots no index is valid: nothing to copy
  if (n_units == 0 || b_max == 0 || n_max == 0) return TRIA_OK;

  // out of place only: dense destinations must not overlap any source
  const int hkv = p->n_kv_heads, d = p->head_dim;
  const tria_kv_view* srcs[2] = {k_src, v_src};
  const tria_kv_view* dsts[2] = {k_dst, v_dst};
  for (const tria_kv_view* dv : dsts) {
    if (dv->block_table) continue;
    uintptr_t d0, d1;
    dense_range(dv, n_units, hkv, b_max, d, d0, d1);
    for (const tria_kv_view* sv : srcs) {
      if (sv->block_table) continue;
      uintptr_t s0, s1;
      dense_range(sv, n_units, hkv, n_max, d, s0, s1);
      if (overlaps(d0, d1, s0, s1)) return fail(TRIA_EOVERLAP, "dense destination overlaps a source cache");
    }
  }
  if (!k_dst->block_table && !v_dst->block_table) {
    uintptr_t a0, a1, b0, b1;
    dense_range(k_dst, n_units, hkv, b_max, d, a0, a1);
    dense_range(v_dst, n_units, hkv, b_max, d, b0, b1);
    if (overlaps(a0, a1, b0, b1)) return fail(TRIA_EOVERLAP, "k_dst and v_dst overlap");
  }
  if (pos_src && pos_dst) {
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(pos_src);
    const uintptr_t s1 = s0 + (size_t)n_units * pos_heads * n_max * 4;
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(pos_dst);
    const uintptr_t d1 = d0 + (size_t)n_units * hkv * b_max * 4;
    if (overlaps(s0, s1, d0, d1)) return fail(TRIA_EOVERLAP, "pos_dst overlaps pos_src");
  }
  if (log_on()) {
    auto same_table = [](const tria_kv_view* x, const tria_kv_view* y) {
      return x->block_table == y->block_table &&
             (!x->block_table || (x->block_size == y->block_size && x->max_blocks == y->max_blocks &&
                                  x->n_pool_blocks == y->n_pool_blocks));
    };
    const bool fast = same_table(k_src, v_src) && same_table(k_dst, v_dst);
    tlog("compact: %d units x %d KV heads, n_max %d, b_max %d, %s -> %s: %s (%d rows per workgroup)%s", n_units,
         hkv, n_max, b_max, layout_name(k_src), layout_name(k_dst),
         fast ? "k_compact_fast" : "k_compact (K and V in different layouts: one row at a time)", tria::kCompactRows,
         pos_src && pos_dst ? ", positions" : "");
  }
  if (dry) return TRIA_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t n_rtiles = (b_max + tria::kCompactRows - 1) / tria::kCompactRows;
  tria::CompactArgs ca{kview(k_src), kview(v_src), mkview(k_dst), mkview(v_dst), pos_src, pos_heads, pos_dst,
                       n_units, n_max, b_max, hkv, d, n_rtiles, len, idx, cnt, nullptr};
  hipError_t e = timed(kIdCompact, s, [&] { return tria::launch_compact(ca, s); });
  return launch_status(e, "k_compact");
}

}  // namespace

extern "C" {

tria_status tria_score(const tria_params* p, const tria_kv_view* k, int32_t n_units, int32_t n_max,
                       const int32_t* len, const int32_t* unit_layer, const int32_t* q_pos,
                       const float* q_mean_re, const float* q_mean_im, const float* q_abs_mean, float* raw,
                       float* agg, void* ws, size_t ws_bytes, void* stream) {
  return score_impl(p, k, n_units, n_max, len, unit_layer, q_pos, q_mean_re, q_mean_im, q_abs_mean, raw, agg, ws,
                    ws_bytes, stream, false);
}

tria_status tria_select(const tria_params* p, int32_t n_units, int32_t n_max, int32_t b_max, const int32_t* len,
                        const int32_t* budget, const float* agg, int32_t* idx, int32_t* cnt, void* ws,
                        size_t ws_bytes, void* stream) {
  return select_impl(p, n_units, n_max, b_max, len, budget, agg, idx, cnt, ws, ws_bytes, stream, false);
}

tria_status tria_compact(const tria_params* p, const tria_kv_view* k_src, const tria_kv_view* v_src,
                         const int32_t* pos_src, int32_t pos_heads, int32_t n_units, int32_t n_max, int32_t b_max,
                         const int32_t* len, const int32_t* idx, const int32_t* cnt, const tria_kv_view* k_dst,
                         const tria_kv_view* v_dst, int32_t* pos_dst, void* stream) {
  return compact_impl(p, k_src, v_src, pos_src, pos_heads, n_units, n_max, b_max, len, idx, cnt, k_dst, v_dst,
                      pos_dst, stream, false);
}

size_t tria_calibrate_workspace_size(const tria_params* p, int32_t n_tokens) {
  if (check_params(p) != TRIA_OK || n_tokens < 1) return 0;
  const size_t lh = (size_t)p->n_layers * p->n_kv_heads * p->group;
  const size_t chunks = ((size_t)n_tokens + tria::kCalibChunk - 1) / tria::kCalibChunk;
  return al256(lh * chunks * (size_t)(p->head_dim / 2) * 5 * sizeof(float));
}

tria_status tria_calibrate(const tria_params* p, const void* q, int64_t stride_layer, int64_t stride_head,
                           int64_t stride_token, int32_t n_tokens, float* q_mean_re, float* q_mean_im,
                           float* q_abs_mean, float* r, float* mrl, void* ws, size_t ws_bytes, void* stream) {
  tria_status st = check_params(p);
  if (st != TRIA_OK) return st;
  if (n_tokens < 1) return fail(TRIA_EINVAL, "n_tokens %d < 1", n_tokens);
  if (!q || !q_mean_re || !q_mean_im || !q_abs_mean) return fail(TRIA_EINVAL, "a required device pointer is NULL");
  if (reinterpret_cast<uintptr_t>(q) % 16) return fail(TRIA_ESHAPE, "q not 16-byte aligned");
  if (stride_layer < 0 || stride_head < 0 || stride_token < 0)
    return fail(TRIA_ESHAPE, "q has a negative stride");
  if (stride_layer % 8 || stride_head % 8 || stride_token % 8)
    return fail(TRIA_ESHAPE, "q strides must be multiples of 8 elements");
  const int64_t lh = (int64_t)p->n_layers * p->n_kv_heads * p->group;
  if (lh > 65535) return fail(TRIA_ESHAPE, "n_layers x query heads = %lld exceeds 65535", (long long)lh);
  if (!ws) return fail(TRIA_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(TRIA_EWORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = tria_calibrate_workspace_size(p, n_tokens);
  if (ws_bytes < need) return fail(TRIA_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  const int32_t n_chunks = (n_tokens + tria::kCalibChunk - 1) / tria::kCalibChunk;
  tlog("calibrate: %d layers x %d query heads x %d tokens, d %d, %s: k_calib over %d chunks of %d tokens, "
       "then k_calib_final", p->n_layers, p->n_kv_heads * p->group, n_tokens, p->head_dim, pairing_name(p->pairing),
       n_chunks, tria::kCalibChunk);
  tria::CalibArgs ca{static_cast<const uint16_t*>(q), stride_layer, stride_head, stride_token, p->n_layers,
                     p->n_kv_heads * p->group, p->head_dim, p->pairing, n_tokens, n_chunks,
                     static_cast<float*>(ws), q_mean_re, q_mean_im, q_abs_mean, r, mrl};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(kIdCalib, s, [&] { return tria::launch_calibrate(ca, s); });
  return launch_status(e, "k_calib");
}

tria_status tria_compact_inplace(const tria_params* p, const tria_kv_view* k, const tria_kv_view* v, int32_t* pos,
                                 int32_t n_units, int32_t n_max, int32_t b_max, int32_t* len,
                                 const int32_t* idx, const int32_t* cnt, void* ws, void* stream) {
  tria_status st = check_params(p);
  if (st != TRIA_OK) return st;
  if (n_units < 0 || n_max < 0 || b_max < 0) return fail(TRIA_EINVAL, "n_units, n_max and b_max must be >= 0");
  if ((st = check_view(k, "k", p->head_dim, n_max)) != TRIA_OK) return st;
  if ((st = check_view(v, "v", p->head_dim, n_max)) != TRIA_OK) return st;
  if (!len || !idx || !cnt) return fail(TRIA_EINVAL, "a required device pointer is NULL");
  if (!ws) return fail(TRIA_EWORKSPACE, "workspace is NULL (its flag word records contract violations)");
  if (n_units == 0 || b_max == 0 || n_max == 0) return TRIA_OK;
  if (!k->block_table && !v->block_table) {
    uintptr_t a0, a1, b0, b1;
    dense_range(k, n_units, p->n_kv_heads, n_max, p->head_dim, a0, a1);
    dense_range(v, n_units, p->n_kv_heads, n_max, p->head_dim, b0, b1);
    if (overlaps(a0, a1, b0, b1)) return fail(TRIA_EOVERLAP, "k and v overlap");
  }
  tlog("compact_inplace: %d units x %d KV heads, n_max %d, b_max %d, %s: k_compact_inplace, then len <- cnt",
       n_units, p->n_kv_heads, n_max, b_max, layout_name(k));
  tria::InplaceArgs ia{mkview(k), mkview(v), pos, n_units, n_max, b_max, p->n_kv_heads, p->head_dim,
                       len, idx, cnt, static_cast<int32_t*>(ws)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed(kIdCompact, s, [&] { return tria::launch_compact_inplace(ia, s); });
  return launch_status(e, "k_compact_inplace");
}

tria_status tria_append(const tria_params* p, const tria_kv_view* k, const tria_kv_view* v, int32_t* pos,
                        int32_t n_units, int32_t n_max, int32_t* len, int32_t* q_pos, int32_t t_new,
                        const void* k_new, const void* v_new, const int32_t* pos_new, void* ws, void* stream) {
  tria_status st = check_params(p);
  if (st != TRIA_OK) return st;
  if (n_units < 0 || n_max < 0 || t_new < 0) return fail(TRIA_EINVAL, "n_units, n_max and t_new must be >= 0");
  if ((st = check_view(k, "k", p->head_dim, n_max)) != TRIA_OK) return st;
  if ((st = check_view(v, "v", p->head_dim, n_max)) != TRIA_OK) return st;
  if (!len || !k_new || !v_new) return fail(TRIA_EINVAL, "a required device pointer is NULL");
  if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16)
    return fail(TRIA_ESHAPE, "k_new and v_new must be 16-byte aligned");
  if (!ws) return fail(TRIA_EWORKSPACE, "workspace is NULL (its flag word records contract violations)");
  if (n_units == 0 || t_new == 0) return TRIA_OK;
  tlog("append: %d units x %d KV heads, %d new rows each, n_max %d, %s: k_append%s", n_units, p->n_kv_heads,
       t_new, n_max, layout_name(k), q_pos ? ", then len += t_new and q_pos <- the newest position" : ", then len += t_new");
  tria::AppendArgs aa{mkview(k), mkview(v), pos, n_units, n_max, p->n_kv_heads, p->head_dim, t_new, len, q_pos,
                      static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), pos_new,
                      static_cast<int32_t*>(ws)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_status(tria::launch_append(aa, s), "k_append");
}

tria_status tria_pass_noalloc(const tria_params* p, const tria_kv_view* k, const tria_kv_view* v, int32_t n_units,
                              int32_t n_max, int32_t b_max, const int32_t* len, const int32_t* unit_layer,
                              const int32_t* q_pos, const int32_t* budget, const float* q_mean_re,
                              const float* q_mean_im, const float* q_abs_mean, const int32_t* pos_src,
                              int32_t pos_heads, float* agg, int32_t* idx, int32_t* cnt, const tria_kv_view* k_dst,
                              const tria_kv_view* v_dst, int32_t* pos_dst, int32_t* flags, void* stream) {
  tria_status st = check_params(p);
  if (st != TRIA_OK) return st;
  if (n_units < 0 || n_max < 0 || b_max < 0) return fail(TRIA_EINVAL, "n_units, n_max and b_max must be >= 0");
  const size_t need = layout(p, n_units, n_max).total;
  if (need > tria::kScratchBytes)
    return fail(TRIA_EWORKSPACE, "the pass needs %zu bytes of workspace; the library's scratch holds %zu", need,
                tria::kScratchBytes);
  hipError_t e = hipSuccess;
  void* ws = tria::scratch_address(&e);
  if (!ws) return fail(TRIA_ELAUNCH, "scratch address: %s", hipGetErrorString(e));
  const size_t wsb = tria::kScratchBytes;
  tlog("pass_noalloc: workspace %zu of the %zu B static scratch at %p", need, wsb, ws);
  // every step's checks before anything is launched
  if ((st = score_impl(p, k, n_units, n_max, len, unit_layer, q_pos, q_mean_re, q_mean_im, q_abs_mean, nullptr, agg,
                       ws, wsb, stream, true)) != TRIA_OK ||
      (st = select_impl(p, n_units, n_max, b_max, len, budget, agg, idx, cnt, ws, wsb, stream, true)) != TRIA_OK ||
      (st = compact_impl(p, k, v, pos_src, pos_heads, n_units, n_max, b_max, len, idx, cnt, k_dst, v_dst, pos_dst,
                         stream, true)) != TRIA_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  struct NoEvents {
    NoEvents() { t_no_events = true; }
    ~NoEvents() { t_no_events = false; }
  } no_events;
  // the flag word starts at zero for every call (the scratch keeps the last call's contents)
  if ((st = launch_status(tria::launch_set_word(static_cast<int32_t*>(ws), 0, s), "flag word")) != TRIA_OK) return st;
  if ((st = score_impl(p, k, n_units, n_max, len, unit_layer, q_pos, q_mean_re, q_mean_im, q_abs_mean, nullptr, agg,
                       ws, wsb, stream, false)) != TRIA_OK ||
      (st = select_impl(p, n_units, n_max, b_max, len, budget, agg, idx, cnt, ws, wsb, stream, false)) != TRIA_OK ||
      (st = compact_impl(p, k, v, pos_src, pos_heads, n_units, n_max, b_max, len, idx, cnt, k_dst, v_dst, pos_dst,
                         stream, false)) != TRIA_OK)
    return st;
  if (flags) st = launch_status(tria::launch_copy_word(flags, static_cast<const int32_t*>(ws), s), "flag word");
  return st;
}

tria_status tria_device_flags(void* ws, int32_t* flags, void* stream) {
  if (!ws || !flags) return fail(TRIA_EINVAL, "ws and flags must be non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ws, sizeof v, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemsetAsync(ws, 0, sizeof v, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(TRIA_ELAUNCH, "tria_device_flags: %s", hipGetErrorString(e));
  *flags = v;
  return TRIA_OK;
}

const char* tria_strerror(tria_status s) {
  switch (s) {
    case TRIA_OK: return "ok";
    case TRIA_EINVAL: return "invalid argument";
    case TRIA_ESHAPE: return "unsupported or inconsistent shape";
    case TRIA_EBUDGET: return "budget below the protected slots";
    case TRIA_EOVERLAP: return "destination overlaps source";
    case TRIA_EWORKSPACE: return "workspace missing or too small";
    case TRIA_ELAUNCH: return "HIP launch failed";
  }
  return "unknown status";
}

const char* tria_last_error(void) { return g_err; }

int32_t tria_select_strategy(int32_t strategy) {
  if (strategy != TRIA_SELECT_PER_GROUP && strategy != TRIA_SELECT_TILED) strategy = TRIA_SELECT_AUTO;
  return g_select_strategy.exchange(strategy);
}

int32_t tria_score_max_workgroups(int32_t cap) {
  return g_score_wg_cap.exchange(cap < 0 ? 0 : cap);
}

int32_t tria_score_wait_polls(int32_t polls) {
  return g_wait_polls.exchange(polls < 0 ? -1 : polls);
}

int32_t tria_log(int32_t on) {
  const int prev = log_on() ? 1 : 0;
  if (on >= 0) g_log.store(on > 0 ? 1 : 0);
  return prev;
}

int32_t tria_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = on != 0;
  return kNumIds;
}

int32_t tria_timing_read(double* ms_sum, int64_t* launches, int32_t n) {
  std::vector<Rec> recs;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    recs.swap(g_recs);
  }
  for (int i = 0; i < n && i < kNumIds; ++i) {
    if (ms_sum) ms_sum[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (const Rec& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess && r.id < n) {
      if (ms_sum) ms_sum[r.id] += ms;
      if (launches) launches[r.id] += 1;
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  return kNumIds;
}

const char* tria_kernel_name(int32_t k) { return (k >= 0 && k < kNumIds) ? kNames[k] : ""; }

}  // extern "C"
