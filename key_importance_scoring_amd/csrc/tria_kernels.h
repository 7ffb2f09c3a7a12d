// Internal interface between the C ABI (tria_abi.cpp) and the gfx950 kernels
// (tria_kernels.hip).  Not installed; the public interface is include/tria.h.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tria {

constexpr int kMaxOffsets = 256;
constexpr int kMaxGroup = 8;
// Up to this many units, the score kernel claims only tiles that hold keys (every
// workgroup keeps all lengths and a prefix of the units' tiles in LDS).
constexpr int kListUnits = 512;
constexpr int kScoreTileMax = 2048;
// keys per score tile: two tiles of scores ([G][tile + 16] fp32 each) live in LDS
#ifndef TRIA_SCORE_TILE_LARGE_G
#define TRIA_SCORE_TILE_LARGE_G 1024
#endif
#ifndef TRIA_SCORE_TILE_SMALL_G
#define TRIA_SCORE_TILE_SMALL_G 2048
#endif
// (the maximum over offsets stages its coefficient blocks beside the tiles: 1024)
// Keys per score tile for rows of n_max slots: the fewest tiles the cap allows
// (2048 keys for G <= 4 with the mean over offsets, else 1024: the tiles' scores
// live in LDS), balanced in multiples of 256 (each wave takes a quarter of a tile
// in 64-key stages), so that a row just past a multiple of the cap is not followed
// by a nearly empty tile.
inline int balanced_tile_keys(int cap, int n_max) {
  if (n_max <= cap) return cap;
  const int nt = (n_max + cap - 1) / cap;
  const int t = ((n_max + nt - 1) / nt + 255) / 256 * 256;
  return t < cap ? t : cap;
}
inline int score_tile_keys(int group, int omax, int n_max) {
  return balanced_tile_keys(group <= 4 && !omax ? TRIA_SCORE_TILE_SMALL_G : TRIA_SCORE_TILE_LARGE_G, n_max);
}
// With one score buffer a workgroup (dense caches, the mean over offsets, G > 4) takes tiles of
// this many keys; tria_score picks that mode when every tile of the call fits on
// the device at once.  The workspace is sized for score_tile_keys' smaller tiles,
// whose tile count bounds this one's.
inline int single_tile_keys(int n_max) { return balanced_tile_keys(TRIA_SCORE_TILE_SMALL_G, n_max); }
// A tile's published moments start as this bit pattern (cleared by k_coef): a NaN
// whose low payload bits are set, which no moment computed from fp32 scores can
// take (NaNs that arithmetic produces keep an fp32 payload or are the default one).
constexpr uint64_t kUnpublished = ~0ull;
// Bounded wait for a group's tile moments: each poll is one memory round trip plus a
// short sleep (~0.1-0.2 s in all); when it runs out the group's moments are computed
// directly from the K cache.
constexpr int kPollLimit = 1 << 16;
// Linear bins of an aggregate (a z-score: scale-free): kBinScale bins per unit over
// [-8, 8), one below, one above, one for +inf (protected slots), one spare.
#ifndef TRIA_BIN_SCALE
#define TRIA_BIN_SCALE 64
#endif
constexpr int kBinScale = TRIA_BIN_SCALE;
constexpr int kBins = 16 * kBinScale + 4;

// Coefficient blocks of the maximum-over-offsets mode (16 MFMA B columns each:
// hi parts in columns 0..7, lo parts in 8..15).  With G' = G rounded up to a power
// of two, a block holds opb = 8 / G' offsets: column q G' + h is query head h at the
// block's q-th offset (offsets in order, the last block padded by repeating the
// last offset, which leaves the maximum unchanged; columns of heads >= G are zero).
struct OffsetBlocks {
  int gp;       // G': column stride of one offset
  int opb;      // offsets per block
  int nblk;     // blocks per (unit, KV head)
};
__host__ __device__ inline OffsetBlocks offset_blocks(int n_offsets, int group) {
  OffsetBlocks ob;
  ob.gp = group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : 8;
  ob.opb = 8 / ob.gp;
  ob.nblk = (n_offsets + ob.opb - 1) / ob.opb;
  return ob;
}

// A cache view with element strides (bf16 elements).
struct KView {
  const uint16_t* base;
  int64_t su, sh, ss;
  const int32_t* bt;   // nullptr: dense
  int32_t bs, mb;
  int64_t npb;
};

struct MutKView {
  uint16_t* base;
  int64_t su, sh, ss;
  const int32_t* bt;
  int32_t bs, mb;
  int64_t npb;
};

struct Offsets {
  double v[kMaxOffsets];
  int32_t n;
};

// Sample slots per (unit, KV head) whose mean band magnitudes are the norm term's
// reference magnitudes (spread evenly over the unit's keys).
constexpr int kRefRows = 16;
static_assert(kRefRows % 8 == 0, "k_coef spreads the sample rows evenly over the 256 / F (at most 8) threads of a band");

struct CoefArgs {
  KView k;                    // the K cache: sample rows for the reference magnitudes
  int32_t n_units, hq, hkv, d, layers, pairing;
  double log_base;            // ln(theta)
  const int32_t* len;
  const int32_t* unit_layer;
  const int32_t* q_pos;
  const float* q_re;
  const float* q_im;
  const float* q_abs;
  int32_t group, n_tiles, tile;  // query heads per KV head; score tiles per (unit, KV head), keys per tile
  int32_t n_max;
  uint32_t* B;                // [U][Hkv][d/16 + d/64][64] 16-byte MFMA B operands and reference magnitudes
  float* nconst;              // [U][Hq] the norm term's shift sum_f n_f r_f per query head
  uint64_t* part;             // [U][Hq][n_tiles][3] tile moments of k_score, set to kUnpublished here
  int32_t* next_tile;         // tile claim counter of k_score, cleared here
  uint32_t* hist;             // [U][Hkv][kBins] aggregate histograms of k_score, cleared here
  int32_t* flags;
  int32_t omax;               // 1: maximum over the offsets
  uint32_t* Bmax;             // omax: [U][Hkv][nblk][d/32][64] 16-byte B operands of the offset blocks
  OffsetBlocks ob;
  uint64_t* gstat;            // [U][Hq] each query head's merged (mean, 1 / deviation), set to kUnpublished here
  int32_t* arrive;            // [U][Hkv] scored tiles counted in, cleared here
};

struct ScoreArgs {
  KView k;
  int32_t n_units, n_max, hkv, group, sink, window, tile, n_tiles, agg_mode;
  const int32_t* len;
  const uint32_t* B;          // [U][Hkv][d/16 + d/64][64] 16-byte MFMA B operands and reference magnitudes
  const float* nconst;        // [U][Hq] the norm term's shift, added back to per-query-head scores
  float* raw;                 // [U][Hq][n_max], may be null
  double* part;               // [U][Hq][n_tiles][3] tile moments (count, mean, sum of squared deviations)
  float* agg;                 // [U][Hkv][n_max]
  int32_t* next_tile;         // next tile to claim
  uint32_t* hist;             // [U][Hkv][kBins] histogram of the aggregates' linear bins
  int32_t* flags;
  int32_t omax;               // 1: maximum over the offsets (B operands of the norm part still in B)
  const uint32_t* Bmax;       // omax: [U][Hkv][nblk][d/32][64] 16-byte B operands of the offset blocks
  OffsetBlocks ob;
  int32_t wait_polls;         // polls of a finalisation's wait (< 0: compute the moments directly at once)
  uint64_t* gstat;            // [U][Hq] merged (mean, 1 / deviation) per query head: two fp32 in one word
  int32_t* arrive;            // [U][Hkv] non-empty tiles that have published their moments
  int32_t single;             // 1: k_score_single (one LDS score buffer, each tile finalised as soon as it is scored)
};

// Per-(unit, KV head) state of the selection, in the workspace.
struct SelState {
  int32_t b1;    // linear bin holding the K-th largest aggregate (-1: keep all; kBins: keep none)
  int32_t krem;  // slots still to take from bin b1
  int32_t K;     // slots kept
  int32_t n;     // cached slots
  int32_t m;     // candidates (slots of bin b1)
  int32_t T;     // threshold order key
  int32_t keq;   // slots equal to T that are kept
  int32_t pad;
};

#ifndef TRIA_SEL_TILE
#define TRIA_SEL_TILE 2048
#endif
constexpr int kSelTile = TRIA_SEL_TILE; // slots per selection tile (kSelTile / 256 per thread)
constexpr int kSelGroupMax = 32768;     // per-group selection: 512 threads x 64 slots in registers
constexpr int kRefineLds = 3072;        // candidates the refinement keeps in LDS
#ifndef TRIA_SEL_RANK_MAX
#define TRIA_SEL_RANK_MAX 256
#endif
constexpr int kSelRankMax = TRIA_SEL_RANK_MAX;   // up to this many candidates: ranks instead of radix passes
static_assert(kSelRankMax <= 512, "one candidate per thread of the 512-thread refinement");
constexpr int kMaxSelTiles = 2048;      // per (unit, KV head): n_max <= 2048 kSelTile

// A selection tile's per-thread bit masks: bit k stands for slot s0 + k of the
// thread's kSelTile / 256 consecutive slots.
using SelMask = std::conditional<(kSelTile / 256 <= 8), uint8_t,
                                 std::conditional<(kSelTile / 256 <= 16), uint16_t, uint32_t>::type>::type;

struct SelectArgs {
  int32_t n_units, n_max, b_max, hkv, sink, window, n_st;
  const int32_t* len;
  const int32_t* budget;
  const float* agg;
  const uint32_t* hist;       // [U][Hkv][kBins] binned aggregates, from k_score
  SelState* st;               // [U][Hkv]
  int32_t* tile_gt;           // [U][Hkv][n_st] slots above b1 per tile
  int32_t* tile_off;          // [U][Hkv][n_st] output offset per tile
  int32_t* tile_m;            // [U][Hkv][n_st] candidates (slots of bin b1) per tile
  int32_t* list;              // [U][Hkv][n_max] candidate slots, tile j's from j * kSelTile
  SelMask* gmask;             // [U][Hkv][n_st][256] per thread: slots above b1
  SelMask* cmask;             // [U][Hkv][n_st][256] per thread: slots of bin b1 (candidates); k_sel_refine
                              // then clears the bits of the candidates it drops
  int32_t* idx;               // [U][Hkv][b_max]
  int32_t* cnt;               // [U]
  int32_t* flags;
};

constexpr int kCalibChunk = 1024;       // query rows per calibration workgroup

struct CalibArgs {
  const uint16_t* q;
  int64_t sl, sh, st;         // element strides: layer, query head, token
  int32_t n_layers, hq, d, pairing, n_tokens, n_chunks;
  float* part;                // [L][Hq][n_chunks][d/2][5] fp32 chunk sums (chunks of kCalibChunk rows)
  float* mean_re;
  float* mean_im;
  float* abs_mean;
  float* r;                   // may be null
  float* mrl;                 // may be null
};

struct CompactArgs {
  KView ks, vs;
  MutKView kd, vd;
  const int32_t* pos_src;
  int32_t pos_heads;
  int32_t* pos_dst;
  int32_t n_units, n_max, b_max, hkv, d, n_rtiles;
  const int32_t* len;
  const int32_t* idx;
  const int32_t* cnt;
  int32_t* flags;             // may be null
};

#ifndef TRIA_COMPACT_ROWS
#define TRIA_COMPACT_ROWS 64
#endif
constexpr int kCompactRows = TRIA_COMPACT_ROWS;   // kept rows per compaction workgroup

hipError_t launch_coef(const CoefArgs& a, const Offsets& offs, hipStream_t s);
hipError_t launch_score(const ScoreArgs& a, int d, int pairing, int max_wg, hipStream_t s);
// Workgroups of k_score that fit on the device at once (-1 on error).  Every tile
// of one (unit, KV head) must be resident together for the moment exchange.
int score_capacity(int d, int pairing, bool paged, int group, int omax, int nblk, int tile, int block_size,
                   int single);
// LDS bytes of one k_score workgroup for tiles of `tile` keys (block_size: of a paged cache)
size_t score_lds(int d, int group, bool paged, int omax, int nblk, int tile, int block_size, int single);
// strategy: 0 automatic, 1 per group (when n_max fits), 2 tiled
hipError_t launch_select(const SelectArgs& a, int strategy, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);
hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s);

// In-place compaction (the decode loop): row j <- row idx[j], j < cnt[u], in the
// cache it reads from.
constexpr int kInplaceRows = 128;       // rows per chunk (one workgroup per (unit, KV head) walks them in order)
struct InplaceArgs {
  MutKView k, v;
  int32_t* pos;               // [U][Hkv][n_max] per-head positions, or null
  int32_t n_units, n_max, b_max, hkv, d;
  int32_t* len;               // read by the move, then set to the kept count
  const int32_t* idx;         // [U][Hkv][b_max]
  const int32_t* cnt;
  int32_t* flags;
};
hipError_t launch_compact_inplace(const InplaceArgs& a, hipStream_t s);

// Appends t_new rows per (unit, KV head) at slots len[u] .. len[u] + t_new - 1.
struct AppendArgs {
  MutKView k, v;
  int32_t* pos;               // [U][Hkv][n_max] or null
  int32_t n_units, n_max, hkv, d, t_new;
  int32_t* len;               // read by the append, then advanced by t_new
  int32_t* q_pos;             // [U] or null: set to the newest appended position
  const uint16_t* k_new;      // [U][Hkv][t_new][d]
  const uint16_t* v_new;      // [U][Hkv][t_new][d]
  const int32_t* pos_new;     // [U][t_new] or null
  int32_t* flags;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

// The no-allocation pass's workspace: a file-scope device array of this many bytes
// in tria_kernels.hip (every benchmark workload's workspace fits; the largest, 64
// layers x 8 KV heads x 32768 slots, needs 80 MiB).
constexpr size_t kScratchBytes = size_t(96) << 20;
// Its device address on the current device (looked up once per device), or null
// with *err set.
void* scratch_address(hipError_t* err);
// One-thread kernels: *dst = v, *dst = *src (flag word handling without memset or copies).
hipError_t launch_set_word(int32_t* dst, int32_t v, hipStream_t s);
hipError_t launch_copy_word(int32_t* dst, const int32_t* src, hipStream_t s);

}  // namespace tria
