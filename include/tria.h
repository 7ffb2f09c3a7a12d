/*
 * tria.h - C ABI of the TriAttention KV-cache pruning pass on MI355X (gfx950).
 *
 * One pruning event is three calls on one HIP stream:
 *
 *   tria_score   : score every cached key of every (unit, KV head) with the
 *                  offset-averaged TriAttention score, z-normalise it per query
 *                  head over the droppable slots and aggregate each GQA group
 *                  onto its KV head;
 *   tria_select  : keep the top-B slots per (unit, KV head), sinks and the
 *                  recent window always included;
 *   tria_compact : gather the kept K rows, V rows and positions into the
 *                  destination cache.
 *
 * A "unit" is one (layer, sequence) pair; units are independent.  Sources of
 * the arithmetic (cited by page title and equation):
 *   - Fold note: academ.us article 2607.13051 (restates the TriAttention score,
 *     Eqs. 1-3, and folds its future-offset average, Eqs. 4-8);
 *   - Blog: "TriAttention, or: what a rotating query already knows" (The Method);
 *   - Calib issue: GitHub issue "Request: publish TriAttention calibration
 *     script (TRIA v2/v3 stats.bin producer)" (pairing conventions, statistics
 *     layout, the port's runtime parameters budget / window / sink).
 *
 * Conventions shared by every entry point:
 *   - Pointers marked [device] are device memory owned by the caller; the
 *     library keeps no pointer after a call returns.  Pointers marked [host]
 *     are read during the call only.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream).  No entry point synchronises, allocates device memory or copies
 *     between host and device, except tria_device_flags and the timing calls.
 *   - Every argument the host can see is validated before anything is
 *     enqueued: a non-OK status means nothing was launched.  Values that live
 *     in device memory (lengths, layers, budgets, block ids) cannot be checked
 *     on the host; the kernels clamp them to safe ranges (no access ever leaves
 *     the caller's buffers) and record the violation in the workspace's flag
 *     word, which tria_device_flags reads.
 *   - Keys and values are bf16 rows of head_dim elements, each row contiguous
 *     and 16-byte aligned.
 *   - Entry points are reentrant; calls that share a workspace must not overlap
 *     in time (use one stream, or one workspace per stream).
 */
#ifndef TRIA_H_
#define TRIA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tria_status {
  TRIA_OK = 0,
  TRIA_EINVAL = 1,      /* null pointer, unknown enum value, negative count   */
  TRIA_ESHAPE = 2,      /* unsupported head_dim / group, inconsistent sizes,
                           strides or alignment                                */
  TRIA_EBUDGET = 3,     /* (device flag) a budget below sink + window while
                           the unit holds more than `budget` keys              */
  TRIA_EOVERLAP = 4,    /* dense destination range overlaps the source range  */
  TRIA_EWORKSPACE = 5,  /* workspace missing or smaller than tria_workspace_size */
  TRIA_ELAUNCH = 6      /* a HIP call failed; tria_last_error() has the detail */
} tria_status;

/* Band pairing of a head's dims into complex numbers [Calib issue]:
 *   NEOX        : band f = dim f + i * dim (f + d/2)
 *   INTERLEAVED : band f = dim 2f + i * dim (2f + 1)                          */
typedef enum { TRIA_PAIR_NEOX = 0, TRIA_PAIR_INTERLEAVED = 1 } tria_pairing;

/* GQA aggregation of a group's z-scores onto its KV head [Fold note, sec. 4:
 * "normalize-then-max"; the mean is the other variant].                        */
typedef enum { TRIA_AGG_MEAN = 0, TRIA_AGG_MAX = 1 } tria_agg;

/* How the score reduces over the future offsets D: the mean (the method,
 * [Fold note, Eq. 4], folded exactly into one weight per band, Eqs. 5-7) or the
 * maximum (the non-default variant [Fold note, sec. 4]; no fold applies, each
 * offset is scored on its own and the largest taken).                         */
typedef enum { TRIA_OFFSETS_MEAN = 0, TRIA_OFFSETS_MAX = 1 } tria_offset_reduce;

/* Device-side contract violations, OR-ed into the workspace flag word.        */
enum {
  TRIA_FLAG_LEN = 1,     /* len[u] < 0 or > n_max: clamped                     */
  TRIA_FLAG_LAYER = 2,   /* unit_layer[u] outside [0, n_layers): unit skipped  */
  TRIA_FLAG_BUDGET = 4,  /* budget[u] < 0, or < min(len, sink + window) while
                            len > budget: the top-B rule is still applied     */
  TRIA_FLAG_BLOCK = 8,   /* block id outside [0, n_pool_blocks): row skipped   */
  TRIA_FLAG_INDEX = 16,  /* compaction index outside [0, len[u]): row skipped  */
  TRIA_FLAG_BMAX = 32,   /* min(budget, len) > b_max: clamped to b_max         */
  TRIA_FLAG_SYNC = 64    /* tria_score, information only: a group's tiles did
                            not all publish their moments within the bounded
                            wait (or tria_score_wait_polls asked for no wait),
                            and a workgroup computed that group's moments
                            directly from the K cache; results remain valid  */
};

/* Shape and method parameters (a host struct, read during the call only). */
typedef struct tria_params {
  int32_t head_dim;        /* d: 64, 128 or 256                                 */
  int32_t n_kv_heads;      /* Hkv >= 1                                          */
  int32_t group;           /* G = query heads per KV head, 1..8; query head h
                              belongs to KV head h / G                          */
  int32_t n_layers;        /* L: leading extent of the statistics arrays        */
  int32_t pairing;         /* tria_pairing                                      */
  int32_t agg;             /* tria_agg                                          */
  double rope_base;        /* theta > 1: band f turns at theta^(-2f/d) rad per
                              position [Fold note, Eq. 2]                       */
  const int64_t* offsets;  /* [host] future offsets D, each in [0, 2^40]; the
                              score is reduced over them (offset_reduce)        */
  int32_t n_offsets;       /* |D|, 1..256                                       */
  int32_t sink;            /* S0 >= 0: the first S0 slots are always kept       */
  int32_t window;          /* W >= 0: the last W slots are always kept          */
  int32_t offset_reduce;   /* tria_offset_reduce; 0 (the mean) for a struct
                              that is zero-initialised                          */
} tria_params;

/* A K or V cache.  Row of (unit u, KV head g, slot i) starts at element
 *   dense : base + u*stride_unit + g*stride_head + i*stride_slot
 *   paged : base + (bt[u*max_blocks + i/block_size]*block_size + i%block_size)
 *                  * stride_slot + g*stride_head
 * (strides in bf16 elements, each a multiple of 8; base 16-byte aligned).
 * tria_score and tria_compact may read (and ignore) rows of slots in
 * [len[u], n_max): a dense source view must be readable for every slot below
 * n_max, and a paged view's table must cover n_max slots (its ids past len[u] may
 * be anything, -1 included).  */
typedef struct tria_kv_view {
  void* base;                 /* [device] bf16 rows                             */
  int64_t stride_unit;        /* dense only                                     */
  int64_t stride_head;
  int64_t stride_slot;
  const int32_t* block_table; /* [device] [n_units][max_blocks]; NULL = dense   */
  int32_t block_size;         /* paged: slots per block (>= 1)                  */
  int32_t max_blocks;         /* paged: row length of block_table               */
  int64_t n_pool_blocks;      /* paged: blocks in the pool; ids are checked
                                 against it on the device                       */
} tria_kv_view;

/* Bytes of workspace tria_score and tria_select need for `n_units` units of at
 * most `n_max` slots.  The first 256 bytes hold the device flag word: zero them
 * once before first use (tria_device_flags clears them on every read).  Returns 0
 * for invalid parameters. */
size_t tria_workspace_size(const tria_params* p, int32_t n_units, int32_t n_max);

/* tria_score - the offset-averaged TriAttention score, z-normalised and
 * aggregated onto each KV head.
 *
 * For unit u (layer l = unit_layer[u], n = len[u] cached slots), KV head g and
 * query head h of g's group, with centre mu_f = q_mean_re + i q_mean_im and
 * mean magnitude a_f = q_abs_mean of (l, h, f), and key bands k_f read in the
 * pairing layout and un-rotated at their positions:
 *   raw[u][h][i] = (1/|D|) sum_{delta in D} sum_f |mu_f||k_f|
 *                    cos(omega_f (q_pos[u] - p_i + delta) + arg mu_f - arg k_f)
 *                + sum_f (a_f - |mu_f|) |k_f|
 * [Fold note, Eqs. 1, 2, 4; the norm term is the reading E|q_f| (1 - R_f) |k_f|
 * of Blog, The Method].  The kernels evaluate it in the folded form of Eq. 7
 * with the inverse rotation absorbed by angle addition, so key positions are
 * not needed: only q_pos.  With p->offset_reduce = TRIA_OFFSETS_MAX the mean
 * over D is replaced by the maximum over D [Fold note, sec. 4]: each offset's
 * band sum is one dot product of the key row with the coefficients
 * mu_f e^{i omega_f (q_pos + delta)}, evaluated for every delta.  That mode
 * stages every offset's coefficients in LDS and returns TRIA_ESHAPE when they
 * do not fit (ceil(|D| G' / 8) * d / 32 KiB, G' = G rounded up to a power of two,
 * beside the score tiles; 17 offsets fit for every head_dim and group except
 * d = 256 with G > 4).
 * Then, over the droppable slots C = [sink, n - window) (the candidates):
 *   z_h(i)     = (raw[u][h][i] - mean_C) / max(std_C, 1e-12)   (population std)
 *   agg[u][g][i] = mean_h z_h(i)  or  max_h z_h(i)   (per p->agg)
 * and agg = +inf on the protected slots [0, sink) and [n - window, n).
 *
 *   k           [device] K cache view (dense or paged)
 *   n_units     U >= 0; n_max >= every len[u] (row length of raw and agg)
 *   len         [device] int32 [U] cached slots per unit
 *   unit_layer  [device] int32 [U] layer of each unit (row of the statistics)
 *   q_pos       [device] int32 [U] position of the current query (the newest
 *               key); future queries sit at q_pos + delta
 *   q_mean_re, q_mean_im, q_abs_mean
 *               [device] fp32 [L][G*Hkv][d/2] calibrated query statistics
 *               E[Re q_f], E[Im q_f], E|q_f| [Calib issue]
 *   raw         [device] fp32 [U][G*Hkv][n_max] per-query-head scores, or NULL
 *               when they are not wanted (the pass never needs them: the
 *               aggregation is fused into the score kernel)
 *   agg         [device] fp32 [U][Hkv][n_max] aggregated scores; slots >= len[u]
 *               are left untouched
 *   ws          [device] workspace of ws_bytes >= tria_workspace_size(...)
 * Execution: the keys of each (unit, KV head) are scored in tiles of up to 2048
 * (1024 for G > 4 or the maximum over offsets, except for a dense cache with the
 * mean over offsets whose 2048-key tiles all fit on the device at once; balanced
 * in multiples of 256 when n_max is larger, e.g. 1280 + 896 for 2176) by
 * concurrent workgroups that publish their tile moments through the workspace;
 * the group's last tile to publish merges them once and publishes each query
 * head's mean and deviation, which the others wait for (boundedly) before
 * normalising.  When a wait runs out
 * (another stream's kernels holding compute units, say), the waiting workgroup
 * scores the group's keys again and forms its moments itself, and TRIA_FLAG_SYNC
 * records that this slower path ran: the results never depend on the tiles'
 * workgroups being resident together.
 */
tria_status tria_score(const tria_params* p, const tria_kv_view* k, int32_t n_units, int32_t n_max,
                       const int32_t* len, const int32_t* unit_layer, const int32_t* q_pos,
                       const float* q_mean_re, const float* q_mean_im, const float* q_abs_mean,
                       float* raw, float* agg, void* ws, size_t ws_bytes, void* stream);

/* tria_select - keep the top-B slots of each (unit, KV head)
 * ("Sort. Keep the top-B. Drop the rest." [Blog, The Method]).
 *
 * Runs after tria_score on the same stream, with the same workspace, parameters,
 * n_units and n_max, and on the agg it produced: tria_score leaves a histogram of
 * the aggregates in the workspace and the selection starts from it.
 *
 * Keeps K_u = min(budget[u], len[u]) slots per (u, g): the slots with the
 * largest agg (protected slots carry +inf, so they are kept whenever
 * budget >= sink + window); among equal agg the lower slot wins.
 *   idx  [device] int32 [U][Hkv][b_max]: kept slots in ascending order in
 *        [0, K_u), -1 in [K_u, b_max)
 *   cnt  [device] int32 [U]: K_u
 * b_max must be >= every K_u (else TRIA_FLAG_BMAX and the keep count is
 * clamped to b_max).
 */
tria_status tria_select(const tria_params* p, int32_t n_units, int32_t n_max, int32_t b_max,
                        const int32_t* len, const int32_t* budget, const float* agg,
                        int32_t* idx, int32_t* cnt, void* ws, size_t ws_bytes, void* stream);

/* tria_compact - gather the kept rows (a bit copy; no conversion).
 *
 * For every unit u, KV head g and j < cnt[u], with i = idx[u][g][j]:
 *   row (u, g, j) of k_dst = row (u, g, i) of k_src;   likewise V;
 *   pos_dst[u][g][j]       = pos_src[u][g or 0][i].
 * k_dst / v_dst address kept slot j like a cache of b_max slots (dense) or
 * through their own block tables (paged).  Out of place only: dense
 * destinations overlapping the source return TRIA_EOVERLAP; for paged views,
 * disjoint source and destination blocks are a precondition.
 *   pos_src   [device] int32 [U][pos_heads][n_max] or NULL (then pos_dst is
 *             ignored); pos_heads is 1 (shared by all KV heads) or Hkv
 *   pos_dst   [device] int32 [U][Hkv][b_max] or NULL
 *   len       [device] int32 [U] (indices are checked against it)
 */
tria_status tria_compact(const tria_params* p, const tria_kv_view* k_src, const tria_kv_view* v_src,
                         const int32_t* pos_src, int32_t pos_heads, int32_t n_units, int32_t n_max,
                         int32_t b_max, const int32_t* len, const int32_t* idx, const int32_t* cnt,
                         const tria_kv_view* k_dst, const tria_kv_view* v_dst, int32_t* pos_dst,
                         void* stream);

/* tria_compact_inplace - tria_compact into the cache it reads from, for a decode
 * loop that prunes a sequence every so many generated tokens and keeps its blocks
 * [Calib issue: the port scores every 128 tokens, interval=128; README mirror:
 * the KV budget].  For unit u, KV head g and j < cnt[u]:
 *   K row (u, g, j) <- K row (u, g, idx[u][g][j]);  V likewise;
 *   pos[u][g][j] <- pos[u][g][idx[u][g][j]]   (when pos is not NULL)
 * with idx as tria_select writes it: ascending, so idx[j] >= j.  Rows with
 * idx[j] == j are not touched; slots >= cnt[u] keep whatever they held.  Then
 * len[u] <- the unit's kept count, min(cnt[u], b_max, len[u]) (negative values
 * count as 0), so that the next append lands right after the kept rows.
 *   k, v        [device] cache views (dense or paged; the same layouts as
 *               tria_compact's sources), read and written
 *   pos         [device] int32 [U][Hkv][n_max] per-head positions, or NULL
 *   len         [device] int32 [U], read, then overwritten with the kept count
 *   idx, cnt, b_max, n_max as for tria_compact
 * Each (unit, KV head) is moved by one workgroup in ascending chunks of 128 rows,
 * a chunk's reads completing before its writes: with ascending indices no row is
 * overwritten before it is read.  An index that is not ascending, below its row
 * or outside [0, len[u]) is flagged (TRIA_FLAG_INDEX) and its row left in place
 * (the head's result is then unspecified).  Errors as tria_compact.  K and V
 * views must not overlap each other.
 */
tria_status tria_compact_inplace(const tria_params* p, const tria_kv_view* k, const tria_kv_view* v, int32_t* pos,
                                 int32_t n_units, int32_t n_max, int32_t b_max, int32_t* len,
                                 const int32_t* idx, const int32_t* cnt, void* ws, void* stream);

/* tria_append - writes t_new new rows per (unit, KV head) at slots len[u] ..
 * len[u] + t_new - 1 (the decode loop's generated tokens), then advances the
 * unit's state on the device: len[u] <- min(len[u] + t_new, n_max) and, when
 * q_pos and pos_new are given, q_pos[u] <- pos_new[u][t_new - 1] (the newest
 * token is the current query of the next tria_score) [Calib issue: the port
 * tracks n_kv between prunes every 128 tokens].
 *   len         [device] int32 [U], read, then advanced
 *   q_pos       [device] int32 [U], or NULL (then not written)
 *   k_new, v_new [device] bf16 [U][Hkv][t_new][d], rows already rotated at their
 *               positions (as a model caches them)
 *   pos_new     [device] int32 [U][t_new] their positions, written to every
 *               head's row of pos ([U][Hkv][n_max]); both may be NULL
 * Slots at or past n_max are flagged (TRIA_FLAG_LEN) and skipped.
 */
tria_status tria_append(const tria_params* p, const tria_kv_view* k, const tria_kv_view* v, int32_t* pos,
                        int32_t n_units, int32_t n_max, int32_t* len, int32_t* q_pos, int32_t t_new,
                        const void* k_new, const void* v_new, const int32_t* pos_new, void* ws, void* stream);

/* tria_calibrate - the calibrated query statistics tria_score reads, from a stream
 * of pre-RoPE query rows [Calib issue, "How it works": per (layer, head, band)
 * means in the RoPE complex pairing; Blog, the calibration step].
 *
 * For layer l < L = p->n_layers, query head h < Hq = p->n_kv_heads * p->group
 * and band f < d/2, over the n_tokens rows q[l][h][t] (bf16, bands in
 * p->pairing's layout):
 *   q_mean_re[l][h][f]  = mean_t Re q_f      q_mean_im[l][h][f] = mean_t Im q_f
 *   q_abs_mean[l][h][f] = mean_t |q_f|
 *   r[l][h][f]   = |mean_t q_f| / mean_t |q_f|  (0 where mean_t |q_f| = 0); the
 *                  concentration whose complement weighs the norm term
 *   mrl[l][h][f] = |mean_t q_f / |q_f||          (q_f = 0 contributes 0); the
 *                  circular mean resultant length of the band's phases
 * The first three are tria_score's statistics arguments as they are.
 *   q           [device] bf16; row (l, h, t) starts at element
 *               l*stride_layer + h*stride_head + t*stride_token (each stride a
 *               multiple of 8 elements, q 16-byte aligned)
 *   n_tokens    >= 1
 *   q_mean_re, q_mean_im, q_abs_mean
 *               [device] fp32 [L][Hq][d/2]
 *   r, mrl      [device] fp32 [L][Hq][d/2], or NULL when not wanted
 *   ws          [device] workspace of ws_bytes >= tria_calibrate_workspace_size
 * Sums run in fp32 over chunks of 1024 tokens, then in fp64 over the chunks in a
 * fixed order: the results do not depend on the launch or on the strides.
 * p->offsets, rope_base, sink, window and agg are not used (but must be valid).
 * Inputs must be finite.  The call only enqueues work on `stream` (no
 * synchronisation); outputs and ws must not be in use by other work meanwhile.
 * Errors: TRIA_EINVAL (bad params, n_tokens < 1, a required pointer NULL),
 * TRIA_ESHAPE (q or a stride not aligned as above, a negative stride, more than
 * 65535 (layer, query head) pairs), TRIA_EWORKSPACE, TRIA_ELAUNCH.
 */
/* Bytes of workspace tria_calibrate needs (0 for invalid params or n_tokens < 1). */
size_t tria_calibrate_workspace_size(const tria_params* p, int32_t n_tokens);
tria_status tria_calibrate(const tria_params* p, const void* q, int64_t stride_layer, int64_t stride_head,
                           int64_t stride_token, int32_t n_tokens, float* q_mean_re, float* q_mean_im,
                           float* q_abs_mean, float* r, float* mrl, void* ws, size_t ws_bytes, void* stream);

/* TRIA statistics files [Calib issue: the port's loader takes a stats file with
 * magic 0x54524941 and versions 1..3, whose header gives the layer count, the KV
 * head count, fc (bands per head), head_dim, optional layer budget scales, and
 * per-head records of E[Re q_f], E[Im q_f], E|q_f| and an MRL field the loader
 * skips; layer budget scales default to 1.0].  The pages give neither the byte
 * order nor the field order; this library reads and writes little-endian:
 *   u32 magic, u32 version, u32 n_layers, u32 n_heads (query heads),
 *   u32 n_kv_heads, u32 fc;  version >= 2: u32 head_dim (= 2 fc);
 *   version >= 3: u32 flags (bit 0: f32 layer_budget_scales[n_layers] follow);
 *   then per (layer, query head), layer-major: f32 q_mean_real[fc],
 *   f32 q_mean_imag[fc], f32 q_abs_mean[fc], and (version >= 2) f32 mrl[fc].
 * Host memory only; no GPU work. */
typedef struct tria_stats_info {
  uint32_t version, n_layers, n_heads, n_kv_heads, fc, head_dim;
  int32_t has_budget_scales;   /* version 3 with the scales present             */
  int32_t mrl_present;         /* version >= 2                                   */
} tria_stats_info;

/* Parses n_bytes of a stats file.  The statistics arrays, when not NULL, receive
 * [n_layers][n_heads][fc] floats each (the layout tria_score reads); mrl zeros for
 * version 1; layer_budget_scales [n_layers] (1.0 where the file has none).  Returns
 * TRIA_EINVAL for a wrong magic, version or flag, TRIA_ESHAPE for inconsistent or
 * truncated data (the size must match the header exactly) or a header beyond 65536
 * layers, 4096 query heads or 4096 bands.  With all arrays NULL it reads the header
 * only; *info is written only on success.  The message is in tria_last_error(). */
tria_status tria_stats_parse(const void* bytes, size_t n_bytes, tria_stats_info* info, float* q_mean_re,
                             float* q_mean_im, float* q_abs_mean, float* mrl, float* layer_budget_scales);

/* Writes a stats file of info->version into out (cap bytes) and returns its size;
 * with out NULL or cap too small it writes nothing and returns the size needed; 0
 * for invalid arguments (as the parser: at most 65536 layers, 4096 query heads,
 * 4096 bands).  mrl may be NULL (zeros); layer_budget_scales is written for
 * version 3 when info->has_budget_scales is set. */
size_t tria_stats_encode(const tria_stats_info* info, const float* q_mean_re, const float* q_mean_im,
                         const float* q_abs_mean, const float* mrl, const float* layer_budget_scales, void* out,
                         size_t cap);

/* Folds a per-band mask m_f >= 0 into statistics of n_rows (layer, head) rows, in
 * place: E[q_f] <- m_f E[q_f] and E|q_f| <- E|q_f| + (m_f - 1) |E[q_f]|, so that
 * the trigonometric term of band f is scaled by m_f while the norm weight
 * E|q_f| - |E q_f| is unchanged [Fold note, sec. 7: the offset-independent
 * high-frequency mask multiplies ||mu'_f|| and commutes with the fold].  Host
 * arrays [n_rows][fc]. */
tria_status tria_stats_band_mask(int32_t n_rows, int32_t fc, const float* mask, float* q_mean_re, float* q_mean_im,
                                 float* q_abs_mean);

/* budgets[u] = round(budget * layer_budget_scales[unit_layer[u]]) for tria_select's
 * per-unit budgets [Calib issue: layer budget scales, 1.0 = uniform].  Host arrays. */
tria_status tria_stats_layer_budgets(int32_t n_units, const int32_t* unit_layer, int32_t n_layers,
                                     const float* layer_budget_scales, int32_t budget, int32_t* budgets);

/* Caps the number of workgroups tria_score's persistent kernel launches (0, the
 * default, means as many as the device holds at once), for callers that keep
 * compute units free for work on other streams.  A cap below the score tiles of
 * one (unit, KV head) (n_max / 2048, or n_max / 1024 when group > 4 or with the
 * maximum over offsets, rounded up)
 * makes tria_score return TRIA_ESHAPE.  Results do not depend on the cap: every
 * tile's arithmetic and every reduction run in a fixed order.  Process-wide;
 * returns the previous cap. */
int32_t tria_score_max_workgroups(int32_t cap);

/* tria_pass_noalloc - the whole pass, tria_score (no per-query-head scores) ->
 * tria_select -> tria_compact with the arguments of those three calls, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving loops
 * or harnesses that forbid allocation): instead of a caller's workspace it uses a
 * device array of the library's own, 96 MiB on each device the library runs on
 * (held until the process ends; the largest workspace the five benchmark workloads
 * need is 80 MiB).  It calls no allocating routine.  A pass whose workspace
 * (tria_workspace_size) exceeds 96 MiB returns TRIA_EWORKSPACE.  Every check of the
 * three calls runs before anything is launched.  The results equal those of the
 * three calls.
 *   flags  [device] int32, or NULL: receives this call's TRIA_FLAG_* word (the
 *          array's flag word is cleared at the start of every call)
 * All calls on one device share its array: calls that overlap in time on one device
 * (other streams, other host threads) race and give unspecified results; order them
 * on one stream. */
tria_status tria_pass_noalloc(const tria_params* p, const tria_kv_view* k, const tria_kv_view* v, int32_t n_units,
                              int32_t n_max, int32_t b_max, const int32_t* len, const int32_t* unit_layer,
                              const int32_t* q_pos, const int32_t* budget, const float* q_mean_re,
                              const float* q_mean_im, const float* q_abs_mean, const int32_t* pos_src,
                              int32_t pos_heads, float* agg, int32_t* idx, int32_t* cnt, const tria_kv_view* k_dst,
                              const tria_kv_view* v_dst, int32_t* pos_dst, int32_t* flags, void* stream);

/* Polls of tria_score's bounded wait for a group's merged moments (the default,
 * 65536, is ~0.1-0.2 s).  When a wait runs out, the workgroup computes the group's
 * moments directly from the K cache instead (TRIA_FLAG_SYNC is raised as
 * information).  A negative value skips the exchange altogether: every
 * finalisation computes its group's moments directly (each re-reads the group's
 * keys: for tests of that path, not for speed).  Results agree with the exchange
 * up to rounding.  Process-wide; returns the previous value.  For callers whose
 * other streams keep compute units busy, and for tests. */
int32_t tria_score_wait_polls(int32_t polls);

/* How tria_select distributes its work.  Both strategies keep the same slots
 * (bit-identical idx and cnt).
 *   TRIA_SELECT_AUTO      the faster one measured on MI355X: tiled (the default);
 *   TRIA_SELECT_PER_GROUP one workgroup selects a whole (unit, KV head) from
 *                         registers (falls back to tiled when n_max > 32768);
 *   TRIA_SELECT_TILED     tiles of 2048 slots count and emit in parallel, with
 *                         per-group threshold and refinement steps between.
 * Process-wide; returns the previous strategy (an unknown value selects AUTO). */
typedef enum { TRIA_SELECT_AUTO = 0, TRIA_SELECT_PER_GROUP = 1, TRIA_SELECT_TILED = 2 } tria_select_strategy_t;
int32_t tria_select_strategy(int32_t strategy);

/* Host decision log: one line per entry-point call on stderr, prefixed "[tria] ",
 * naming what the host chose (kernel variant, tile size and count, grid, LDS bytes,
 * selection strategy, compaction variant, workspace use), plus one line for every
 * error an entry point returns (status, name, detail).  Off unless the environment
 * variable TRIA_LOG is set to anything but "" or "0" when the library first logs.
 * tria_log(1) turns it on, tria_log(0) off, a negative value only queries.
 * Process-wide; returns the previous state (0 or 1). */
int32_t tria_log(int32_t on);

/* Reads (after synchronising `stream`) and clears the device flag word of a
 * workspace.  Returns TRIA_OK and the OR of TRIA_FLAG_* in *flags. */
tria_status tria_device_flags(void* ws, int32_t* flags, void* stream);

/* Human-readable name of a status code (static storage). */
const char* tria_strerror(tria_status s);

/* Detail of the last TRIA_ELAUNCH or validation failure on this thread. */
const char* tria_last_error(void);

/* Kernel timing with HIP events recorded on the launch stream around every
 * kernel launch.  tria_timing_enable(1) starts recording (0 stops);
 * tria_timing_read synchronises on the recorded events and returns, for each
 * kernel id k < n (see tria_kernel_name), the summed milliseconds and the
 * number of launches since the last read.  Returns the number of kernel ids. */
int32_t tria_timing_enable(int32_t on);
int32_t tria_timing_read(double* ms_sum, int64_t* launches, int32_t n);
const char* tria_kernel_name(int32_t k);

#ifdef __cplusplus
}
#endif

#endif /* TRIA_H_ */
