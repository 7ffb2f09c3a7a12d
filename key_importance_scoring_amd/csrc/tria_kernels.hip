// gfx950 kernels of the TriAttention score -> select -> compact pass.
//
// Sources (page title + equation):
//   Fold note  - academ.us article 2607.13051: the TriAttention score (Eqs. 1-3)
//                and the exact fold of its future-offset average (Eqs. 4-8);
//   Blog       - "TriAttention, or: what a rotating query already knows"
//                (The Method: keep the top-B, drop the rest; the norm term);
//   Calib issue - GitHub issue "Request: publish TriAttention calibration
//                script (TRIA v2/v3 stats.bin producer)" (band pairings,
//                statistics E[Re q_f], E[Im q_f], E|q_f|, budget/window/sink).
//
// Data flow of one pruning event (one stream):
//   k_coef    : per unit, the folded complex weights
//                 c_{h,f} = E[q_f] * W_f * e^{i w_f q_pos},
//                 W_f = (1/|D|) sum_delta e^{i w_f delta}    [Fold note, Eqs. 5-7]
//               written as a real d-vector in the key's pairing layout, and the
//               norm weights n_{h,f} = E|q_f| - |E[q_f]|;
//   k_score   : streams the bf16 K cache once; per key and query head
//                 s = sum_j C[j] K[j] + sum_f n_f |k_f|
//               on MFMA (hi/lo bf16 split of the fp32 coefficients), plus fp64
//               moment partials over the candidate slots;
//   k_agg     : z-normalisation per query head and GQA mean/max aggregation;
//               protected slots (sinks + recent window) get +inf;
//   k_select  : top-B per (unit, KV head) by LDS radix select on order-preserving
//               uint32 keys, ties to the lower slot, kept slots ascending;
//   k_compact : gathers kept K/V rows (16 B per lane) and positions.
//
// Why p_k never appears: the key's band in the pre-rotation frame is
// k_f = kr_f e^{-i w_f p_k}, and conj(k_f) e^{i w_f (q_pos - p_k + delta)} =
// conj(kr_f) e^{i w_f (q_pos + delta)}: the inverse rotation cancels against
// the distance rotation by angle addition (the rotary dot product of the Fold
// note's Eq. 3), so each score is a dot product of the cached row with a
// per-(unit, query head) coefficient vector.
#include "tria_kernels.h"

namespace tria {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int32_t kFlagLen = 1, kFlagLayer = 2, kFlagBudget = 4, kFlagBlock = 8, kFlagIndex = 16,
                  kFlagBmax = 32;

__device__ inline void raise_flag(int32_t* flags, int32_t bit) {
  if (flags) atomicOr(flags, bit);
}

__device__ inline int clamp_len(const int32_t* len, int u, int n_max, int32_t* flags) {
  int n = len[u];
  if (n < 0 || n > n_max) {
    raise_flag(flags, kFlagLen);
    n = n < 0 ? 0 : n_max;
  }
  return n;
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 (round to nearest even).
__device__ inline uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// hi/lo split of two fp32 values: x ~= hi + lo, both bf16, |x - hi - lo| <= 2^-17 |x|.
__device__ inline void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - bf_lo(hi), b - bf_hi(hi));
}

template <class V>
__device__ inline const uint16_t* row_ptr(const V& v, int u, int g, int slot, int32_t* flags) {
  if (v.bt == nullptr)
    return v.base + (int64_t)u * v.su + (int64_t)g * v.sh + (int64_t)slot * v.ss;
  const int blk = v.bt[(int64_t)u * v.mb + slot / v.bs];
  if (blk < 0 || blk >= v.npb) {
    raise_flag(flags, kFlagBlock);
    return nullptr;
  }
  return v.base + ((int64_t)blk * v.bs + slot % v.bs) * v.ss + (int64_t)g * v.sh;
}

// ============================================================================ k_coef
// One workgroup per unit.  Per-(band, offset) twiddles e^{i w_f delta} are summed
// by F x (256/F) threads into LDS partials; W_f and the rotation to q_pos are
// formed once per band; then every (query head, band) coefficient of the unit.
__global__ __launch_bounds__(256) void k_coef(CoefArgs a, Offsets offs) {
  const int u = blockIdx.x;
  const int F = a.d / 2;
  const int t = threadIdx.x;
  const int subs = 256 / F;
  const int f = t % F;
  const int s = t / F;
  __shared__ double tw_re[256], tw_im[256];
  __shared__ double rot_re[128], rot_im[128];

  // band frequency w_f = theta^(-2f/d)  [Fold note, sec. 2, Eq. 2 bullets]
  const double w = exp(-(2.0 * f / a.d) * a.log_base);
  double cs = 0.0, sn = 0.0;
  for (int j = s; j < offs.n; j += subs) {
    double sv, cv;
    sincos(w * offs.v[j], &sv, &cv);
    cs += cv;
    sn += sv;
  }
  tw_re[t] = cs;
  tw_im[t] = sn;
  __syncthreads();
  if (t < F) {
    double wr = 0.0, wi = 0.0;
    for (int j = 0; j < subs; ++j) {
      wr += tw_re[j * F + t];
      wi += tw_im[j * F + t];
    }
    wr /= offs.n;  // W_f  [Fold note, Eq. 6]
    wi /= offs.n;
    double sv, cv;
    sincos(w * (double)a.q_pos[u], &sv, &cv);
    rot_re[t] = wr * cv - wi * sv;  // W_f e^{i w_f q_pos}
    rot_im[t] = wr * sv + wi * cv;
  }
  __syncthreads();

  const int layer = a.unit_layer[u];
  const bool ok = layer >= 0 && layer < a.layers;
  if (!ok && t == 0) raise_flag(a.flags, kFlagLayer);
  for (int p = t; p < a.hq * F; p += 256) {
    const int h = p / F, b = p % F;
    double mr = 0.0, mi = 0.0, ab = 0.0;
    if (ok) {
      const size_t si = ((size_t)layer * a.hq + h) * F + b;
      mr = a.q_re[si];
      mi = a.q_im[si];
      ab = a.q_abs[si];
    }
    // c = mu' e^{i w q_pos} with mu' = E[q_f] W_f  [Fold note, Eq. 7]
    const double cr = mr * rot_re[b] - mi * rot_im[b];
    const double ci = mr * rot_im[b] + mi * rot_re[b];
    // Re(c conj(k)) = Re(c) Re(k) + Im(c) Im(k): coefficients sit where the key's
    // real / imaginary parts sit in the pairing layout  [Calib issue, pairing]
    float* crow = a.C + ((size_t)u * a.hq + h) * a.d;
    const int ire = a.pairing == 0 ? b : 2 * b;
    const int iim = a.pairing == 0 ? b + F : 2 * b + 1;
    crow[ire] = (float)cr;
    crow[iim] = (float)ci;
    // norm weight E|q_f| - |E q_f| = E|q_f| (1 - R_f)  [Blog, The Method; reading]
    a.N[((size_t)u * a.hq + h) * F + b] = (float)(ab - sqrt(mr * mr + mi * mi));
  }
}

// ============================================================================ k_score
// MFMA 16x16x32 bf16 layout (gfx950): lane l feeds A row (l & 15) and B column
// (l & 15) with k-elements [8 (l >> 4), 8 (l >> 4) + 8); it receives D rows
// 4 (l >> 4) + t, t < 4, of column (l & 15).
//
// Keys are A rows: a wave scores 16 keys per MFMA chain.  The contraction order
// over a row's elements is free, so lane group c = l >> 4 takes the elements
// [c d/8, (c+1) d/8) of each half of the row: that is d/32 16-byte loads per lane
// per key, and every band (both of its components) in the lane, for either
// pairing.  The norm term's magnitudes |k_f| are formed in-lane and fed to the
// MFMA as a second A operand.
//
// B columns: 0..G-1 carry the hi part of query head h's coefficients, 8..8+G-1
// the lo part; one DPP row shift by 8 adds them.  Magnitudes are split hi/lo
// too; the lo magnitudes meet only hi coefficients (the lo*lo product is below
// 2^-16 of the term).
template <int D>
struct Shape {
  static constexpr int F = D / 2;
  static constexpr int HC = D / 64;     // 8-element chunks per half per lane
  static constexpr int NKC = D / 32;    // chunks per lane = MFMAs of the dot part
  static constexpr int NQ = D / 8;      // bands per lane
  static constexpr int NNC = D / 64;    // MFMAs per norm part
};

template <int D>
__device__ inline int chunk_elem(int i, int c) {
  constexpr int HC = D / 64;
  return (i / HC) * (D / 2) + c * (D / 8) + (i % HC) * 8;
}

template <int D, int P>
__device__ inline int lane_band(int q, int c) {
  if (P == 0) return c * (D / 8) + q;                 // NEOX
  if (q < D / 16) return c * (D / 16) + q;            // interleaved, first half
  return D / 4 + c * (D / 16) + (q - D / 16);         // interleaved, second half
}

// |k_f|^2 for the lane's band q from its loaded chunks.
template <int D, int P>
__device__ inline float band_sq(const u32x4 (&ch)[D / 32], int q) {
  constexpr int HC = D / 64;
  if (P == 0) {
    const int i = q / 8, w = (q % 8) / 2;
    const uint32_t re = ch[i][w], im = ch[HC + i][w];
    const uint32_t pr = (q & 1) ? __builtin_amdgcn_perm(im, re, 0x07060302u)
                                : __builtin_amdgcn_perm(im, re, 0x05040100u);
    const bf16x2 v = __builtin_bit_cast(bf16x2, pr);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, 0.0f, false);
  } else {
    const int i = q < D / 16 ? q / 4 : HC + (q - D / 16) / 4;
    const uint32_t wv = ch[i][q % 4];
    const bf16x2 v = __builtin_bit_cast(bf16x2, wv);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, 0.0f, false);
  }
}

#ifndef TRIA_SCORE_NBI
#define TRIA_SCORE_NBI 4
#endif

// 16-key blocks per pipeline stage (d = 256 rows are twice as large: half as many)
template <int D>
constexpr int stage_blocks() { return D >= 256 ? (TRIA_SCORE_NBI + 1) / 2 : TRIA_SCORE_NBI; }

// One pipeline stage of a wave: stage_blocks blocks of 16 keys, d/32 16-byte chunks per lane each.
template <int D>
using Stage = u32x4[stage_blocks<D>()][D / 32];

// Issues the loads of one stage.  Keys at or past `kend` (the end of the wave's
// range) are clamped to its last key, whose row is already in cache: their scores
// are computed but never stored or counted.  Every load is unconditional, so the
// compiler can keep the next stage in flight while the current one computes.
template <int D, bool PAGED>
__device__ inline void load_stage(Stage<D>& ch, const KView& k, int u, int g, int kb, int kend, int col, int grp,
                                  const int* s_bt, int page0) {
#pragma unroll
  for (int b = 0; b < stage_blocks<D>(); ++b) {
    const int key = min(kb + 16 * b + col, kend - 1);
    const uint16_t* rp;
    if (!PAGED) {
      rp = k.base + (int64_t)u * k.su + (int64_t)g * k.sh + (int64_t)key * k.ss;
    } else {
      const int blk = s_bt[key / k.bs - page0];
      rp = k.base + ((int64_t)blk * k.bs + key % k.bs) * k.ss + (int64_t)g * k.sh;
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) ch[b][i] = *reinterpret_cast<const u32x4*>(rp + chunk_elem<D>(i, grp));
  }
}

template <int D, int P, bool PAGED>
__global__ __launch_bounds__(256) void k_score(ScoreArgs a) {
  using S = Shape<D>;
  constexpr int NBI = stage_blocks<D>();
  constexpr int KPW = kScoreTile / 4;  // keys per wave
  constexpr int STAGE = 16 * NBI;      // keys per pipeline stage
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int tile = blockIdx.x % a.n_tiles;
  const int ug = blockIdx.x / a.n_tiles;
  const int u = ug / a.hkv;
  const int g = ug % a.hkv;
  const int G = a.group;
  const int hq = a.hkv * G;
  const int n = clamp_len(a.len, u, a.n_max, threadIdx.x == 0 ? a.flags : nullptr);
  const int tile0 = tile * kScoreTile;

  // ---- paged caches: the tile's block ids, staged in LDS (checked once)
  __shared__ int s_bt[PAGED ? kScoreTile + 1 : 1];
  int page0 = 0;
  if (PAGED) {
    page0 = tile0 / a.k.bs;
    const int last = min(tile0 + kScoreTile, n) - 1;
    const int npages = last >= tile0 ? last / a.k.bs - page0 + 1 : 0;
    for (int i = threadIdx.x; i < npages; i += 256) {
      int blk = a.k.bt[(int64_t)u * a.k.mb + page0 + i];
      if (blk < 0 || blk >= a.k.npb) {
        raise_flag(a.flags, kFlagBlock);
        blk = 0;  // any in-pool block: the scores of this page are unspecified
      }
      s_bt[i] = blk;
    }
    __syncthreads();
  }

  // ---- B operands of this lane's column
  int head = -1;
  bool lo = false;
  if (col < G) head = col;
  else if (col >= 8 && col < 8 + G) { head = col - 8; lo = true; }
  bf16x8 bdot[S::NKC], bna[S::NNC], bnb[S::NNC];
  {
    const float* crow = a.C + ((size_t)u * hq + g * G + (head < 0 ? 0 : head)) * D;
    const float* nrow = a.N + ((size_t)u * hq + g * G + (head < 0 ? 0 : head)) * S::F;
#pragma unroll
    for (int i = 0; i < S::NKC; ++i) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (head >= 0) {
        const int e0 = chunk_elem<D>(i, grp);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t hi, lw;
          split_bf16(crow[e0 + 2 * j], crow[e0 + 2 * j + 1], hi, lw);
          w[j] = lo ? lw : hi;
        }
      }
      bdot[i] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int i = 0; i < S::NNC; ++i) {
      u32x4 wa = {0u, 0u, 0u, 0u}, wb = {0u, 0u, 0u, 0u};
      if (head >= 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = nrow[lane_band<D, P>(8 * i + 2 * j, grp)];
          const float x1 = nrow[lane_band<D, P>(8 * i + 2 * j + 1, grp)];
          uint32_t hi, lw;
          split_bf16(x0, x1, hi, lw);
          wa[j] = lo ? lw : hi;
          wb[j] = lo ? 0u : hi;
        }
      }
      bna[i] = __builtin_bit_cast(bf16x8, wa);
      bnb[i] = __builtin_bit_cast(bf16x8, wb);
    }
  }

  const bool owner = col >= 8 && col < 8 + G;  // lanes that hold a final score
  const int c_lo = a.sink, c_hi = n - a.window;  // candidates: [sink, n - window)
  float* raw_row = a.raw + ((size_t)u * hq + g * G + (owner ? col - 8 : 0)) * a.n_max;
  double msum = 0.0, msq = 0.0;
  int mcnt = 0;

  const int kw0 = tile0 + wave * KPW;
  const int kend = min(kw0 + KPW, n);   // this wave's keys: [kw0, kend)

  // scores of one loaded stage: magnitudes, MFMA chain, hi+lo merge, store, moments
  auto compute = [&](const Stage<D>& ch, int kb) {
#pragma unroll
    for (int b = 0; b < NBI; ++b) {
      bf16x8 mhi[S::NNC], mlo[S::NNC];
#pragma unroll
      for (int i = 0; i < S::NNC; ++i) {
        u32x4 h4, l4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float m0 = __builtin_amdgcn_sqrtf(band_sq<D, P>(ch[b], 8 * i + 2 * j));
          const float m1 = __builtin_amdgcn_sqrtf(band_sq<D, P>(ch[b], 8 * i + 2 * j + 1));
          uint32_t hi, lw;
          split_bf16(m0, m1, hi, lw);
          h4[j] = hi;
          l4[j] = lw;
        }
        mhi[i] = __builtin_bit_cast(bf16x8, h4);
        mlo[i] = __builtin_bit_cast(bf16x8, l4);
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < S::NKC; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ch[b][i]), bdot[i], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < S::NNC; ++i) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mhi[i], bna[i], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mlo[i], bnb[i], acc, 0, 0, 0);
      }
      // column c + 8 <- column c + column c + 8 (hi + lo of one query head)
      f32x4 sc;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int other = __builtin_amdgcn_mov_dpp(__float_as_int(acc[t]), 0x118, 0xF, 0xF, true);
        sc[t] = acc[t] + __int_as_float(other);
      }
      if (owner) {
        const int r0 = kb + 16 * b + 4 * grp;
        if (r0 + 3 < kend) {
          *reinterpret_cast<f32x4*>(raw_row + r0) = sc;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (r0 + t < kend) raw_row[r0 + t] = sc[t];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = r0 + t;
          if (r >= c_lo && r < c_hi && r < kend) {
            const double v = (double)sc[t];
            msum += v;
            msq += v * v;
            mcnt += 1;
          }
        }
      }
    }
  };

  // ---- two-stage register pipeline over the wave's keys [kw0, kend): the loads of
  // the next stage are in flight while the current stage computes
  if (kw0 < kend) {
    Stage<D> cA, cB;
    load_stage<D, PAGED>(cA, a.k, u, g, kw0, kend, col, grp, s_bt, page0);
    for (int kb = kw0;; kb += 2 * STAGE) {
      load_stage<D, PAGED>(cB, a.k, u, g, kb + STAGE, kend, col, grp, s_bt, page0);
      compute(cA, kb);
      if (kb + STAGE >= kend) break;
      load_stage<D, PAGED>(cA, a.k, u, g, kb + 2 * STAGE, kend, col, grp, s_bt, page0);
      compute(cB, kb + STAGE);
      if (kb + 2 * STAGE >= kend) break;
    }
  }

  // ---- moment partials of the tile: reduce over lane groups, then waves
  msum += __shfl_xor(msum, 16);
  msq += __shfl_xor(msq, 16);
  mcnt += __shfl_xor(mcnt, 16);
  msum += __shfl_xor(msum, 32);
  msq += __shfl_xor(msq, 32);
  mcnt += __shfl_xor(mcnt, 32);
  __shared__ double red_s[4][8], red_q[4][8];
  __shared__ int red_c[4][8];
  if (grp == 0 && owner) {
    red_s[wave][col - 8] = msum;
    red_q[wave][col - 8] = msq;
    red_c[wave][col - 8] = mcnt;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    double s = 0.0, q = 0.0;
    int c = 0;
    for (int w = 0; w < 4; ++w) {
      s += red_s[w][h];
      q += red_q[w][h];
      c += red_c[w][h];
    }
    double* p = a.part + (((size_t)u * hq + g * G + h) * a.n_tiles + tile) * 3;
    p[0] = (double)c;
    p[1] = s;
    p[2] = q;
  }
}

// ============================================================================ k_agg
// z-normalisation per query head over the candidate slots, then GQA aggregation.
__global__ __launch_bounds__(256) void k_agg(AggArgs a) {
  const int at = blockIdx.x % a.n_atiles;
  const int ug = blockIdx.x / a.n_atiles;
  const int u = ug / a.hkv;
  const int g = ug % a.hkv;
  const int G = a.group;
  const int hq = a.hkv * G;
  int n = a.len[u];
  n = n < 0 ? 0 : (n > a.n_max ? a.n_max : n);
  __shared__ float mean_s[kMaxGroup], inv_s[kMaxGroup];
  if ((int)threadIdx.x < G) {
    const double* p = a.part + ((size_t)u * hq + g * G + threadIdx.x) * a.n_tiles * 3;
    double c = 0.0, s = 0.0, q = 0.0;
    for (int i = 0; i < a.n_tiles; ++i) {
      c += p[3 * i];
      s += p[3 * i + 1];
      q += p[3 * i + 2];
    }
    const double m = c > 0.0 ? s / c : 0.0;
    const double var = c > 0.0 ? fmax(q / c - m * m, 0.0) : 0.0;
    mean_s[threadIdx.x] = (float)m;
    inv_s[threadIdx.x] = (float)(1.0 / fmax(sqrt(var), 1e-12));
  }
  __syncthreads();
  const int k0 = at * kAggTile + 4 * threadIdx.x;
  if (k0 >= n) return;
  f32x4 out;
#pragma unroll
  for (int t = 0; t < 4; ++t) out[t] = a.agg == 0 ? 0.0f : -__builtin_inff();
  const bool full = k0 + 3 < n;
  for (int h = 0; h < G; ++h) {
    const float* row = a.raw + ((size_t)u * hq + g * G + h) * a.n_max;
    f32x4 v;
    if (full) {
      v = *reinterpret_cast<const f32x4*>(row + k0);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = k0 + t < n ? row[k0 + t] : 0.0f;
    }
    const float m = mean_s[h], inv = inv_s[h];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float z = (v[t] - m) * inv;
      out[t] = a.agg == 0 ? out[t] + z : fmaxf(out[t], z);
    }
  }
  const float invg = 1.0f / (float)G;
  float* dst = a.out + ((size_t)u * a.hkv + g) * a.n_max;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int k = k0 + t;
    if (a.agg == 0) out[t] *= invg;
    if (k < a.sink || k >= n - a.window) out[t] = __builtin_inff();
  }
  if (full) {
    *reinterpret_cast<f32x4*>(dst + k0) = out;
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (k0 + t < n) dst[k0 + t] = out[t];
  }
}

// ============================================================================ k_select
__device__ inline uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);  // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the 1024 threads of the workgroup.
__device__ inline uint32_t block_scan_incl(uint32_t v, uint32_t* wtot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  __syncthreads();
  return v + base;
}

__global__ __launch_bounds__(kSelectThreads) void k_select(SelectArgs a) {
  const int ug = blockIdx.x;
  const int u = ug / a.hkv;
  const int g = ug % a.hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = clamp_len(a.len, u, a.n_max, g == 0 ? a.flags : nullptr);
  int B = a.budget[u];
  const int prot = min(n, a.sink + a.window);
  if (B < 0 || (n > B && B < prot)) {
    if (g == 0 && tid == 0) raise_flag(a.flags, kFlagBudget);
    B = B < 0 ? 0 : B;
  }
  int K = B < n ? B : n;
  if (K > a.b_max) {
    if (g == 0 && tid == 0) raise_flag(a.flags, kFlagBmax);
    K = a.b_max;
  }
  const float* v = a.agg + ((size_t)u * a.hkv + g) * a.n_max;
  int32_t* out = a.idx + ((size_t)u * a.hkv + g) * a.b_max;
  if (g == 0 && tid == 0) a.cnt[u] = K;

  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wtot[16], wg[16], we[16];
  __shared__ uint32_t sh_digit, sh_above;

  const bool keep_all = K >= n;
  uint32_t prefix = 0, pmask = 0;
  uint32_t krem = (uint32_t)K;
  if (!keep_all && K > 0) {
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = shifts[pass];
      const uint32_t nb = 1u << widths[pass];
      for (int i = tid; i < 2048; i += kSelectThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelectThreads) {
        const uint32_t key = order_key(v[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      // thread t owns bins nb-1-2t and nb-2-2t (descending): find the digit whose
      // cumulative count from the top first reaches krem
      const int b0 = (int)nb - 1 - 2 * tid, b1 = b0 - 1;
      const uint32_t c0 = b0 >= 0 ? hist[b0] : 0u, c1 = b1 >= 0 ? hist[b1] : 0u;
      const uint32_t incl = block_scan_incl(c0 + c1, wtot);
      const uint32_t excl = incl - c0 - c1;
      if (excl < krem && krem <= incl) {
        if (excl + c0 >= krem) {
          sh_digit = (uint32_t)b0;
          sh_above = excl;
        } else {
          sh_digit = (uint32_t)b1;
          sh_above = excl + c0;
        }
      }
      __syncthreads();
      prefix |= sh_digit << sh;
      pmask |= (nb - 1) << sh;
      krem -= sh_above;
      __syncthreads();
    }
  }
  // emission in ascending slot order: keep key > T, and the first krem slots with key == T
  const uint32_t T = prefix;
  const uint32_t keq = krem;
  uint32_t gt_base = 0, eq_base = 0;
  if (K > 0) {
    for (int base = 0; base < n; base += kSelectThreads) {
      const int i = base + tid;
      const bool valid = i < n;
      const uint32_t key = valid ? order_key(v[i]) : 0u;
      const bool gt = valid && (keep_all || key > T);
      const bool eq = valid && !keep_all && key == T;
      const uint64_t bg = __ballot(gt), be = __ballot(eq);
      if (lane == 0) {
        wg[wave] = (uint32_t)__popcll(bg);
        we[wave] = (uint32_t)__popcll(be);
      }
      __syncthreads();
      uint32_t pg = 0, pe = 0, tg = 0, te = 0;
      for (int w = 0; w < kSelectThreads / 64; ++w) {
        const uint32_t x = wg[w], y = we[w];
        if (w < wave) {
          pg += x;
          pe += y;
        }
        tg += x;
        te += y;
      }
      const uint32_t gb = gt_base + pg + lanes_below(bg);
      const uint32_t eb = eq_base + pe + lanes_below(be);
      // positions are < K by construction; the bound keeps a miscount from ever
      // writing past the caller's b_max row
      const uint32_t pos = gb + (eb < keq ? eb : keq);
      if ((gt || (eq && eb < keq)) && pos < (uint32_t)K) out[pos] = i;
      gt_base += tg;
      eq_base += te;
      __syncthreads();
    }
  }
  for (int j = K + tid; j < a.b_max; j += kSelectThreads) out[j] = -1;
}

// ============================================================================ k_compact
__global__ __launch_bounds__(256) void k_compact(CompactArgs a) {
  const int rt = blockIdx.x % a.n_rtiles;
  const int ug = blockIdx.x / a.n_rtiles;
  const int u = ug / a.hkv;
  const int g = ug % a.hkv;
  int K = a.cnt[u];
  K = K < 0 ? 0 : (K > a.b_max ? a.b_max : K);
  int n = a.len[u];
  n = n < 0 ? 0 : (n > a.n_max ? a.n_max : n);
  const int j0 = rt * kCompactRows;
  if (j0 >= K) return;
  const int lpr = a.d / 8;  // lanes per row, 16 bytes each
  const int rpp = 256 / lpr;
  const int part = threadIdx.x % lpr;
  const int32_t* ix = a.idx + ((size_t)u * a.hkv + g) * a.b_max;
  for (int r = threadIdx.x / lpr; r < kCompactRows; r += rpp) {
    const int j = j0 + r;
    if (j >= K) break;
    const int slot = ix[j];
    if (slot < 0 || slot >= n) {
      if (part == 0) raise_flag(a.flags, kFlagIndex);
      continue;
    }
    const uint16_t* ks = row_ptr(a.ks, u, g, slot, a.flags);
    const uint16_t* vs = row_ptr(a.vs, u, g, slot, a.flags);
    uint16_t* kd = const_cast<uint16_t*>(row_ptr(a.kd, u, g, j, a.flags));
    uint16_t* vd = const_cast<uint16_t*>(row_ptr(a.vd, u, g, j, a.flags));
    if (ks && kd)
      reinterpret_cast<u32x4*>(kd)[part] = reinterpret_cast<const u32x4*>(ks)[part];
    if (vs && vd)
      reinterpret_cast<u32x4*>(vd)[part] = reinterpret_cast<const u32x4*>(vs)[part];
    if (part == 0 && a.pos_src && a.pos_dst) {
      const int ph = a.pos_heads > 1 ? g : 0;
      a.pos_dst[((size_t)u * a.hkv + g) * a.b_max + j] =
          a.pos_src[((size_t)u * a.pos_heads + ph) * a.n_max + slot];
    }
  }
}

}  // namespace

// ============================================================================ launches
hipError_t launch_coef(const CoefArgs& a, const Offsets& offs, hipStream_t s) {
  if (a.n_units == 0) return hipSuccess;
  hipLaunchKernelGGL(k_coef, dim3(a.n_units), dim3(256), 0, s, a, offs);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, int d, int pairing, hipStream_t s) {
  const long blocks = (long)a.n_units * a.hkv * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), blk(256);
  const bool paged = a.k.bt != nullptr;
#define TRIA_SCORE_CASE(DD, PP, PG)                                        \
  if (d == DD && pairing == PP && paged == PG) {                           \
    hipLaunchKernelGGL((k_score<DD, PP, PG>), grid, blk, 0, s, a);        \
    return hipGetLastError();                                              \
  }
  TRIA_SCORE_CASE(64, 0, false)
  TRIA_SCORE_CASE(64, 1, false)
  TRIA_SCORE_CASE(128, 0, false)
  TRIA_SCORE_CASE(128, 1, false)
  TRIA_SCORE_CASE(256, 0, false)
  TRIA_SCORE_CASE(256, 1, false)
  TRIA_SCORE_CASE(64, 0, true)
  TRIA_SCORE_CASE(64, 1, true)
  TRIA_SCORE_CASE(128, 0, true)
  TRIA_SCORE_CASE(128, 1, true)
  TRIA_SCORE_CASE(256, 0, true)
  TRIA_SCORE_CASE(256, 1, true)
#undef TRIA_SCORE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_agg(const AggArgs& a, hipStream_t s) {
  const long blocks = (long)a.n_units * a.hkv * a.n_atiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_agg, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const long blocks = (long)a.n_units * a.hkv;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_select, dim3((unsigned)blocks), dim3(kSelectThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const long blocks = (long)a.n_units * a.hkv * a.n_rtiles;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_compact, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tria
