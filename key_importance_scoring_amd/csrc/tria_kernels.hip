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
//               on MFMA (hi/lo bf16 split of the fp32 coefficients).  A tile's
//               scores stay in LDS; the tiles of one (unit, KV head) exchange their
//               moments, then each z-normalises its scores per query head,
//               aggregates the GQA group (mean or max) and writes the aggregate;
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

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace tria {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int32_t kFlagLen = 1, kFlagLayer = 2, kFlagBudget = 4, kFlagBlock = 8, kFlagIndex = 16,
                  kFlagBmax = 32, kFlagSync = 64;

__device__ inline void raise_flag(int32_t* flags, int32_t bit) {
  if (flags) atomicOr(flags, bit);
}

__device__ inline int fix_len(int n, int n_max, int32_t* flags) {
  if (n < 0 || n > n_max) {
    raise_flag(flags, kFlagLen);
    n = n < 0 ? 0 : n_max;
  }
  return n;
}

__device__ inline int clamp_len(const int32_t* len, int u, int n_max, int32_t* flags) {
  return fix_len(len[u], n_max, flags);
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

// Linear bin of an aggregate: monotone non-decreasing in x, so a slot in a higher
// bin always ranks above a slot in a lower one (NaN, outside the contract, -> 0).
__device__ inline int lin_bin(float x) {
  if (!(x == x)) return 0;
  if (x == __builtin_inff()) return kBins - 1;
  if (x >= 8.0f) return kBins - 2;
  if (x < -8.0f) return 0;
  return 1 + (int)((x + 8.0f) * (float)kBinScale);  // [1, 16 kBinScale + 1]
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

// ============================================================================ MFMA operand layout
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
// 2^-16 of the term).  k_coef writes each lane's B operands (coefficients and
// norm weights, hi/lo split, zero in unused columns) in this order, so that
// k_score loads them with one coalesced 16-byte load per operand.
template <int D>
struct Shape {
  static constexpr int F = D / 2;
  static constexpr int HC = D / 64;     // 8-element chunks per half per lane
  static constexpr int NKC = D / 32;    // chunks per lane = MFMAs of the dot part
  static constexpr int NQ = D / 8;      // bands per lane
  static constexpr int NNC = D / 64;    // MFMAs per norm part
  static constexpr int NR = D / 64;     // 16-byte slots of a lane's reference magnitudes (NQ bf16)
  static constexpr int NBT = NKC + 2 * NNC + NR;   // 16-byte operands per lane written by k_coef
};

template <int D>
__device__ inline int chunk_elem(int i, int c) {
  constexpr int HC = D / 64;
  return (i / HC) * (D / 2) + c * (D / 8) + (i % HC) * 8;
}

// The band a lane's q-th magnitude belongs to (the order band_sq forms them in).
template <int D, int P>
__device__ inline int lane_band(int q, int c) {
  constexpr int HC = D / 64;
  if (P == 0) return chunk_elem<D>(q / 8, c) + q % 8;                 // NEOX: real parts in chunks < HC
  const int i = q < D / 16 ? q / 4 : HC + (q - D / 16) / 4;             // interleaved: (re, im) pairs
  return chunk_elem<D>(i, c) / 2 + q % 4;
}

// ============================================================================ k_coef
// Grid (unit, KV head).  Per-(band, offset) twiddles e^{i w_f delta} are summed by
// F x (256/F) threads into LDS partials; W_f and the rotation to q_pos are formed
// once per band; each (query head, band) of the group then forms its coefficient
// into LDS, and the block finally writes them as k_score's MFMA B operands, in the
// order its lanes load them (the MFMA operand layout above).  The block also
// resets its (unit, KV head)'s tile moments and merged moments to kUnpublished and
// its tile arrival count to 0, and clears its
// aggregate histogram; block (0, 0) clears the tile claim counter.
// sin and cos of an fp64 angle: reduced modulo 2 pi in fp64, then the fp32 sine and
// cosine of the remainder (|error| ~1e-7, far below the ~2^-17 relative precision of
// the split bf16 operands the coefficients end up in).
__device__ inline void sincos_reduced(double ang, double* sv, double* cv) {
  const float r = (float)(ang - 6.283185307179586 * rint(ang * 0.15915494309189535));
  float s, c;
  sincosf(r, &s, &c);
  *sv = s;
  *cv = c;
}

template <int D, int P>
__global__ __launch_bounds__(256) void k_coef(CoefArgs a, Offsets offs) {
  using S = Shape<D>;
  constexpr int F = D / 2;
  constexpr int NB = S::NKC + 2 * S::NNC;
  constexpr int PER = (kMaxGroup * F + 255) / 256;  // (head, band) pairs per thread
  const int u = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int G = a.group;
  const int hq = a.hkv * G;
  const size_t ug = (size_t)u * a.hkv + g;
  __shared__ double tw_re[256], tw_im[256];
  __shared__ double rot_re[F], rot_im[F];
  __shared__ float s_c[kMaxGroup * D];  // coefficient rows, pairing layout
  __shared__ float s_n[kMaxGroup * F];  // norm weights
  __shared__ double s_mur[kMaxGroup * F], s_mui[kMaxGroup * F], s_w[F];  // maximum over offsets

  __shared__ float s_ref[F];            // reference magnitudes (bf16 values)
  __shared__ float s_rsum[256];

  // blockIdx.z > 0: with the maximum over offsets, a block that writes a share of
  // the offset blocks' operands and nothing else; with the mean over offsets and few
  // (unit, KV head) pairs, one block per query head hz, each forming and writing
  // that head's coefficients, norm weights and shift (block 0 also the rest)
  const bool first = blockIdx.z == 0;
  const int hz = !a.omax && gridDim.z > 1 ? (int)blockIdx.z : -1;
  const bool own_b = first || hz >= 0;   // writes B operands (its head's, or all heads')
  const int n_u = clamp_len(a.len, u, a.n_max, nullptr);
  // Reference magnitudes of the norm term: r_f = the mean |k_f| over kRefRows slots
  // spread over the unit's keys.  The score kernel forms sum_f n_f (|k_f| - r_f) and
  // the constant sum_f n_f r_f is added back only where per-query-head scores are
  // written: the z-score does not change under a constant shift, and the bf16 hi/lo
  // operands then carry each key's deviation from the reference, not its whole
  // magnitude (so the error of a score stays small against the spread of the
  // scores even when the norm term dominates their mean).  Any r_f gives the same
  // scores in exact arithmetic.  Loaded first: they overlap the statistics' loads.
  constexpr int RPT = kRefRows / (256 / F);   // sample rows per thread
  uint32_t ref_re[RPT], ref_im[RPT];            // consumed after the twiddles: the loads overlap them
  {
    constexpr int subs = 256 / F;
    const int f = t % F, sub = t / F;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      ref_re[i] = ref_im[i] = 0u;
      if (own_b && n_u > 0) {
        const int r = sub + subs * i;
        const int slot = (int)(((2 * (int64_t)r + 1) * n_u) / (2 * kRefRows));
        const uint16_t* row = row_ptr(a.k, u, g, slot, nullptr);
        if (row) {
          ref_re[i] = row[P == 0 ? f : 2 * f];
          ref_im[i] = row[P == 0 ? f + F : 2 * f + 1];
        }
      }
    }
  }
  // tiles past len[u] hold no keys: their moments are published here, as zeros
  if (first) {
    const int64_t per = (int64_t)G * a.n_tiles * 3;
    for (int64_t i = t; i < per; i += 256) {
      const int tile = (int)((i / 3) % a.n_tiles);
      a.part[ug * per + i] = (int64_t)tile * a.tile >= n_u ? 0ull : kUnpublished;
    }
    for (int i = t; i < kBins; i += 256) a.hist[ug * kBins + i] = 0u;
    if (t < G) a.gstat[ug * G + t] = kUnpublished;
    if (t == 0) a.arrive[ug] = 0;
    if (u == 0 && g == 0 && t == 0) *a.next_tile = 0;
  }

  // statistics of this thread's (query head, band) pairs, loaded while the twiddles are formed
  const int layer = a.unit_layer[u];
  const bool ok = layer >= 0 && layer < a.layers;
  if (!ok && t == 0 && g == 0 && first) raise_flag(a.flags, kFlagLayer);
  double mr[PER], mi[PER], ab[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int p = t + 256 * k, h = p / F, b = p % F;
    mr[k] = mi[k] = ab[k] = 0.0;
    if (ok && h < G && (hz < 0 || h == hz)) {
      const size_t si = ((size_t)layer * hq + g * G + h) * F + b;
      mr[k] = a.q_re[si];
      mi[k] = a.q_im[si];
      ab[k] = a.q_abs[si];
    }
  }

  // band frequency w_f = theta^(-2f/d)  [Fold note, sec. 2, Eq. 2 bullets]
  constexpr int subs = 256 / F;
  const int f = t % F, sub = t / F;
  const double w = exp(-(2.0 * f / D) * a.log_base);
  double cs = 0.0, sn = 0.0;
  for (int j = sub; j < offs.n; j += subs) {
    double sv, cv;
    sincos_reduced(w * offs.v[j], &sv, &cv);
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
    sincos_reduced(w * (double)a.q_pos[u], &sv, &cv);
    rot_re[t] = wr * cv - wi * sv;  // W_f e^{i w_f q_pos}
    rot_im[t] = wr * sv + wi * cv;
  }
  __syncthreads();

#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int p = t + 256 * k, h = p / F, b = p % F;
    if (h >= G || (hz >= 0 && h != hz)) continue;
    // c = mu' e^{i w q_pos} with mu' = E[q_f] W_f  [Fold note, Eq. 7]
    const double cr = mr[k] * rot_re[b] - mi[k] * rot_im[b];
    const double ci = mr[k] * rot_im[b] + mi[k] * rot_re[b];
    // Re(c conj(k)) = Re(c) Re(k) + Im(c) Im(k): coefficients sit where the key's
    // real / imaginary parts sit in the pairing layout  [Calib issue, pairing]
    s_c[h * D + (P == 0 ? b : 2 * b)] = (float)cr;
    s_c[h * D + (P == 0 ? b + F : 2 * b + 1)] = (float)ci;
    // norm weight E|q_f| - |E q_f| = E|q_f| (1 - R_f)  [Blog, The Method; reading]
    s_n[h * F + b] = (float)(ab[k] - sqrt(mr[k] * mr[k] + mi[k] * mi[k]));
    if (a.omax) {
      s_mur[h * F + b] = mr[k];
      s_mui[h * F + b] = mi[k];
    }
  }
  if (a.omax && t < F) s_w[t] = w;
  {
    float rsum = 0.0f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float x = __uint_as_float(ref_re[i] << 16), y = __uint_as_float(ref_im[i] << 16);
      rsum += sqrtf(x * x + y * y);
    }
    s_rsum[t] = rsum;
  }
  __syncthreads();
  if (t < F) {
    float r = 0.0f;
    for (int j = 0; j < 256 / F; ++j) r += s_rsum[j * F + t];
    r *= 1.0f / (float)kRefRows;
    s_ref[t] = bf_lo(pack_bf16(r, 0.0f));   // the bf16 value the operands carry
  }
  __syncthreads();
  // the constant each query head's norm term was shifted by: sum_f n_f r_f (fp64)
  if (own_b) {
    const int lane = t & 63, wave = t >> 6;
    for (int h = wave; h < G; h += 4) {
      if (hz >= 0 && h != hz) continue;
      double c = 0.0;
      for (int f = lane; f < F; f += 64) c += (double)s_n[h * F + f] * (double)s_ref[f];
      for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
      if (lane == 0) a.nconst[(size_t)u * hq + g * G + h] = (float)c;
    }
  }

  // B operands: operand s of lane l at B[(u, g)][s][l]; s < NKC are the dot part's
  // chunks, then the norm part's hi-magnitude and lo-magnitude operands, then the
  // lane's reference magnitudes (bf16 pairs, in the order band_sq forms its bands)
  u32x4* dst = reinterpret_cast<u32x4*>(a.B) + ug * S::NBT * 64;
  for (int q = own_b ? t : S::NBT * 64; q < S::NBT * 64; q += 256) {
    const int s = q / 64, lane = q % 64;
    const int col = lane & 15, grp = lane >> 4;
    if (s >= NB) {
      if (hz > 0) continue;   // the reference magnitudes: block 0
      u32x4 w4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qb = 8 * (s - NB) + 2 * j;    // the lane's bands qb, qb + 1
        w4[j] = pack_bf16(s_ref[lane_band<D, P>(qb, grp)], s_ref[lane_band<D, P>(qb + 1, grp)]);
      }
      dst[s * 64 + lane] = w4;
      continue;
    }
    int head = -1;
    bool lo = false;
    if (col < G) head = col;
    else if (col >= 8 && col < 8 + G) { head = col - 8; lo = true; }
    if (hz >= 0 && head != hz && !(head < 0 && hz == 0)) continue;   // another block's head (zeros: block 0)
    u32x4 w4 = {0u, 0u, 0u, 0u};
    if (head >= 0) {
      if (s < S::NKC) {
        const int e0 = chunk_elem<D>(s, grp);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t hi, lw;
          split_bf16(s_c[head * D + e0 + 2 * j], s_c[head * D + e0 + 2 * j + 1], hi, lw);
          w4[j] = lo ? lw : hi;
        }
      } else {
        const int i = (s - S::NKC) % S::NNC;
        const bool second = s >= S::NKC + S::NNC;  // the operand that meets lo magnitudes
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = s_n[head * F + lane_band<D, P>(8 * i + 2 * j, grp)];
          const float x1 = s_n[head * F + lane_band<D, P>(8 * i + 2 * j + 1, grp)];
          uint32_t hi, lw;
          split_bf16(x0, x1, hi, lw);
          w4[j] = second ? (lo ? 0u : hi) : (lo ? lw : hi);
        }
      }
    }
    dst[s * 64 + lane] = w4;
  }

  // maximum over offsets: one coefficient row per (query head, offset),
  // c = E[q_f] e^{i w_f (q_pos + delta)}, nothing averaged [Fold note, sec. 4; Eq. 3
  // per offset], written as the offset blocks' B operands: column j = q G' + h < 8
  // of block cb is the hi part of head h at offset cb opb + q, column 8 + j the lo
  // part.  The angle is reduced modulo 2 pi in fp64 before an fp32 sine and cosine
  // (the operands keep ~16 bits).
  if (a.omax) {
    const OffsetBlocks ob = a.ob;
    const double qp = (double)a.q_pos[u];
    u32x4* dstm = reinterpret_cast<u32x4*>(a.Bmax) + ug * ob.nblk * S::NKC * 64;
    const int nq = ob.nblk * S::NKC * 64;
    const int share = (nq + (int)gridDim.z - 1) / (int)gridDim.z;   // this block's operands
    const int q1 = min(nq, share * ((int)blockIdx.z + 1));
    for (int q = share * (int)blockIdx.z + t; q < q1; q += 256) {
      const int cb = q / (S::NKC * 64), i = (q / 64) % S::NKC, lane = q % 64;
      const int col = lane & 15, grp = lane >> 4, j = col & 7;
      const bool lo = col >= 8;
      const int head = j % ob.gp < G ? j % ob.gp : -1;
      const int oi = min(cb * ob.opb + j / ob.gp, offs.n - 1);
      u32x4 w4 = {0u, 0u, 0u, 0u};
      if (head >= 0) {
        const double x = qp + offs.v[oi];
        const int e0 = chunk_elem<D>(i, grp);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int el = e0 + e;
          const int bnd = P == 0 ? (el < F ? el : el - F) : el / 2;
          const bool im = P == 0 ? el >= F : (el & 1);
          const double ang = s_w[bnd] * x;
          const float r = (float)(ang - 6.283185307179586 * rint(ang * 0.15915494309189535));
          float sv, cv;
          sincosf(r, &sv, &cv);
          const double mr = s_mur[head * F + bnd], mi = s_mui[head * F + bnd];
          v[e] = (float)(im ? mr * (double)sv + mi * (double)cv : mr * (double)cv - mi * (double)sv);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          uint32_t hi, lw;
          split_bf16(v[2 * jj], v[2 * jj + 1], hi, lw);
          w4[jj] = lo ? lw : hi;
        }
      }
      dstm[q] = w4;
    }
  }
}


// Inclusive prefix sum over a workgroup of NT threads (wtot: NT / 64 slots).
template <int NT>
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

// ============================================================================ k_score
// re^2 + im^2 of a packed bf16 pair (re in the low half), products exact in fp32.
// Kept as the builtin (not hand-written asm) so the compiler sees the instruction
// and inserts the wait states its consumers (v_sqrt) need.
__device__ inline float sq_bf16x2(uint32_t w) {
  const bf16x2 v = __builtin_bit_cast(bf16x2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, 0.0f, false);
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
    return sq_bf16x2(pr);
  } else {
    const int i = q < D / 16 ? q / 4 : HC + (q - D / 16) / 4;
    return sq_bf16x2(ch[i][q % 4]);
  }
}

#ifndef TRIA_SCORE_NBI
#define TRIA_SCORE_NBI 4
#endif

// 16-key blocks per pipeline stage (d = 256 rows are twice as large: half as many;
// the maximum over offsets keeps more accumulators: half as many again)
template <int D, bool MAXO = false>
constexpr int stage_blocks() {
  return MAXO ? (D >= 256 ? 2 : 4) : (D >= 256 ? (TRIA_SCORE_NBI + 1) / 2 : TRIA_SCORE_NBI);
}
// a wave's keys must be whole stages: a stage's scores are written to LDS for all its
// keys, and a partial last stage would write into the next wave's range.  Tiles are
// multiples of 256 keys (score_tile_keys balances them in steps of 256), so a wave
// takes a multiple of 64 keys: every stage size must divide 64.
template <int D, bool MAXO>
constexpr bool stage_divides_64() { return 64 % (16 * stage_blocks<D, MAXO>()) == 0; }
static_assert(stage_divides_64<64, false>() && stage_divides_64<128, false>() && stage_divides_64<256, false>() &&
                  stage_divides_64<64, true>() && stage_divides_64<128, true>() && stage_divides_64<256, true>(),
              "stage size must divide a wave's share of a tile (a multiple of 64 keys)");

// One pipeline stage of a wave: stage_blocks blocks of 16 keys, d/32 16-byte chunks per lane each.
template <int D, bool MAXO = false>
using Stage = u32x4[stage_blocks<D, MAXO>()][D / 32];

// Issues the loads of one stage.  Keys at or past `kend` (the end of the wave's
// range) are clamped to its last key, whose row is already in cache: their scores
// are computed but never counted.  Every load is unconditional, so the
// compiler can keep the next stage in flight while the current one computes.
template <int D, bool PAGED, bool MAXO = false>
__device__ inline void load_stage(Stage<D, MAXO>& ch, const KView& k, int u, int g, int kb, int kend, int col,
                                  int grp, const int* s_bt, int page0) {
#pragma unroll
  for (int b = 0; b < stage_blocks<D, MAXO>(); ++b) {
    const int key = min(kb + 16 * b + col, kend - 1);
    const uint16_t* rp;
    if (!PAGED) {
      rp = k.base + (int64_t)u * k.su + (int64_t)g * k.sh + (int64_t)key * k.ss;
    } else {
      const int b0 = s_bt[key / k.bs - page0];
      const int blk = b0 >= 0 && b0 < k.npb ? b0 : 0;
      rp = k.base + ((int64_t)blk * k.bs + key % k.bs) * k.ss + (int64_t)g * k.sh;
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      ch[b][i] = *reinterpret_cast<const u32x4*>(rp + chunk_elem<D>(i, grp));
    }
  }
}

// Per-tile indices.  Tiles of one (unit, KV head) are consecutive: t = ug * n_tiles + tile.
struct TileInfo {
  int ug, u, g, tile, n, tile0, tlen;
};

// The tile's place; its length fields are filled by tile_len (kept apart so that a
// tile's first loads need not wait for len[u]).
__device__ inline TileInfo tile_info(const ScoreArgs& a, int ug, int tile) {
  TileInfo ti;
  ti.tile = tile;
  ti.ug = ug;
  ti.u = ti.ug / a.hkv;
  ti.g = ti.ug % a.hkv;
  ti.tile0 = ti.tile * a.tile;
  ti.n = ti.tlen = 0;
  return ti;
}

__device__ inline void tile_len(const ScoreArgs& a, TileInfo& ti, int n_loaded, bool flag) {
  ti.n = fix_len(n_loaded, a.n_max, flag && threadIdx.x == 0 ? a.flags : nullptr);
  ti.tlen = max(0, min(a.tile, ti.n - ti.tile0));
}

// Registers a tile carries from tile_begin into tile_body: the wave's first stage of
// keys, the (unit, KV head)'s MFMA B operands and the unit's length as loaded.
template <int D, bool MAXO>
struct TileRegs {
  Stage<D, MAXO> cA;
  bf16x8 bdot[D / 32], bna[D / 64], bnb[D / 64];
  u32x4 rref[D / 64];   // the lane's reference magnitudes, bf16 pairs
  int n_loaded;
  int page0;
};

// Starts a tile: its block ids (paged caches) into LDS, then the loads of the B
// operands and of every wave's first stage of keys, issued before len[u] is known.
// Returns with those loads in flight, so that the work that follows (the previous
// tile's moments and finalisation) overlaps them.
template <int D, int P, bool PAGED, bool MAXO>
__device__ inline void tile_begin(const ScoreArgs& a, const TileInfo& ti, int n_known, int* s_bt,
                                  TileRegs<D, MAXO>& r) {
  using S = Shape<D>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int kpw = a.tile / 4;      // keys per wave
  const int u = ti.u, g = ti.g, tile0 = ti.tile0;
  const int kw0 = tile0 + wave * kpw;
  const int kw1 = kw0 + kpw;
  // the slots the first stage may read: up to len[u] when it is known (n_known >= 0);
  // else up to n_max (a dense view is readable, and a paged view's table covers, n_max
  // slots), so that the first stage is issued before len[u] arrives
  const int kcap = max(min(kw1, n_known >= 0 ? n_known : a.n_max), min(kw0 + 1, a.n_max));
  r.n_loaded = n_known >= 0 ? n_known : a.len[u];

  // ---- paged caches: the tile's block ids in LDS.  Ids of pages past len[u] may be
  // anything: load_stage maps an out-of-pool id to block 0, and only pages that
  // hold cached slots are checked (tile_body)
  r.page0 = 0;
  if (PAGED) {
    r.page0 = tile0 / a.k.bs;
    const int npcap = (min(tile0 + a.tile, a.n_max) - 1) / a.k.bs - r.page0 + 1;  // tile0 < n_max
    for (int i = threadIdx.x; i < npcap; i += 256) s_bt[i] = a.k.bt[(int64_t)u * a.k.mb + r.page0 + i];
    __syncthreads();
  }

  // ---- B operands of this lane's column, in the order k_coef wrote them
  {
    constexpr int NB = S::NKC + 2 * S::NNC;
    const u32x4* bsrc = reinterpret_cast<const u32x4*>(a.B) + (size_t)ti.ug * S::NBT * 64 + lane;
#pragma unroll
    for (int i = 0; i < S::NKC; ++i) r.bdot[i] = __builtin_bit_cast(bf16x8, bsrc[i * 64]);
#pragma unroll
    for (int i = 0; i < S::NNC; ++i) {
      r.bna[i] = __builtin_bit_cast(bf16x8, bsrc[(S::NKC + i) * 64]);
      r.bnb[i] = __builtin_bit_cast(bf16x8, bsrc[(S::NKC + S::NNC + i) * 64]);
    }
    if constexpr (!MAXO) {
#pragma unroll
      for (int i = 0; i < S::NR; ++i) r.rref[i] = bsrc[(NB + i) * 64];
    }
  }

  // the first stage, unconditionally: a wave with no keys reloads row kcap - 1, which
  // is below n_max and at or past tile0
  load_stage<D, PAGED, MAXO>(r.cA, a.k, u, g, kw0, kcap, col, grp, s_bt, r.page0);
}

// Scores a started tile into LDS (s_raw, [G][tile + 16]); ends with a barrier, the
// tile's scores complete in LDS.
template <int D, int P, bool PAGED, bool MAXO>
__device__ inline void tile_body(const ScoreArgs& a, TileInfo& ti, float* s_raw, const int* s_bt, u32x4* s_bmax,
                                 int* s_bug, TileRegs<D, MAXO>& r) {
  using S = Shape<D>;
  constexpr int NBI = stage_blocks<D, MAXO>();
  constexpr int STAGE = 16 * NBI;  // keys per pipeline stage
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;
  const int RS = a.tile + 16;      // LDS row stride: heads start 16 banks apart
  const int kpw = a.tile / 4;      // keys per wave
  const int u = ti.u, g = ti.g, tile0 = ti.tile0;
  const int kw0 = tile0 + wave * kpw;
  const int page0 = r.page0;
  Stage<D, MAXO>& cA = r.cA;
  Stage<D, MAXO> cB;
  const bf16x8(&bdot)[S::NKC] = r.bdot;
  const bf16x8(&bna)[S::NNC] = r.bna;
  const bf16x8(&bnb)[S::NNC] = r.bnb;
  // |k_f| - r_f for the lane's q-th band (the reference packed two per word; the
  // maximum over offsets, whose score loop has no registers to spare, keeps the
  // lane's references in LDS after its staged offset blocks)
  const u32x4* s_rref = s_bmax + a.ob.nblk * S::NKC * 64;
  auto mag_ref = [&](const u32x4 (&ch)[D / 32], int q, const u32x4 (&rr)[S::NR]) {
    const float m = __builtin_amdgcn_sqrtf(band_sq<D, P>(ch, q));
    const uint32_t w = rr[q / 8][(q % 8) / 2];
    return m - ((q & 1) ? bf_hi(w) : bf_lo(w));
  };
  auto mag = [&](const u32x4 (&ch)[D / 32], int q) { return mag_ref(ch, q, r.rref); };

  // maximum over offsets: the (unit, KV head)'s offset blocks into LDS, unless the
  // previous tile of this workgroup already staged them (its reads have ended at the
  // barrier that closed its score loop)
  if constexpr (MAXO) {
    if (*s_bug != ti.ug) {
      const int nq = a.ob.nblk * S::NKC * 64;
      const u32x4* src = reinterpret_cast<const u32x4*>(a.Bmax) + (size_t)ti.ug * nq;
      // the lane's reference magnitudes after the blocks (from k_coef's operands)
      if (threadIdx.x < 64) {
        constexpr int NB = S::NKC + 2 * S::NNC;
        const u32x4* rsrc = reinterpret_cast<const u32x4*>(a.B) + (size_t)ti.ug * S::NBT * 64 + threadIdx.x;
#pragma unroll
        for (int i = 0; i < S::NR; ++i) s_bmax[nq + i * 64 + threadIdx.x] = rsrc[(NB + i) * 64];
      }
      for (int q0 = 0; q0 < nq; q0 += 256 * 8) {
        u32x4 tmp[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int q = min(q0 + (int)threadIdx.x + 256 * k, nq - 1);
          tmp[k] = src[q];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int q = q0 + (int)threadIdx.x + 256 * k;
          if (q < nq) s_bmax[q] = tmp[k];
        }
      }
      __syncthreads();
      if (threadIdx.x == 0) *s_bug = ti.ug;
    }
  }

  tile_len(a, ti, r.n_loaded, true);
  const int n = ti.n;
  if (PAGED) {
    const int last = min(tile0 + a.tile, n) - 1;
    const int npages = last >= tile0 ? last / a.k.bs - page0 + 1 : 0;
    for (int i = threadIdx.x; i < npages; i += 256) {
      const int blk = s_bt[i];
      if (blk < 0 || blk >= a.k.npb) raise_flag(a.flags, kFlagBlock);  // those scores are unspecified
    }
  }

  const bool owner = col >= 8 && col < 8 + G;  // lanes that hold a final score
  float* s_row = s_raw + (owner ? col - 8 : 0) * RS - tile0;
  const int kend = min(kw0 + kpw, n);   // this wave's keys: [kw0, kend)

  // scores of one loaded stage: dot-product MFMAs of every block first (independent
  // accumulators), then per block the magnitudes and the norm-term MFMAs
  auto compute = [&](const Stage<D, MAXO>& ch, int kb) {
    f32x4 acc[NBI];
#pragma unroll
    for (int b = 0; b < NBI; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < S::NKC; ++i)
#pragma unroll
      for (int b = 0; b < NBI; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ch[b][i]), bdot[i], acc[b], 0,
                                                         0, 0);
#pragma unroll
    for (int b = 0; b < NBI; ++b) {
#pragma unroll
      for (int i = 0; i < S::NNC; ++i) {
        u32x4 h4, l4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float m0 = mag(ch[b], 8 * i + 2 * j);
          const float m1 = mag(ch[b], 8 * i + 2 * j + 1);
          uint32_t hi, lw;
          split_bf16(m0, m1, hi, lw);
          h4[j] = hi;
          l4[j] = lw;
        }
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h4), bna[i], acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l4), bnb[i], acc[b], 0, 0, 0);
      }
    }
#pragma unroll
    for (int b = 0; b < NBI; ++b) {
      // column c + 8 <- column c + column c + 8 (hi + lo of one query head)
      f32x4 sc;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int other = __builtin_amdgcn_mov_dpp(__float_as_int(acc[b][t]), 0x118, 0xF, 0xF, true);
        sc[t] = acc[b][t] + __int_as_float(other);
      }
      if (owner) *reinterpret_cast<f32x4*>(s_row + kb + 16 * b + 4 * grp) = sc;
    }
  };

  // maximum over offsets, two stages at once: every offset block's B operands are
  // read from LDS once for both stages' key blocks (the LDS is this mode's busiest
  // unit); the norm term is formed last, so that its accumulators are not held
  // across the offset blocks.  TWO = false: the first stage only (a wave's tail).
  auto compute_max = [&](auto two, const Stage<D, MAXO>& c0, const Stage<D, MAXO>& c1, int kb) {
    constexpr bool TWO = decltype(two)::value;
    constexpr int NB2 = TWO ? 2 * NBI : NBI;
    // key block bb of the pair: blocks 0 .. NBI-1 from the first stage, then the second's
    auto blk = [&](int bb) -> const u32x4 (&)[D / 32] { return bb < NBI ? c0[bb] : c1[bb - NBI]; };
    f32x4 best[NB2];
#pragma unroll
    for (int bb = 0; bb < NB2; ++bb)
#pragma unroll
      for (int t = 0; t < 4; ++t) best[bb][t] = -__builtin_inff();
    const int nblk = a.ob.nblk;
    for (int cb = 0; cb < nblk; ++cb) {
      bf16x8 bo[S::NKC];
#pragma unroll
      for (int i = 0; i < S::NKC; ++i) bo[i] = __builtin_bit_cast(bf16x8, s_bmax[(cb * S::NKC + i) * 64 + lane]);
      f32x4 acc[NB2];
#pragma unroll
      for (int bb = 0; bb < NB2; ++bb) acc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < S::NKC; ++i)
#pragma unroll
        for (int bb = 0; bb < NB2; ++bb)
          acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, blk(bb)[i]), bo[i], acc[bb],
                                                            0, 0, 0);
      // hi + lo of each (offset, head) into lanes 8..15, then the running maximum
#pragma unroll
      for (int bb = 0; bb < NB2; ++bb)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int other = __builtin_amdgcn_mov_dpp(__float_as_int(acc[bb][t]), 0x118, 0xF, 0xF, true);
          best[bb][t] = __builtin_elementwise_maximum(best[bb][t], acc[bb][t] + __int_as_float(other));
        }
    }
    // the offsets held by lanes 8 + q G' + h, q < opb, meet in lane 8 + h
    for (int sft = a.ob.gp; sft < 8; sft *= 2) {
#pragma unroll
      for (int bb = 0; bb < NB2; ++bb)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int x = __float_as_int(best[bb][t]);
          const int y = sft == 1 ? __builtin_amdgcn_mov_dpp(x, 0x101, 0xF, 0xF, true)
                      : sft == 2 ? __builtin_amdgcn_mov_dpp(x, 0x102, 0xF, 0xF, true)
                                 : __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, true);
          best[bb][t] = __builtin_elementwise_maximum(best[bb][t], __int_as_float(y));
        }
    }
    // the norm term (no offset), hi + lo merged into the owner lanes as well; the
    // lane's references from LDS, once for all the blocks
    u32x4 rr[S::NR];
#pragma unroll
    for (int i = 0; i < S::NR; ++i) rr[i] = s_rref[i * 64 + lane];
#pragma unroll
    for (int bb = 0; bb < NB2; ++bb) {
      f32x4 nrm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < S::NNC; ++i) {
        u32x4 h4, l4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float m0 = mag_ref(blk(bb), 8 * i + 2 * j, rr);
          const float m1 = mag_ref(blk(bb), 8 * i + 2 * j + 1, rr);
          uint32_t hi, lw;
          split_bf16(m0, m1, hi, lw);
          h4[j] = hi;
          l4[j] = lw;
        }
        nrm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h4), bna[i], nrm, 0, 0, 0);
        nrm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l4), bnb[i], nrm, 0, 0, 0);
      }
      f32x4 sc;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int other = __builtin_amdgcn_mov_dpp(__float_as_int(nrm[t]), 0x118, 0xF, 0xF, true);
        sc[t] = best[bb][t] + nrm[t] + __int_as_float(other);
      }
      if (owner) *reinterpret_cast<f32x4*>(s_row + kb + 16 * bb + 4 * grp) = sc;
    }
  };

  // ---- register double buffer over the wave's keys [kw0, kend): the next stage's
  // loads are issued while the current stage computes.  (Keeping two stages in
  // flight across each wait measured slower on the full cache: more outstanding
  // requests per wave did not raise the delivered bandwidth.)
  if constexpr (MAXO) {
    // the maximum over offsets takes two stages per pass over the offset blocks:
    // both are loaded (the second issued here, the first at the previous step),
    // then computed together; the wave's other stage loads follow the compute
    for (int kb = kw0; kb < kend; kb += 2 * STAGE) {
      if (kb + STAGE < kend) {
        load_stage<D, PAGED, MAXO>(cB, a.k, u, g, kb + STAGE, kend, col, grp, s_bt, page0);
        compute_max(std::true_type{}, cA, cB, kb);
      } else {
        compute_max(std::false_type{}, cA, cA, kb);
      }
      if (kb + 2 * STAGE < kend) load_stage<D, PAGED, MAXO>(cA, a.k, u, g, kb + 2 * STAGE, kend, col, grp, s_bt, page0);
    }
  } else if (kw0 < kend) {
    for (int kb = kw0;; kb += 2 * STAGE) {
      load_stage<D, PAGED, MAXO>(cB, a.k, u, g, kb + STAGE, kend, col, grp, s_bt, page0);
      compute(cA, kb);
      if (kb + STAGE >= kend) break;
      load_stage<D, PAGED, MAXO>(cA, a.k, u, g, kb + 2 * STAGE, kend, col, grp, s_bt, page0);
      compute(cB, kb + STAGE);
      if (kb + 2 * STAGE >= kend) break;
    }
  }
  __syncthreads();
}

// Adds the moments (nb, mb, M2b) of a set of scores to the running (n, m, M2):
// count, mean and sum of squared deviations of the union (the pairwise update of
// Chan, Golub and LeVeque).  An empty set (nb = 0) changes nothing; an empty running
// set takes the other's moments as they are.
__device__ inline void chan_merge(double& n, double& m, double& M2, double nb, double mb, double M2b) {
  const double nt = n + nb;
  if (nt > 0.0) {
    const double d = mb - m;
    const double f = nb / nt;
    m += d * f;
    M2 += M2b + d * d * n * f;
  }
  n = nt;
}

// One query head's moments over every tile of its (unit, KV head), from each tile's
// (count, mean, M2) by the pairwise update of Chan, Golub and LeVeque (no difference
// of large sums), in a fixed order: lane j merges tiles j, j + 64, ... in turn, then
// a fixed shuffle tree merges the lanes.  One wave; polls until none of the head's
// moments reads kUnpublished, at most a.wait_polls times.  Returns false when the
// wait ran out; else every lane holds the group's count c, mean m and M2.
__device__ inline bool merge_head(const ScoreArgs& a, size_t qh, double& c, double& m, double& m2) {
  const int lane = threadIdx.x & 63;
  const unsigned long long* p = reinterpret_cast<const unsigned long long*>(a.part + qh * a.n_tiles * 3);
  for (int polls = 0;; ++polls) {
    c = m = m2 = 0.0;
    bool missing = false;
    for (int j = lane; j < a.n_tiles; j += 64) {
      const unsigned long long x0 = __hip_atomic_load(p + 3 * j + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned long long x1 = __hip_atomic_load(p + 3 * j + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned long long x2 = __hip_atomic_load(p + 3 * j + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      missing |= (x0 == kUnpublished) | (x1 == kUnpublished) | (x2 == kUnpublished);
      chan_merge(c, m, m2, __longlong_as_double(x0), __longlong_as_double(x1), __longlong_as_double(x2));
    }
    if (__ballot(missing) == 0) break;
    if (polls >= a.wait_polls) return false;
    __builtin_amdgcn_s_sleep(8);
  }
  for (int o = 32; o > 0; o >>= 1) {
    const double oc = __shfl_xor(c, o), om = __shfl_xor(m, o), om2 = __shfl_xor(m2, o);
    chan_merge(c, m, m2, oc, om, om2);
  }
  return true;
}

// The group's mean and inverse standard deviation of one query head from its merged
// moments, as two fp32 in one word (mean in the low half).
__device__ inline uint64_t pack_stats(double c, double m, double m2) {
  const double var = c > 0.0 ? fmax(m2 / c, 0.0) : 0.0;
  const float mean = (float)(c > 0.0 ? m : 0.0);
  const float inv = (float)(1.0 / fmax(sqrt(var), 1e-12));
  return (uint64_t)__float_as_uint(mean) | ((uint64_t)__float_as_uint(inv) << 32);
}

// The end of a scored tile (lengths filled by tile_body): its per-query-head scores
// (if wanted) and its candidate moments (count, mean, sum of squared deviations),
// published for the other tiles of its (unit, KV head).
// UNROLL: the moment passes' loops unrolled (the mean over offsets: faster; the
// maximum, whose score loop has no registers to spare: slower).
template <bool UNROLL>
__device__ inline void tile_end(const ScoreArgs& a, const TileInfo& ti, const float* s_raw) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = a.group;
  const int hq = a.hkv * G;
  const int RS = a.tile + 16;
  const int u = ti.u, g = ti.g, tile0 = ti.tile0;
  const int n = ti.n;

  // ---- per-query-head scores, if the caller wants them: full lines per head
  const int tlen = ti.tlen;
  // (the tile's scores in LDS are shifted by the head's norm constant; added back here)
  if (a.raw) {
    for (int h = 0; h < G; ++h) {
      float* dst = a.raw + ((size_t)u * hq + g * G + h) * a.n_max + tile0;
      const float* src = s_raw + h * RS;
      const float c = a.nconst[(size_t)u * hq + g * G + h];
      for (int i = 4 * threadIdx.x; i < tlen; i += 4 * 256) {
        if (i + 3 < tlen) {
          f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] += c;
          *reinterpret_cast<f32x4*>(dst + i) = v;
        } else {
          for (int t = i; t < tlen; ++t) dst[t] = src[t] + c;
        }
      }
    }
  }

  // ---- moments of the tile over its candidate slots [sink, n - window): two
  // passes over LDS (mean, then squared deviations), one wave per query head.
  // Published with agent-scope stores: the other tiles of this (unit, KV head)
  // run on other CUs and XCDs.
  const int c0 = max(a.sink, tile0) - tile0;
  const int c1 = min(n - a.window, tile0 + tlen) - tile0;
  // lane l reads 16-byte groups 4 (l + 64 k): all of a pass's LDS loads are
  // independent, and the unrolled loop (8 groups at 2048 keys) keeps them in flight
  // together
  const int ngrp = (a.tile / 4 + 63) / 64;     // 16-byte groups per lane
  for (int h = wave; h < G; h += 4) {
    const float* src = s_raw + h * RS;
    float acc = 0.0f;
    auto sum_group = [&](int k) {
      const int i = 4 * (lane + 64 * k);
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + i);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (i + t >= c0 && i + t < c1) acc += x[t];
    };
    if constexpr (UNROLL) {
#pragma unroll 8
      for (int k = 0; k < ngrp; ++k) sum_group(k);
    } else {
      for (int k = 0; k < ngrp; ++k) sum_group(k);
    }
    double sum = (double)acc;
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    const int cnt = max(0, c1 - c0);
    const double mean = cnt > 0 ? sum / cnt : 0.0;
    const float mf = (float)mean;
    float q = 0.0f;
    auto sq_group = [&](int k) {
      const int i = 4 * (lane + 64 * k);
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + i);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float dv = x[t] - mf;
        if (i + t >= c0 && i + t < c1) q = __builtin_fmaf(dv, dv, q);
      }
    };
    if constexpr (UNROLL) {
#pragma unroll 8
      for (int k = 0; k < ngrp; ++k) sq_group(k);
    } else {
      for (int k = 0; k < ngrp; ++k) sq_group(k);
    }
    double m2 = (double)q;
    for (int o = 32; o > 0; o >>= 1) m2 += __shfl_xor(m2, o);
    // pass-two deviations are about mf (the mean rounded to fp32): shift back
    const double dm = mean - (double)mf;
    m2 = fmax(m2 - (double)cnt * dm * dm, 0.0);
    if (lane == 0) {
      unsigned long long* p =
          reinterpret_cast<unsigned long long*>(a.part + (((size_t)u * hq + g * G + h) * a.n_tiles + ti.tile) * 3);
      __hip_atomic_store(p + 0, (unsigned long long)__double_as_longlong((double)cnt), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p + 1, (unsigned long long)__double_as_longlong(mean), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p + 2, (unsigned long long)__double_as_longlong(m2), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // nothing waits for these stores: each moment is a single-copy-atomic 8-byte
  // store, and a reader takes it as published once it no longer reads kUnpublished

  // The last non-empty tile of the (unit, KV head) to count itself in merges every
  // tile's moments once (instead of once per finalisation) and publishes each query
  // head's mean and inverse deviation; the others' moments are already issued, so its
  // wait is short.  If that wait runs out, nothing is published and the finalisations
  // compute the moments directly.
  if (tlen > 0 && a.wait_polls >= 0) {
    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(a.arrive + ti.ug, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
               (n + a.tile - 1) / a.tile;
    __syncthreads();
    if (s_last) {
      for (int h = wave; h < G; h += 4) {
        double c, m, m2;
        const size_t qh = (size_t)u * hq + g * G + h;
        if (merge_head(a, qh, c, m, m2) && lane == 0)
          __hip_atomic_store(a.gstat + qh, (unsigned long long)pack_stats(c, m, m2), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------------------- direct moments
// The slow path of the moment exchange: when a finalisation's wait for the other
// tiles' moments runs out (or the host asks for it, see tria_score_wait_polls), the
// workgroup scores every candidate slot of the group again, straight from the K
// cache, and forms the group's moments itself: the result then never depends on the
// other tiles' workgroups being resident.  The scores are the score kernel's own
// (the same MFMA sequence per key); the moments are Welford updates per lane in fp64
// merged in a fixed order, so they equal the exchanged ones up to rounding.

// Scores of one 16-key block for every query head of the group, in the MFMA output
// layout: after the hi + lo merge, lane (8 + h, grp) holds query head h's scores of
// keys 4 grp .. 4 grp + 3 of the block (the same operation order as tile_body).
template <int D, int P, bool MAXO>
__device__ inline f32x4 block_scores(const ScoreArgs& a, size_t ug, const u32x4 (&ch)[D / 32],
                                     const bf16x8 (&bdot)[D / 32], const bf16x8 (&bna)[D / 64],
                                     const bf16x8 (&bnb)[D / 64], const u32x4 (&rref)[D / 64]) {
  using S = Shape<D>;
  const int lane = threadIdx.x & 63;
  auto mag = [&](int q) {
    const uint32_t w = rref[q / 8][(q % 8) / 2];
    return __builtin_amdgcn_sqrtf(band_sq<D, P>(ch, q)) - ((q & 1) ? bf_hi(w) : bf_lo(w));
  };
  auto norm_part = [&](f32x4 acc) {
#pragma unroll
    for (int i = 0; i < S::NNC; ++i) {
      u32x4 h4, l4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t hi, lw;
        split_bf16(mag(8 * i + 2 * j), mag(8 * i + 2 * j + 1), hi, lw);
        h4[j] = hi;
        l4[j] = lw;
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h4), bna[i], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l4), bnb[i], acc, 0, 0, 0);
    }
    return acc;
  };
  f32x4 sc;
  if constexpr (!MAXO) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < S::NKC; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ch[i]), bdot[i], acc, 0, 0, 0);
    acc = norm_part(acc);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int other = __builtin_amdgcn_mov_dpp(__float_as_int(acc[t]), 0x118, 0xF, 0xF, true);
      sc[t] = acc[t] + __int_as_float(other);
    }
  } else {
    f32x4 best;
#pragma unroll
    for (int t = 0; t < 4; ++t) best[t] = -__builtin_inff();
    const u32x4* bm = reinterpret_cast<const u32x4*>(a.Bmax) + ug * a.ob.nblk * S::NKC * 64 + lane;
    for (int cb = 0; cb < a.ob.nblk; ++cb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < S::NKC; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ch[i]),
                                                      __builtin_bit_cast(bf16x8, bm[(cb * S::NKC + i) * 64]), acc,
                                                      0, 0, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int other = __builtin_amdgcn_mov_dpp(__float_as_int(acc[t]), 0x118, 0xF, 0xF, true);
        best[t] = __builtin_elementwise_maximum(best[t], acc[t] + __int_as_float(other));
      }
    }
    for (int sft = a.ob.gp; sft < 8; sft *= 2) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int x = __float_as_int(best[t]);
        const int y = sft == 1 ? __builtin_amdgcn_mov_dpp(x, 0x101, 0xF, 0xF, true)
                    : sft == 2 ? __builtin_amdgcn_mov_dpp(x, 0x102, 0xF, 0xF, true)
                               : __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, true);
        best[t] = __builtin_elementwise_maximum(best[t], __int_as_float(y));
      }
    }
    const f32x4 nrm = norm_part(f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int other = __builtin_amdgcn_mov_dpp(__float_as_int(nrm[t]), 0x118, 0xF, 0xF, true);
      sc[t] = best[t] + nrm[t] + __int_as_float(other);
    }
  }
  return sc;
}

// The moments (count, mean, M2) of every query head of group ug over its candidate
// slots [sink, n - window), computed by the whole workgroup from the K cache; the
// results go to s_mean / s_inv.  s_part: LDS scratch of kMaxGroup * 16 * 3 doubles.
// finalize_tile lends the histogram region (kBins words) to group_moments_direct
static_assert(kBins >= kMaxGroup * 16 * 3 * 2, "the histogram region holds the direct moments' scratch");

template <int D, int P, bool PAGED, bool MAXO>
__device__ inline void group_moments_direct(const ScoreArgs& a, int ug, int n, double* s_part, float* s_mean,
                                            float* s_inv) {
  using S = Shape<D>;
  constexpr int NB = S::NKC + 2 * S::NNC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int G = a.group;
  const int u = ug / a.hkv, g = ug % a.hkv;
  bf16x8 bdot[S::NKC], bna[S::NNC], bnb[S::NNC];
  u32x4 rref[S::NR];
  {
    const u32x4* bsrc = reinterpret_cast<const u32x4*>(a.B) + (size_t)ug * S::NBT * 64 + lane;
#pragma unroll
    for (int i = 0; i < S::NKC; ++i) bdot[i] = __builtin_bit_cast(bf16x8, bsrc[i * 64]);
#pragma unroll
    for (int i = 0; i < S::NNC; ++i) {
      bna[i] = __builtin_bit_cast(bf16x8, bsrc[(S::NKC + i) * 64]);
      bnb[i] = __builtin_bit_cast(bf16x8, bsrc[(S::NKC + S::NNC + i) * 64]);
    }
#pragma unroll
    for (int i = 0; i < S::NR; ++i) rref[i] = bsrc[(NB + i) * 64];
  }
  const int c0 = min(a.sink, n), c1 = max(c0, n - a.window);
  const bool owner = col >= 8 && col < 8 + G;
  double cnt = 0.0, mean = 0.0, m2 = 0.0;      // Welford, per owner lane
  for (int kb = c0 - c0 % 16 + 16 * wave; kb < c1; kb += 64) {
    u32x4 ch[D / 32];
    const int key = min(kb + col, n - 1);
    const uint16_t* rp;
    if (!PAGED) {
      rp = a.k.base + (int64_t)u * a.k.su + (int64_t)g * a.k.sh + (int64_t)key * a.k.ss;
    } else {
      const int b0 = a.k.bt[(int64_t)u * a.k.mb + key / a.k.bs];
      const int blk = b0 >= 0 && b0 < a.k.npb ? b0 : 0;
      rp = a.k.base + ((int64_t)blk * a.k.bs + key % a.k.bs) * a.k.ss + (int64_t)g * a.k.sh;
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) ch[i] = *reinterpret_cast<const u32x4*>(rp + chunk_elem<D>(i, grp));
    const f32x4 sc = block_scores<D, P, MAXO>(a, (size_t)ug, ch, bdot, bna, bnb, rref);
    if (owner) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = kb + 4 * grp + t;
        if (k >= c0 && k < c1) {
          const double x = (double)sc[t];
          cnt += 1.0;
          const double d = x - mean;
          mean += d / cnt;
          m2 += d * (x - mean);
        }
      }
    }
  }
  // partials [head][wave * 4 + grp], merged in that order
  if (owner) {
    double* q = s_part + ((col - 8) * 16 + wave * 4 + grp) * 3;
    q[0] = cnt;
    q[1] = mean;
    q[2] = m2;
  }
  __syncthreads();
  if ((int)threadIdx.x < G) {
    const int h = threadIdx.x;
    double c = 0.0, m = 0.0, mm = 0.0;
    for (int i = 0; i < 16; ++i) chan_merge(c, m, mm, s_part[(h * 16 + i) * 3], s_part[(h * 16 + i) * 3 + 1],
                                            s_part[(h * 16 + i) * 3 + 2]);
    const double var = c > 0.0 ? fmax(mm / c, 0.0) : 0.0;
    s_mean[h] = (float)(c > 0.0 ? m : 0.0);
    s_inv[h] = (float)(1.0 / fmax(sqrt(var), 1e-12));
  }
  __syncthreads();
}

// Waits until the group's last tile has published the merged moments of the (unit,
// KV head) of `ti` (tile_end), then z-normalises the tile's scores (still in LDS) per query head, aggregates the
// GQA group onto the KV head [Fold note, sec. 4: normalize-then-max; mean is the
// other variant] and writes the aggregate; protected slots (sinks, recent window)
// get +inf.
template <int D, int P, bool PAGED, bool MAXO>
__device__ inline void finalize_tile(const ScoreArgs& a, TileInfo ti, int n_known, const float* s_raw,
                                     uint32_t* s_hist) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = a.group;
  const int hq = a.hkv * G;
  const int RS = a.tile + 16;
  __shared__ float s_mean[kMaxGroup], s_inv[kMaxGroup];
  __shared__ int s_direct;   // a head's wait ran out: the group's moments are computed directly
  tile_len(a, ti, n_known >= 0 ? n_known : a.len[ti.u], false);
  // an empty tile (past its unit's length: claimed only when the units are not
  // listed) has no aggregates and no histogram counts, and must not wait: in a unit
  // of length 0 no tile publishes the group's moments
  if (ti.tlen == 0) return;
  if (threadIdx.x == 0) s_direct = a.wait_polls < 0;
  __syncthreads();

  // the group's mean and inverse standard deviation per query head, merged once by
  // the group's last tile (tile_end): wave 0 polls the G words until none reads
  // kUnpublished, at most a.wait_polls times
  if (wave == 0 && a.wait_polls >= 0) {
    const unsigned long long* p =
        reinterpret_cast<const unsigned long long*>(a.gstat + (size_t)ti.u * hq + ti.g * G);
    for (int polls = 0;; ++polls) {
      const unsigned long long w =
          lane < G ? __hip_atomic_load(p + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
      if (__ballot(w == kUnpublished) == 0) {
        if (lane < G) {
          s_mean[lane] = __uint_as_float((uint32_t)w);
          s_inv[lane] = __uint_as_float((uint32_t)(w >> 32));
        }
        break;
      }
      if (polls >= a.wait_polls) {
        if (lane == 0) s_direct = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  __syncthreads();
  if (s_direct) {
    // the histogram region is free until it is cleared below
    if (threadIdx.x == 0) raise_flag(a.flags, kFlagSync);
    group_moments_direct<D, P, PAGED, MAXO>(a, ti.ug, ti.n, reinterpret_cast<double*>(s_hist), s_mean, s_inv);
  }
  for (int i = threadIdx.x; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();

  const int tlen = ti.tlen, tile0 = ti.tile0, n = ti.n;
  float* dst = a.agg + ((size_t)ti.u * a.hkv + ti.g) * a.n_max + tile0;
  const float invg = 1.0f / (float)G;
  for (int i = 4 * threadIdx.x; i < tlen; i += 4 * 256) {
    f32x4 out;
#pragma unroll
    for (int t = 0; t < 4; ++t) out[t] = a.agg_mode == 0 ? 0.0f : -__builtin_inff();
    for (int h = 0; h < G; ++h) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(s_raw + h * RS + i);
      const float m = s_mean[h], inv = s_inv[h];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float z = (v[t] - m) * inv;
        out[t] = a.agg_mode == 0 ? out[t] + z : fmaxf(out[t], z);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = tile0 + i + t;
      if (a.agg_mode == 0) out[t] *= invg;
      if (key < a.sink || key >= n - a.window) out[t] = __builtin_inff();
    }
    if (i + 3 < tlen) {
      *reinterpret_cast<f32x4*>(dst + i) = out;
    } else {
      for (int t = 0; t < 4 && i + t < tlen; ++t) dst[i + t] = out[t];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (i + t < tlen) atomicAdd(&s_hist[lin_bin(out[t])], 1u);
  }
  // the tile's bins join the (unit, KV head) histogram the selection starts from
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)ti.ug * kBins;
  for (int i = threadIdx.x; i < kBins; i += 256) {
    const uint32_t c = s_hist[i];
    if (c) __hip_atomic_fetch_add(gh + i, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Block ids a score tile of `tile` slots can touch in a paged cache of block size bs.
__host__ __device__ inline int tile_pages(int tile, int bs) { return (tile + bs - 1) / bs + 1; }

// 32-bit words of the score kernel's LDS region shared by a tile's block ids (paged)
// and the finalisation's histogram (the mean over offsets only).
__host__ __device__ inline int score_scratch(bool omax, bool paged, int tile, int bs) {
  const int pages = paged ? tile_pages(tile, bs) : 0;
  return omax ? pages : (pages > kBins ? pages : kBins);
}

// Persistent score kernel: as many workgroups as fit on the device claim tiles in
// order from a counter.  Each workgroup scores and publishes its current tile, and
// only then finalises its previous one (two LDS score buffers): by that time the
// previous tile's group has nearly always published, so the moment exchange hides
// behind the streaming.  In the single-buffer mode (SINGLE, k_score_single; dense
// caches and the mean over offsets: every tile of the call resident at once, with
// tiles twice as long as two buffers would allow) each tile is finalised right after
// it is published; a workgroup then waits holding no unpublished tile.  With at most kListUnits units every workgroup first reads
// all lengths into LDS, and the claims run over the tiles that hold keys only (the
// tiles of a (unit, KV head) still consecutive); k_coef has published empty tiles'
// moments as zeros.  A workgroup waits only on tiles that are already
// claimed-and-published or claimed by running workgroups that publish before they
// wait; with P workgroups each holding at most two tiles, a circular wait would
// need 2P <= n_tiles, and P >= n_tiles (the host checks it), so the wait always ends
// (it is also bounded, and flagged, as a last resort).
//
// (Measured and dropped: claiming the next tile and issuing its first loads before
// the previous tile's finalisation, and two other key layouts over the waves: none
// changed the score kernel's time on the Qwen3-8B-shaped cache by more than 2 %, the
// first made it 2 % slower.)
template <int D, int P, bool PAGED, bool MAXO, bool SINGLE = false>
__device__ __forceinline__ void score_kernel(const ScoreArgs& a) {
  static_assert(!SINGLE || (!PAGED && !MAXO), "the single-buffer mode: dense caches, the mean over offsets");
  extern __shared__ float s_dyn[];
  __shared__ int s_t;
  __shared__ int s_bug;   // maximum over offsets: the (unit, KV head) whose offset blocks are staged
  const int G = a.group;
  const int RS = a.tile + 16;
  constexpr int nbuf = SINGLE ? 1 : 2;
  float* buf0 = s_dyn;
  float* buf1 = s_dyn + (nbuf - 1) * G * RS;
  // LDS after the two score buffers: one region for the tile's block ids (paged)
  // and the finalisation's histogram (they are never live together; the maximum over
  // offsets keeps the histogram in the staged offset blocks' region instead, restaged
  // after every finalisation), the units' lengths and tile prefix, the staged offset
  // blocks (the maximum over offsets)
  const int scratch = score_scratch(MAXO, PAGED, a.tile, a.k.bs);
  int* s_bt = reinterpret_cast<int*>(s_dyn + nbuf * G * RS);
  int* s_len = s_bt + scratch;            // [kListUnits] lengths
  int* s_pre = s_len + kListUnits;        // [kListUnits + 1] tiles of the units before
  const int used = nbuf * G * RS + scratch + 2 * kListUnits + 1;
  u32x4* s_bmax = reinterpret_cast<u32x4*>(s_dyn + ((used + 3) & ~3));   // 16-byte aligned
  uint32_t* s_hist = MAXO ? reinterpret_cast<uint32_t*>(s_bmax) : reinterpret_cast<uint32_t*>(s_bt);
  if (threadIdx.x == 0) s_bug = -1;
  const int U = a.n_units;
  const bool listed = U <= kListUnits;
  int total = U * a.hkv * a.n_tiles;
  if (listed) {
    // thread t takes units [2t, 2t + 2): lengths, then the prefix of their tiles
    __shared__ uint32_t wtot[4];
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = 2 * threadIdx.x + k;
      if (i < U) {
        const int n = fix_len(a.len[i], a.n_max, a.flags);
        s_len[i] = n;
        cnt += (uint32_t)((n + a.tile - 1) / a.tile * a.hkv);
      }
    }
    uint32_t run = block_scan_incl<256>(cnt, wtot) - cnt;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = 2 * threadIdx.x + k;
      if (i < U) {
        s_pre[i] = (int)run;
        run += (uint32_t)((s_len[i] + a.tile - 1) / a.tile * a.hkv);
      }
    }
    // the thread holding the last unit (or thread 0 when there is none) ends the prefix
    if ((2 * (int)threadIdx.x < U && 2 * (int)threadIdx.x + 2 >= U) || (U == 0 && threadIdx.x == 0))
      s_pre[U] = (int)run;
    __syncthreads();
    total = s_pre[U];
  }
  // claim index -> (unit x KV head, tile)
  auto place = [&](int t) {
    int ug, tile;
    if (!listed) {
      tile = t % a.n_tiles;
      ug = t / a.n_tiles;
    } else {
      int lo = 0, hi = U - 1;   // the last unit whose tiles start at or before t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const int r = t - s_pre[lo];
      const int nt = (s_len[lo] + a.tile - 1) / a.tile;
      ug = lo * a.hkv + r / nt;
      tile = r % nt;
    }
    return tile_info(a, ug, tile);
  };
  auto known_len = [&](const TileInfo& ti) { return listed ? s_len[ti.u] : -1; };

  TileRegs<D, MAXO> regs;
  TileInfo prev{};
  bool have_prev = false, b = false;
  for (;;) {
    if (threadIdx.x == 0) s_t = atomicAdd(a.next_tile, 1);
    __syncthreads();
    const int t = s_t;
    __syncthreads();
    TileInfo cur{};
    if (t < total) {
      cur = place(t);
      float* sbuf = b ? buf1 : buf0;
      tile_begin<D, P, PAGED, MAXO>(a, cur, known_len(cur), s_bt, regs);
      tile_body<D, P, PAGED, MAXO>(a, cur, sbuf, s_bt, s_bmax, &s_bug, regs);   // ends with a barrier
      tile_end<!MAXO>(a, cur, sbuf);
      if constexpr (SINGLE) {
        // one score buffer: the tile is finalised at once (its buffer is rewritten
        // only after the barrier of the next claim)
        finalize_tile<D, P, PAGED, MAXO>(a, cur, known_len(cur), sbuf, s_hist);
        continue;
      }
    }
    // finalize uses the histogram region (for the maximum over offsets, the staged
    // offset blocks' region, restaged for the next tile)
    if (have_prev) {
      finalize_tile<D, P, PAGED, MAXO>(a, prev, known_len(prev), b ? buf0 : buf1, s_hist);
      if (MAXO && threadIdx.x == 0) s_bug = -1;
    }
    if (t >= total) break;
    prev = cur;
    have_prev = true;
    b = !b;
  }
}

template <int D, int P, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_score(ScoreArgs a) {
  score_kernel<D, P, PAGED, false>(a);
}

// The single-buffer mode of the mean over offsets (dense caches; see score_kernel).
template <int D, int P>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_score_single(ScoreArgs a) {
  score_kernel<D, P, false, false, true>(a);
}

// The maximum over offsets: two workgroups per CU when LDS allows (G <= 4), so at
// most 256 registers a lane.
template <int D, int P, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_score_max(ScoreArgs a) {
  score_kernel<D, P, PAGED, true>(a);
}

// ============================================================================ selection
// tria_select keeps, per (unit, KV head), the K = min(B, n) slots with the largest
// aggregates (ties to the lower slot), in four steps; the two tile-parallel steps
// carry all the per-slot work, the per-group steps touch only histograms, a short
// candidate list and per-tile counts:
//   k_sel_thresh  (per group, one wave) the histogram of the aggregates' linear
//                 bins, built by k_score, gives the bin b1 holding the K-th largest;
//                 the binning is monotone, so every slot in a higher bin is kept and
//                 every slot in a lower bin dropped;
//   k_sel_collect (per tile)  counts the tile's slots above b1 and lists its slots of
//                 b1 in the tile's own segment of the group's candidate list;
//   k_sel_refine  (per group) exact radix passes (11 + 11 + 10 bits of the
//                 order-preserving key; a digit all candidates share is skipped)
//                 over the candidates, or for at most kSelRankMax candidates each
//                 one's rank among them, give the threshold key T
//                 and how many slots equal to T are kept (the lowest ones); clears
//                 the dropped candidates from the tiles' candidate masks; then each
//                 tile's output offset;
//   k_sel_emit    (per tile)  writes the tile's kept slots (its masks) in ascending order.
__device__ inline uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);  // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The bin whose cumulative count from the top first reaches krem (1 <= krem <=
// total), and the count strictly above it.
template <int NT>
__device__ inline void find_digit(const uint32_t* hist, int nb, uint32_t krem, uint32_t* wtot, uint32_t* sh,
                                  uint32_t& digit, uint32_t& above) {
  const int c = (nb + NT - 1) / NT;
  const int top = nb - 1 - (int)threadIdx.x * c;  // this thread's bins: top, top-1, ..., top-c+1
  uint32_t local = 0;
  for (int i = 0; i < c; ++i)
    if (top - i >= 0) local += hist[top - i];
  const uint32_t incl = block_scan_incl<NT>(local, wtot);
  const uint32_t excl = incl - local;
  if (excl < krem && krem <= incl) {
    uint32_t acc = excl;
    for (int i = 0; i < c && top - i >= 0; ++i) {
      const uint32_t h = hist[top - i];
      if (acc + h >= krem) {
        sh[0] = (uint32_t)(top - i);
        sh[1] = acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
  digit = sh[0];
  above = sh[1];
  __syncthreads();
}

// The selection's bounds for group ug: n cached slots, K kept, and the bin b1
// holding the K-th largest aggregate (-1: keep everything; kBins: keep nothing) with
// krem slots still to take from it.  Formed by one wave from the group's kBins bins
// (`bins`: a copy in LDS, or the histogram itself), every lane returning the same
// values: lane l holds the kSelPL consecutive bins from kSelPL l, an inclusive scan
// from the top lane down gives each lane the count in its bins and above, the lane
// where that count first reaches K walks its own bins from the top.  A histogram
// holding fewer than K slots (len changed since tria_score, outside the contract)
// gives b1 = -1: the first K slots are kept.  `lead` raises the group's flags.
constexpr int kSelPL = (kBins + 63) / 64;
struct SelBounds {
  int n, K, b1;
  uint32_t krem;
};

__device__ inline SelBounds sel_bounds(const SelectArgs& a, const uint32_t* bins, int u, bool lead) {
  const int lane = threadIdx.x & 63;
  uint32_t h[kSelPL];
#pragma unroll
  for (int i = 0; i < kSelPL; ++i) h[i] = kSelPL * lane + i < kBins ? bins[kSelPL * lane + i] : 0u;
  int32_t* flags = lead && lane == 0 ? a.flags : nullptr;
  SelBounds r;
  r.n = clamp_len(a.len, u, a.n_max, flags);
  int B = a.budget[u];
  const int prot = min(r.n, a.sink + a.window);
  if (B < 0 || (r.n > B && B < prot)) {
    if (flags) raise_flag(flags, kFlagBudget);
    B = B < 0 ? 0 : B;
  }
  r.K = B < r.n ? B : r.n;
  if (r.K > a.b_max) {
    if (flags) raise_flag(flags, kFlagBmax);
    r.K = a.b_max;
  }
  r.krem = 0;
  if (r.K == 0) {
    r.b1 = kBins;
  } else if (r.K >= r.n) {
    r.b1 = -1;
  } else {
    const uint32_t K = (uint32_t)r.K;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < kSelPL; ++i) local += h[i];
    uint32_t incl = local;   // slots in the bins of this lane and every lane above it
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_down(incl, o);
      if (lane + o < 64) incl += v;
    }
    const uint32_t excl = incl - local;
    const bool mine = excl < K && K <= incl;
    int bin = 0;
    uint32_t above = 0, acc = excl;
    bool done = false;
#pragma unroll
    for (int i = kSelPL - 1; i >= 0; --i) {
      const bool hit = mine && !done && acc + h[i] >= K;
      if (hit) {
        bin = kSelPL * lane + i;
        above = acc;
      }
      done |= hit;
      acc += h[i];
    }
    const unsigned long long m = __ballot(mine);
    if (m == 0) {
      r.b1 = -1;
    } else {
      const int src = __ffsll((long long)m) - 1;
      r.b1 = __shfl(bin, src);
      r.krem = K - (uint32_t)__shfl((int)above, src);
    }
  }
  return r;
}

// Writes the group's selection state (and cnt[u] from KV head 0).
__device__ inline void put_bounds(const SelectArgs& a, int ug, int u, int g, const SelBounds& r) {
  SelState& st = a.st[ug];
  st.b1 = r.b1;
  st.krem = (int32_t)r.krem;
  st.K = r.K;
  st.n = r.n;
  st.m = 0;
  st.T = 0;
  st.keq = 0;
  if (g == 0) a.cnt[u] = r.K;
}

// One wave per group: the histogram, loaded coalesced into LDS (every load in
// flight at once), then the bounds, recorded for the other selection kernels.
__global__ __launch_bounds__(64) void k_sel_thresh(SelectArgs a) {
  constexpr int NL = (kBins + 63) / 64;
  const int ug = blockIdx.x;
  const int u = ug / a.hkv, g = ug % a.hkv;
  const int lane = threadIdx.x;
  __shared__ uint32_t s_bins[kBins];
  {
    const uint32_t* gh = a.hist + (size_t)ug * kBins;
    uint32_t hb[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) hb[i] = lane + 64 * i < kBins ? gh[lane + 64 * i] : 0u;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (lane + 64 * i < kBins) s_bins[lane + 64 * i] = hb[i];
  }
  __syncthreads();
  const SelBounds r = sel_bounds(a, s_bins, u, g == 0);
  if (lane == 0) put_bounds(a, ug, u, g, r);
}

// A selection tile's slots per thread: thread t takes the kSelTile / 256 consecutive
// slots from s0 = tile0 + t kSelTile / 256.
constexpr int kSelSpt = kSelTile / 256;
static_assert(kSelSpt % 4 == 0 && kSelSpt <= 32, "slots per thread: whole 16-byte loads, one 32-bit mask");

// Loads the slots [s0, s0 + kSelSpt) of a row with 16-byte loads, each clamped inside
// the row (n_max is a multiple of 16): values of slots at or past n_max are garbage
// and never used.
__device__ inline void load_slots(const float* row, int s0, int n_max, float (&x)[kSelSpt]) {
#pragma unroll
  for (int i = 0; i < kSelSpt / 4; ++i) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + min(s0 + 4 * i, n_max - 4));
#pragma unroll
    for (int t = 0; t < 4; ++t) x[4 * i + t] = v[t];
  }
}

__global__ __launch_bounds__(256) void k_sel_collect(SelectArgs a) {
  const int ug = blockIdx.x / a.n_st;
  const int j = blockIdx.x % a.n_st;
  const int tid = threadIdx.x;
  __shared__ uint32_t wtot[4];
  // the tile's aggregates and the group's bounds, together
  const int s0 = j * kSelTile + kSelSpt * tid;
  float x[kSelSpt];
  load_slots(a.agg + (size_t)ug * a.n_max, s0, a.n_max, x);
  const SelState bd = a.st[ug];
  const int b1 = bd.b1, n = bd.n;
  uint32_t gm = 0, cmk = 0;   // per-slot bits: above b1, in b1
#pragma unroll
  for (int k = 0; k < kSelSpt; ++k) {
    if (s0 + k < n) {
      const int bin = lin_bin(x[k]);
      gm |= (bin > b1 ? 1u : 0u) << k;
      cmk |= (bin == b1 ? 1u : 0u) << k;
    }
  }
  // the masks, for k_sel_emit (which then reads the aggregates of candidates only)
  a.gmask[(size_t)blockIdx.x * 256 + tid] = (SelMask)gm;
  a.cmask[(size_t)blockIdx.x * 256 + tid] = (SelMask)cmk;
  const uint32_t cm = (uint32_t)__popc(cmk);
  const uint32_t gt_tot = block_scan_incl<256>((uint32_t)__popc(gm), wtot);
  const uint32_t m_incl = block_scan_incl<256>(cm, wtot);
  if (tid == 255) {
    a.tile_gt[blockIdx.x] = (int32_t)gt_tot;
    a.tile_m[blockIdx.x] = (int32_t)m_incl;
  }
  // this tile's candidates, in slot order, at the start of its segment
  // [j kSelTile, (j + 1) kSelTile) of the group's list
  if (cm) {
    int32_t* list = a.list + (size_t)ug * a.n_max + (size_t)j * kSelTile;
    uint32_t pos = m_incl - cm;
    for (uint32_t m = cmk; m; m &= m - 1) list[pos++] = s0 + __ffs(m) - 1;
  }
}

// Clears the candidate-mask bit of `slot` (a candidate the refinement drops).  Masks
// narrower than 32 bits are cleared through the aligned 32-bit word that holds them
// (the four threads' masks of one word belong to the same tile).
__device__ inline void drop_candidate(const SelectArgs& a, int ug, int slot) {
  constexpr int PW = 4 / (int)sizeof(SelMask);   // masks per 32-bit word
  const int j = slot / kSelTile, local = slot - j * kSelTile;
  const size_t e = ((size_t)ug * a.n_st + j) * 256 + local / kSelSpt;
  uint32_t* w = reinterpret_cast<uint32_t*>(a.cmask) + e / PW;
  atomicAnd(w, ~(1u << ((int)(e % PW) * 8 * (int)sizeof(SelMask) + local % kSelSpt)));
}

__global__ __launch_bounds__(512) void k_sel_refine(SelectArgs a) {
  const int ug = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = a.agg + (size_t)ug * a.n_max;
  const int32_t* list = a.list + (size_t)ug * a.n_max;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wtot[8];
  __shared__ uint32_t sh[2];
  __shared__ int32_t s_gtb[kMaxSelTiles], s_eqc[kMaxSelTiles];
  __shared__ int32_t s_pre[kMaxSelTiles + 1];   // candidates before each tile's segment
  __shared__ __attribute__((aligned(16))) uint32_t s_key[kRefineLds];   // candidates' order keys and slots, when
  __shared__ int32_t s_slot[kRefineLds];        // they fit (else read again per pass)

  const SelState bd = a.st[ug];
  // candidate i lives in tile seg(i)'s segment, at position i - s_pre[seg(i)]
  {
    const int per = (a.n_st + 511) / 512;   // consecutive tiles per thread
    const int t0 = tid * per;
    int32_t c[4] = {0, 0, 0, 0};            // per <= kMaxSelTiles / 512 = 4
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < per && t0 + i < a.n_st) {
        c[i] = a.tile_m[(size_t)ug * a.n_st + t0 + i];
        local += (uint32_t)c[i];
      }
    uint32_t run = block_scan_incl<512>(local, wtot) - local;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < per && t0 + i < a.n_st) {
        s_pre[t0 + i] = (int32_t)run;
        run += (uint32_t)c[i];
      }
    if (t0 < a.n_st && t0 + per >= a.n_st) s_pre[a.n_st] = (int32_t)run;   // the thread with the last tile
    if (a.n_st == 0 && tid == 0) s_pre[0] = 0;
  }
  __syncthreads();
  const int m = s_pre[a.n_st];
  auto cand = [&](int i) {
    int lo = 0, hi = a.n_st - 1;   // the last tile whose segment starts at or before i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return list[(size_t)lo * kSelTile + (i - s_pre[lo])];
  };

  uint32_t T = 0, keq = 0;
  const bool refine = bd.b1 >= 0 && bd.b1 < kBins;
  // candidate i's slot and key: from LDS when all fit, else from the list and agg
  const bool staged = m <= kRefineLds;
  if (refine && staged) {
    for (int i = tid; i < m; i += 512) {
      const int slot = cand(i);
      s_slot[i] = slot;
      s_key[i] = order_key(row[slot]);
    }
  }
  __syncthreads();
  auto cand_slot = [&](int i) { return staged ? s_slot[i] : cand(i); };
  auto cand_key = [&](int i) { return staged ? s_key[i] : order_key(row[cand(i)]); };
  if (refine && staged && m <= kSelRankMax) {
    // few candidates: candidate i's key is the threshold T when fewer than krem keys
    // lie above it and at least krem at or above it; keq = krem - (keys above T).
    // (No candidate qualifies only for a histogram inconsistent with the scores:
    // T = 0, keq = 0 then.)
    __shared__ uint32_t s_tk[2];
    if (tid == 0) s_tk[0] = s_tk[1] = 0u;
    __syncthreads();
    const uint32_t krem = (uint32_t)bd.krem;
    if (tid < m) {
      const uint32_t k = s_key[tid];
      uint32_t gt = 0, ge = 0;
      const int m4 = m & ~3;
#pragma unroll 4
      for (int i = 0; i < m4; i += 4) {   // every lane reads the same 16 bytes: a broadcast
        const u32x4 o = *reinterpret_cast<const u32x4*>(s_key + i);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          gt += o[t] > k ? 1u : 0u;
          ge += o[t] >= k ? 1u : 0u;
        }
      }
      for (int i = m4; i < m; ++i) {
        gt += s_key[i] > k ? 1u : 0u;
        ge += s_key[i] >= k ? 1u : 0u;
      }
      if (gt < krem && krem <= ge) {   // every such candidate holds the same key
        s_tk[0] = k;
        s_tk[1] = krem - gt;
      }
    }
    __syncthreads();
    T = s_tk[0];
    keq = s_tk[1];
  } else if (refine) {
    // the bits every candidate shares (AND and OR of the keys): a digit made of such
    // bits needs no pass, since every candidate holds it and none lies above it (the
    // candidates share a linear bin, so usually the sign, the exponent and the top of
    // the mantissa: the whole first digit)
    __shared__ uint32_t s_and[8], s_or[8];
    uint32_t ka = ~0u, ko = 0u;
    for (int i = tid; i < m; i += 512) {
      const uint32_t key = cand_key(i);
      ka &= key;
      ko |= key;
    }
    for (int o = 32; o > 0; o >>= 1) {
      ka &= __shfl_xor(ka, o);
      ko |= __shfl_xor(ko, o);
    }
    if ((tid & 63) == 0) {
      s_and[tid >> 6] = ka;
      s_or[tid >> 6] = ko;
    }
    __syncthreads();
    ka = ~0u;
    ko = 0u;
    for (int w = 0; w < 8; ++w) {
      ka &= s_and[w];
      ko |= s_or[w];
    }
    const uint32_t common = ~(ka ^ ko);
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)bd.krem;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int sft = pass == 0 ? 21 : (pass == 1 ? 10 : 0);   // digits of 11, 11, 10 bits
      const int nb = pass == 2 ? 1024 : 2048;
      const uint32_t dmask = (uint32_t)(nb - 1) << sft;
      if ((common & dmask) == dmask) {   // the same for every thread
        prefix |= ka & dmask;
        pmask |= dmask;
        continue;
      }
      for (int i = tid; i < nb; i += 512) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < m; i += 512) {
        const uint32_t key = cand_key(i);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sft) & (nb - 1)], 1u);
      }
      __syncthreads();
      uint32_t d, ab;
      find_digit<512>(hist, nb, krem, wtot, sh, d, ab);
      prefix |= d << sft;
      pmask |= (uint32_t)(nb - 1) << sft;
      krem -= ab;
    }
    T = prefix;
    keq = krem;
  }
  // per tile: candidates above T and equal to T; and each candidate's fate for the
  // emission: kept above T, or among the lowest keq slots equal to T (the list holds
  // the candidates in slot order, so a tied candidate's rank is the number of tied
  // ones before it in the list, counted in chunks of 512); the others are dropped
  // from the candidate masks
  __shared__ uint32_t s_run;   // tied candidates in the chunks before
  for (int i = tid; i < a.n_st; i += 512) {
    s_gtb[i] = 0;
    s_eqc[i] = 0;
  }
  if (tid == 0) s_run = 0;
  __syncthreads();
  if (refine) {
    for (int c0 = 0; c0 < m; c0 += 512) {
      const int i = c0 + tid;
      const bool in = i < m;
      const int slot = in ? cand_slot(i) : 0;
      const uint32_t key = in ? cand_key(i) : 0u;
      const bool gt = in && key > T, eq = in && key == T;
      if (gt) atomicAdd(&s_gtb[slot / kSelTile], 1);
      else if (eq) atomicAdd(&s_eqc[slot / kSelTile], 1);
      const uint32_t f = eq ? 1u : 0u;
      const uint32_t incl = block_scan_incl<512>(f, wtot);
      const uint32_t rank = s_run + incl - f;
      if (in && !gt && !(eq && rank < keq)) drop_candidate(a, ug, slot);
      __syncthreads();   // every thread has read s_run
      if (tid == 511) s_run += incl;
      __syncthreads();
    }
  }
  __syncthreads();
  // tied slots are kept lowest first: tile j keeps min(eq_j, keq - eq before j);
  // output offsets are the prefix sums of the tiles' kept counts
  const int per = (a.n_st + 511) / 512;
  const int j0 = tid * per;
  uint32_t eq_local = 0;
  for (int i = 0; i < per && j0 + i < a.n_st; ++i) eq_local += (uint32_t)s_eqc[j0 + i];
  uint32_t eq_before = block_scan_incl<512>(eq_local, wtot) - eq_local;
  uint32_t kept_local[1] = {0};
  // first sweep: kept counts (needs eq_before per tile)
  uint32_t eb = eq_before;
  for (int i = 0; i < per && j0 + i < a.n_st; ++i) {
    const int jj = j0 + i;
    const uint32_t e = (uint32_t)s_eqc[jj];
    const uint32_t share = eb >= keq ? 0u : min(e, keq - eb);
    eb += e;
    kept_local[0] += (uint32_t)a.tile_gt[(size_t)ug * a.n_st + jj] + (uint32_t)s_gtb[jj] + share;
  }
  uint32_t off = block_scan_incl<512>(kept_local[0], wtot) - kept_local[0];
  eb = eq_before;
  for (int i = 0; i < per && j0 + i < a.n_st; ++i) {
    const int jj = j0 + i;
    const uint32_t e = (uint32_t)s_eqc[jj];
    const uint32_t share = eb >= keq ? 0u : min(e, keq - eb);
    eb += e;
    a.tile_off[(size_t)ug * a.n_st + jj] = (int32_t)off;
    off += (uint32_t)a.tile_gt[(size_t)ug * a.n_st + jj] + (uint32_t)s_gtb[jj] + share;
  }
  if (tid == 0) {
    a.st[ug].m = m;
    a.st[ug].T = (int32_t)T;
    a.st[ug].keq = (int32_t)keq;
  }
  int32_t* out = a.idx + (size_t)ug * a.b_max;
  for (int i = bd.K + tid; i < a.b_max; i += 512) out[i] = -1;
}

__global__ __launch_bounds__(256) void k_sel_emit(SelectArgs a) {
  const int ug = blockIdx.x / a.n_st;
  const int tid = threadIdx.x;
  __shared__ uint32_t wtot[4];
  __shared__ uint32_t s_cnt;
  __shared__ int32_t s_out[kSelTile];   // the tile's kept slots, in order
  // every load at once: the thread's kept slots (above b1 from k_sel_collect, and the
  // candidates k_sel_refine kept), the group's counts and the tile's offset
  const int s0 = (blockIdx.x % a.n_st) * kSelTile + kSelSpt * tid;
  const uint32_t keep = (uint32_t)a.gmask[(size_t)blockIdx.x * 256 + tid] |
                        (uint32_t)a.cmask[(size_t)blockIdx.x * 256 + tid];
  const SelState st = a.st[ug];
  const uint32_t K = (uint32_t)st.K;
  const uint32_t off = (uint32_t)a.tile_off[blockIdx.x];
  const uint32_t nk = (uint32_t)__popc(keep);
  const uint32_t incl = block_scan_incl<256>(nk, wtot);
  uint32_t pos = incl - nk;
  int32_t* out = a.idx + (size_t)ug * a.b_max + off;
  // The run's places are < K by construction; the bounds keep a miscount from ever
  // writing past the caller's b_max row.  Where more than one slot in eight is kept,
  // the run goes through LDS and out with coalesced stores (each thread's own
  // stores would spread over many lines); sparser runs are written directly.
  if ((int64_t)st.K * 8 > (int64_t)st.n) {   // the same for the whole workgroup
    for (uint32_t m = keep; m; m &= m - 1) s_out[pos++] = s0 + __ffs(m) - 1;
    if (tid == 255) s_cnt = incl;
    __syncthreads();
    const uint32_t lim = off < K ? min(s_cnt, K - off) : 0u;
    for (uint32_t i = tid; i < lim; i += 256) out[i] = s_out[i];
  } else {
    for (uint32_t m = keep; m; m &= m - 1) {
      if (off + pos < K) out[pos] = s0 + __ffs(m) - 1;
      ++pos;
    }
  }
}

// ---------------------------------------------------------------------------- per group
// The whole selection of one (unit, KV head) in one workgroup of 512 threads, for
// rows of at most kSelGroupMax slots: thread t holds the aggregates of the 64
// consecutive slots [64 t, 64 t + 64) in registers.  The histogram built by k_score
// gives b1 and krem (sel_bounds); three radix passes run straight over the
// thread's values of bin b1 (no candidate list); then per-thread counts of kept and
// tied slots, two block scans, and the thread writes its kept slots in order.  Ties
// at the threshold key are kept lowest slot first, as in the tile-parallel kernels.
// Makes the compiler treat the values as changed, so that keys and bins are formed
// again in each pass instead of being kept in 64 more registers per thread.
template <int N>
__device__ inline void opaque(float (&x)[N]) {
#pragma unroll
  for (int v = 0; v < N; ++v) asm volatile("" : "+v"(x[v]));
}

__global__ __launch_bounds__(512) void k_sel_group(SelectArgs a) {
  constexpr int NT = 512, VPT = 64;
  const int ug = blockIdx.x;
  const int u = ug / a.hkv, g = ug % a.hkv;
  const int tid = threadIdx.x;
  __shared__ uint32_t hist[2048];   // radix digits
  __shared__ uint32_t wtot[NT / 64];
  __shared__ uint32_t sh[2];
  __shared__ SelBounds s_bd;

  // the thread's values, loaded first (16-byte loads, clamped inside the row)
  const float* row = a.agg + (size_t)ug * a.n_max;
  const int s_lo = tid * VPT;
  float x[VPT];
#pragma unroll
  for (int i = 0; i < VPT / 4; ++i) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + min(s_lo + 4 * i, a.n_max - 4));
#pragma unroll
    for (int t = 0; t < 4; ++t) x[4 * i + t] = v[t];
  }

  // bounds (wave 0): n cached slots, K kept, the bin b1 of the K-th largest
  if (tid < 64) {
    const SelBounds r = sel_bounds(a, a.hist + (size_t)ug * kBins, u, g == 0);
    if (tid == 0) {
      s_bd = r;
      if (g == 0) a.cnt[u] = r.K;
    }
  }
  __syncthreads();
  const int n = s_bd.n, K = s_bd.K, b1 = s_bd.b1;

  // the threshold: every slot of a bin above b1 is kept; in bin b1, keys above T and
  // the lowest keq slots equal to T
  uint32_t T = 0, keq = 0;
  if (b1 >= 0 && b1 < kBins) {
    uint32_t krem = s_bd.krem;
    uint32_t prefix = 0, pmask = 0;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int sft = pass == 0 ? 21 : (pass == 1 ? 10 : 0);   // digits of 11, 11, 10 bits
      const int nb = pass == 2 ? 1024 : 2048;
      for (int i = tid; i < nb; i += NT) hist[i] = 0;
      __syncthreads();
      opaque(x);
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        const uint32_t key = order_key(x[v]);
        if (s_lo + v < n && lin_bin(x[v]) == b1 && (key & pmask) == prefix)
          atomicAdd(&hist[(key >> sft) & (nb - 1)], 1u);
      }
      __syncthreads();
      uint32_t dd, ab;
      find_digit<NT>(hist, nb, krem, wtot, sh, dd, ab);
      prefix |= dd << sft;
      pmask |= (uint32_t)(nb - 1) << sft;
      krem -= ab;
    }
    T = prefix;
    keq = krem;
  }

  // kept and tied slots of this thread (bit v: slot s_lo + v)
  opaque(x);
  uint64_t keep = 0, eq = 0;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int bin = lin_bin(x[v]);
    const uint32_t key = order_key(x[v]);
    const bool in = s_lo + v < n;
    const bool gt = bin > b1 || (bin == b1 && key > T);
    keep |= (uint64_t)(in && gt) << v;
    eq |= (uint64_t)(in && bin == b1 && key == T) << v;
  }
  const uint32_t ne = (uint32_t)__popcll(eq);
  uint32_t r = block_scan_incl<NT>(ne, wtot) - ne;   // tied slots in lower slots
  for (uint64_t m = eq; m; m &= m - 1) {
    if (r < keq) keep |= m & (~m + 1);
    ++r;
  }
  const uint32_t nk = (uint32_t)__popcll(keep);
  uint32_t pos = block_scan_incl<NT>(nk, wtot) - nk;
  int32_t* out = a.idx + (size_t)ug * a.b_max;
  for (uint64_t m = keep; m; m &= m - 1) {
    // positions are < K by construction; the bound keeps a miscount from ever
    // writing past the caller's b_max row
    if (pos < (uint32_t)K) out[pos] = s_lo + __ffsll((unsigned long long)m) - 1;
    ++pos;
  }
  for (int i = K + tid; i < a.b_max; i += NT) out[i] = -1;
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
      __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks) + part),
                                  reinterpret_cast<u32x4*>(kd) + part);
    if (vs && vd)
      __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs) + part),
                                  reinterpret_cast<u32x4*>(vd) + part);
    if (part == 0 && a.pos_src && a.pos_dst) {
      const int ph = a.pos_heads > 1 ? g : 0;
      a.pos_dst[((size_t)u * a.hkv + g) * a.b_max + j] =
          a.pos_src[((size_t)u * a.pos_heads + ph) * a.n_max + slot];
    }
  }
}

}  // namespace

// Fast compaction for the common layouts: K and V sources both dense, or both paged
// through one block table (likewise the destinations).  A thread copies 16 bytes of R rows; all of a step's loads
// are issued before any is used, so a workgroup's 64 rows take one round trip for
// the indices (and destination block ids), one for the source block ids and
// positions (paged sources), and one for the rows.  Every load is unconditional:
// rows past the count and invalid slots or block ids read a clamped, existing
// address and are not stored.  The rows are loaded and stored non-temporally (both
// compaction kernels): they are touched once, and dirty lines left in the caches would
// otherwise be written back while the next pass's score kernel streams the cache.
template <int D, bool SP, bool DP>
__global__ __launch_bounds__(256) void k_compact_fast(CompactArgs a) {
  constexpr int LPR = D / 8;                // lanes per row, 16 bytes each
  constexpr int RPP = 256 / LPR;            // rows per pass
  constexpr int R = kCompactRows / RPP;     // rows per thread
  const int rt = blockIdx.x % a.n_rtiles;
  const int ug = blockIdx.x / a.n_rtiles;
  const int u = ug / a.hkv, g = ug % a.hkv;
  int K = a.cnt[u];
  K = K < 0 ? 0 : (K > a.b_max ? a.b_max : K);
  int n = a.len[u];
  n = n < 0 ? 0 : (n > a.n_max ? a.n_max : n);
  const int j0 = rt * kCompactRows;
  if (j0 >= K) return;
  const int part = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
  const int32_t* ix = a.idx + (size_t)ug * a.b_max;
  const int ph = a.pos_heads > 1 ? g : 0;
  // without positions the (ignored) position loads read idx[0] of this row
  const int32_t* psrc = a.pos_src ? a.pos_src + ((size_t)u * a.pos_heads + ph) * a.n_max : ix;
  const int pmask = a.pos_src ? -1 : 0;

  // step 1: kept slots and destination block ids
  int slot[R], dblk[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int j = min(j0 + r0 + k * RPP, K - 1);
    slot[k] = ix[j];
    if (DP) dblk[k] = a.kd.bt[(int64_t)u * a.kd.mb + j / a.kd.bs];
  }
  // step 2: validity, source block ids, positions
  bool ok[R];
  int sblk[R], pos[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const bool in = j0 + r0 + k * RPP < K;
    const bool valid = slot[k] >= 0 && slot[k] < n;
    if (in && !valid && part == 0) raise_flag(a.flags, kFlagIndex);
    ok[k] = in && valid;
    slot[k] = valid ? slot[k] : 0;
    if (SP) sblk[k] = a.ks.bt[(int64_t)u * a.ks.mb + slot[k] / a.ks.bs];
    pos[k] = psrc[slot[k] & pmask];
  }
  // step 3: the rows
  u32x4 kv[R], vv[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    int64_t ko, vo;
    if (SP) {
      const bool bad = sblk[k] < 0 || sblk[k] >= a.ks.npb;
      if (ok[k] && bad && part == 0) raise_flag(a.flags, kFlagBlock);
      ok[k] = ok[k] && !bad;
      const int64_t b = bad ? 0 : sblk[k];
      ko = (b * a.ks.bs + slot[k] % a.ks.bs) * a.ks.ss + (int64_t)g * a.ks.sh;
      vo = (b * a.vs.bs + slot[k] % a.vs.bs) * a.vs.ss + (int64_t)g * a.vs.sh;
    } else {
      ko = (int64_t)u * a.ks.su + (int64_t)g * a.ks.sh + (int64_t)slot[k] * a.ks.ss;
      vo = (int64_t)u * a.vs.su + (int64_t)g * a.vs.sh + (int64_t)slot[k] * a.vs.ss;
    }
    kv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.ks.base + ko) + part);
    vv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vs.base + vo) + part);
  }
  // step 4: stores
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int j = j0 + r0 + k * RPP;
    int64_t ko, vo;
    bool okd = ok[k];
    if (DP) {
      const bool bad = dblk[k] < 0 || dblk[k] >= a.kd.npb;
      if (okd && bad && part == 0) raise_flag(a.flags, kFlagBlock);
      okd = okd && !bad;
      ko = ((int64_t)dblk[k] * a.kd.bs + j % a.kd.bs) * a.kd.ss + (int64_t)g * a.kd.sh;
      vo = ((int64_t)dblk[k] * a.vd.bs + j % a.vd.bs) * a.vd.ss + (int64_t)g * a.vd.sh;
    } else {
      ko = (int64_t)u * a.kd.su + (int64_t)g * a.kd.sh + (int64_t)j * a.kd.ss;
      vo = (int64_t)u * a.vd.su + (int64_t)g * a.vd.sh + (int64_t)j * a.vd.ss;
    }
    if (okd) {
      __builtin_nontemporal_store(kv[k], reinterpret_cast<u32x4*>(a.kd.base + ko) + part);
      __builtin_nontemporal_store(vv[k], reinterpret_cast<u32x4*>(a.vd.base + vo) + part);
      if (part == 0 && a.pos_src && a.pos_dst) a.pos_dst[(size_t)ug * a.b_max + j] = pos[k];
    }
  }
}

// ============================================================================ calibration
// tria_calibrate: per (layer, query head, band) means of Re q_f, Im q_f, |q_f| and of
// the unit phasor q_f / |q_f| over a stream of pre-RoPE query rows [Calib issue,
// "How it works"].  k_calib: workgroup (chunk, layer x head) sums kCalibChunk rows in
// fp32.  Lane p of a row owns bands 8p .. 8p + 7 and loads both parts of them itself:
// in NEOX rows the real parts at elements [8p, 8p + 8) and the imaginary parts d/2
// further on, in interleaved rows the 16 elements [16p, 16p + 16).  The next rows'
// loads are issued before the current rows' sums.  k_calib_final adds the chunks in
// fp64, in chunk order, and divides.

// Adds one band's contributions: re, im, |q|, re / |q|, im / |q| (0, 0 for q = 0).
// The band is scaled by a power of two to a magnitude in [0.5, 1) before squaring, so
// that no finite bf16 value overflows or loses precision to underflow; one reciprocal
// square root (1 ulp) then gives both |q| and the unit phasor.  A nonzero m2 lies in
// [0.25, 2), where adding 2^-100 changes nothing; for q = 0 the addition keeps the
// reciprocal square root finite and every contribution 0.
__device__ inline void calib_band(float re, float im, float (&acc)[5]) {
  const int e = __builtin_amdgcn_frexp_expf(fabsf(re) > fabsf(im) ? re : im);   // of the larger part
  const float a = __builtin_amdgcn_ldexpf(re, -e), b = __builtin_amdgcn_ldexpf(im, -e);
  const float m2 = fmaf(a, a, b * b);                      // in [0.25, 2), or 0
  const float r = __builtin_amdgcn_rsqf(m2 + 0x1p-100f);
  acc[0] += re;
  acc[1] += im;
  acc[2] += __builtin_amdgcn_ldexpf(m2 * r, e);
  acc[3] = fmaf(a, r, acc[3]);
  acc[4] = fmaf(b, r, acc[4]);
}

// A lane's rows of one chunk: t0, t0 + RPP, ... (NR of them), in batches of NB whose
// loads are issued one batch ahead of the sums.  FULL: every row exists.  Otherwise
// rows at or past t1 load row t1 - 1 (a valid address) and count as zero.
template <int D, int P, int NR, int NB, int RPP, bool FULL>
__device__ inline void calib_rows(const uint16_t* base, int64_t st, int t0, int t1, int e0, int e1,
                                  float (&acc)[8][5]) {
  auto load = [&](u32x4 (&w)[NB][2], int b) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int t = t0 + (b + j) * RPP;
      const uint16_t* row = base + (int64_t)(FULL ? t : min(t, t1 - 1)) * st;
      w[j][0] = *reinterpret_cast<const u32x4*>(row + e0);
      w[j][1] = *reinterpret_cast<const u32x4*>(row + e1);
    }
    // keep the batch's loads ahead of the previous batch's sums
    __builtin_amdgcn_sched_barrier(0);
  };
  auto sums = [&](const u32x4 (&w)[NB][2], int b) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool live = FULL || t0 + (b + j) * RPP < t1;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t wr, wi;
        bool hi;
        if (P == 0) {      // real parts in piece 0, imaginary parts in piece 1
          wr = w[j][0][k / 2];
          wi = w[j][1][k / 2];
          hi = k & 1;
        } else {           // (re, im) pairs, four per piece
          wr = wi = w[j][k / 4][k % 4];
          hi = false;
        }
        if (!FULL) {
          wr = live ? wr : 0u;
          wi = live ? wi : 0u;
        }
        const float re = hi ? bf_hi(wr) : bf_lo(wr);
        const float im = (P == 0 && !hi) ? bf_lo(wi) : bf_hi(wi);
        calib_band(re, im, acc[k]);
      }
    }
  };
  static_assert(NR % (2 * NB) == 0, "rows per lane");
  u32x4 wa[NB][2], wb[NB][2];
  load(wa, 0);
#pragma unroll 1
  for (int b = 0; b < NR - 2 * NB; b += 2 * NB) {
    load(wb, b + NB);
    sums(wa, b);
    load(wa, b + 2 * NB);
    sums(wb, b + NB);
  }
  load(wb, NR - NB);
  sums(wa, NR - 2 * NB);
  sums(wb, NR - NB);
}

template <int D, int P>
__global__ __launch_bounds__(256) void k_calib(CalibArgs a) {
  constexpr int LPR = D / 16, RPP = 256 / LPR, F = D / 2;
  constexpr int NR = kCalibChunk / RPP, NB = 2;    // rows per lane, rows per batch
  const int chunk = blockIdx.x, lh = blockIdx.y;
  const int l = lh / a.hq, h = lh % a.hq;
  const int tid = threadIdx.x, p = tid % LPR, r0 = tid / LPR;
  // element offsets of the lane's two 16-byte pieces within a row
  const int e0 = P == 0 ? 8 * p : 16 * p, e1 = P == 0 ? F + 8 * p : 16 * p + 8;
  const uint16_t* base = a.q + (int64_t)l * a.sl + (int64_t)h * a.sh;
  const int t0 = chunk * kCalibChunk + r0;
  float acc[8][5];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int s = 0; s < 5; ++s) acc[k][s] = 0.0f;
  if ((chunk + 1) * kCalibChunk <= a.n_tokens)
    calib_rows<D, P, NR, NB, RPP, true>(base, a.st, t0, a.n_tokens, e0, e1, acc);
  else
    calib_rows<D, P, NR, NB, RPP, false>(base, a.st, t0, a.n_tokens, e0, e1, acc);

  // the rows of a pass share their bands: add them in row order through LDS
  __shared__ float s_acc[RPP][F * 5];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int s = 0; s < 5; ++s) s_acc[r0][(8 * p + k) * 5 + s] = acc[k][s];
  __syncthreads();
  float* out = a.part + ((size_t)lh * a.n_chunks + chunk) * F * 5;
  for (int i = tid; i < F * 5; i += 256) {
    float v = 0.0f;
#pragma unroll 8
    for (int r = 0; r < RPP; ++r) v += s_acc[r][i];
    out[i] = v;
  }
}

__global__ __launch_bounds__(256) void k_calib_final(CalibArgs a) {
  const int lh = blockIdx.x, F = a.d / 2, FV = F * 5;
  __shared__ double s_sum[128 * 5];
  const float* pp = a.part + (size_t)lh * a.n_chunks * FV;
  for (int i = threadIdx.x; i < FV; i += 256) {
    double v = 0.0;
    for (int c = 0; c < a.n_chunks; ++c) v += (double)pp[(size_t)c * FV + i];
    s_sum[i] = v;
  }
  __syncthreads();
  const int f = threadIdx.x;
  if (f >= F) return;
  const double* sf = s_sum + 5 * f;
  const double T = (double)a.n_tokens;
  const double mr = sf[0] / T, mi = sf[1] / T, ab = sf[2] / T;
  const size_t o = (size_t)lh * F + f;
  a.mean_re[o] = (float)mr;
  a.mean_im[o] = (float)mi;
  a.abs_mean[o] = (float)ab;
  if (a.r) a.r[o] = ab > 0.0 ? (float)(sqrt(mr * mr + mi * mi) / ab) : 0.0f;
  if (a.mrl) a.mrl[o] = (float)(sqrt(sf[3] * sf[3] + sf[4] * sf[4]) / T);
}

// ============================================================================ decode loop
// In place: for every (unit, KV head), row j <- row idx[j] for j < cnt[u] (K, V and,
// when given, the head's position), in the cache the rows are read from, so that a
// pruned sequence keeps its own blocks.  The kept slots ascend and idx[j] >= j, so
// the rows written by chunk c (j in [c C, c C + C)) are read only by chunks <= c:
// one workgroup per (unit, KV head) walks the chunks in order, and each chunk's
// reads all complete (every load waited for, then a barrier) before any of its
// writes.  A chunk issues its indices', its source block ids' and its rows' loads
// each together.  Rows with idx[j] == j stay where they are.  An index that breaks
// the order (not ascending, below j, or outside [0, len[u])) is flagged and its row
// left as it is.
template <int D>
__global__ __launch_bounds__(256) void k_compact_inplace(InplaceArgs a) {
  constexpr int LPR = D / 8, RPP = 256 / LPR, NP = kInplaceRows / RPP;
  const int ug = blockIdx.x, u = ug / a.hkv, g = ug % a.hkv;
  const int n = min(max(a.len[u], 0), a.n_max);
  const int K = min(max(a.cnt[u], 0), min(a.b_max, n));
  const int part = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
  const int32_t* ix = a.idx + (size_t)ug * a.b_max;
  int32_t* ps = a.pos ? a.pos + (size_t)ug * a.n_max : nullptr;
  for (int c0 = 0; c0 < K; c0 += kInplaceRows) {
    int sl[NP], pr[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int j = min(c0 + r0 + p * RPP, K - 1);
      sl[p] = ix[j];
      pr[p] = j > 0 ? ix[j - 1] : -1;
    }
    bool mv[NP];
    int kb[NP], vb[NP];   // paged: the source rows' block ids (slot 0's for rows that stay)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int j = c0 + r0 + p * RPP;
      const bool ok = sl[p] >= j && sl[p] < n && (j == 0 || sl[p] > pr[p]);
      if (j < K && !ok && part == 0) raise_flag(a.flags, kFlagIndex);
      mv[p] = j < K && ok && sl[p] != j;
      const int ss = mv[p] ? sl[p] : 0;
      kb[p] = a.k.bt ? a.k.bt[(int64_t)u * a.k.mb + ss / a.k.bs] : 0;
      vb[p] = a.v.bt ? a.v.bt[(int64_t)u * a.v.mb + ss / a.v.bs] : 0;
    }
    const uint16_t* kp[NP];
    const uint16_t* vp[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const bool kbad = a.k.bt && (kb[p] < 0 || kb[p] >= a.k.npb);
      const bool vbad = a.v.bt && (vb[p] < 0 || vb[p] >= a.v.npb);
      if (mv[p] && (kbad || vbad) && part == 0) raise_flag(a.flags, kFlagBlock);
      mv[p] = mv[p] && !kbad && !vbad;
      const int ss = sl[p];
      kp[p] = a.k.bt ? a.k.base + ((int64_t)kb[p] * a.k.bs + ss % a.k.bs) * a.k.ss + (int64_t)g * a.k.sh
                     : a.k.base + (int64_t)u * a.k.su + (int64_t)g * a.k.sh + (int64_t)ss * a.k.ss;
      vp[p] = a.v.bt ? a.v.base + ((int64_t)vb[p] * a.v.bs + ss % a.v.bs) * a.v.ss + (int64_t)g * a.v.sh
                     : a.v.base + (int64_t)u * a.v.su + (int64_t)g * a.v.sh + (int64_t)ss * a.v.ss;
    }
    u32x4 kr[NP], vr[NP];
    int pv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (mv[p]) {
        kr[p] = reinterpret_cast<const u32x4*>(kp[p])[part];
        vr[p] = reinterpret_cast<const u32x4*>(vp[p])[part];
        pv[p] = ps ? ps[sl[p]] : 0;
      }
    }
    // every read of this chunk has returned before any thread writes it
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (!mv[p]) continue;
      const int j = c0 + r0 + p * RPP;
      uint16_t* kd = const_cast<uint16_t*>(row_ptr(a.k, u, g, j, a.flags));
      uint16_t* vd = const_cast<uint16_t*>(row_ptr(a.v, u, g, j, a.flags));
      if (kd) reinterpret_cast<u32x4*>(kd)[part] = kr[p];
      if (vd) reinterpret_cast<u32x4*>(vd)[part] = vr[p];
      if (ps && part == 0) ps[j] = pv[p];
    }
  }
}

// After the move: the unit now holds its kept count, len[u] <- cnt[u] (clamped as the
// move clamped it).  A kernel of its own, so that every (unit, KV head) of the move
// has read len[u] before it changes.
__global__ __launch_bounds__(256) void k_set_len(InplaceArgs a) {
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= a.n_units) return;
  const int n = min(max(a.len[u], 0), a.n_max);
  a.len[u] = min(max(a.cnt[u], 0), min(a.b_max, n));
}

// Appends t_new rows of each (unit, KV head) at slots len[u] + t (K, V and the
// unit's positions into every head's position row); slots past n_max are flagged.
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
  const int ug = blockIdx.x, u = ug / a.hkv, g = ug % a.hkv;
  const int lpr = a.d / 8, rpp = 256 / lpr;
  const int part = threadIdx.x % lpr;
  const int n0 = max(a.len[u], 0);
  for (int t = blockIdx.y * rpp + threadIdx.x / lpr; t < a.t_new; t += gridDim.y * rpp) {
    const int sl = n0 + t;
    if (sl >= a.n_max) {
      if (part == 0) raise_flag(a.flags, kFlagLen);
      continue;
    }
    const size_t src = ((size_t)ug * a.t_new + t) * a.d;
    uint16_t* kd = const_cast<uint16_t*>(row_ptr(a.k, u, g, sl, a.flags));
    uint16_t* vd = const_cast<uint16_t*>(row_ptr(a.v, u, g, sl, a.flags));
    if (kd) reinterpret_cast<u32x4*>(kd)[part] = reinterpret_cast<const u32x4*>(a.k_new + src)[part];
    if (vd) reinterpret_cast<u32x4*>(vd)[part] = reinterpret_cast<const u32x4*>(a.v_new + src)[part];
    if (a.pos && a.pos_new && part == 0) a.pos[(size_t)ug * a.n_max + sl] = a.pos_new[(size_t)u * a.t_new + t];
  }
}

// After the rows are in: len[u] <- min(len[u] + t_new, n_max) and, with positions
// given, the current query position q_pos[u] <- the newest appended position.  A
// kernel of its own, so that every block of k_append has read len[u] first.
__global__ __launch_bounds__(256) void k_append_advance(AppendArgs a) {
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= a.n_units) return;
  const int n0 = max(a.len[u], 0);
  a.len[u] = min(n0 + a.t_new, a.n_max);
  if (a.q_pos && a.pos_new) a.q_pos[u] = a.pos_new[(size_t)u * a.t_new + a.t_new - 1];
}

// ============================================================================ launches
hipError_t launch_coef(const CoefArgs& a, const Offsets& offs, hipStream_t s) {
  if (a.n_units == 0) return hipSuccess;
  // the maximum over offsets writes nblk * d/32 * 64 operands per (unit, KV head):
  // with few pairs, they are shared out over up to nblk blocks per pair so that the
  // launch fills the device
  // the mean over offsets with few pairs: one block per query head, so that each
  // block's chain of dependent steps covers one head
  const long pairs = (long)a.n_units * a.hkv;
  int zs = 1;
  if (a.omax) zs = (int)std::max(1L, std::min<long>(a.ob.nblk, (1024 + pairs - 1) / pairs));
  else if (pairs <= 64 && a.group > 1) zs = a.group;
  const dim3 grid((unsigned)a.n_units, (unsigned)a.hkv, (unsigned)zs);
#define TRIA_COEF_CASE(DD, PP)                                                   \
  if (a.d == DD && a.pairing == PP) {                                           \
    hipLaunchKernelGGL((k_coef<DD, PP>), grid, dim3(256), 0, s, a, offs);       \
    return hipGetLastError();                                                   \
  }
  TRIA_COEF_CASE(64, 0)
  TRIA_COEF_CASE(64, 1)
  TRIA_COEF_CASE(128, 0)
  TRIA_COEF_CASE(128, 1)
  TRIA_COEF_CASE(256, 0)
  TRIA_COEF_CASE(256, 1)
#undef TRIA_COEF_CASE
  return hipErrorInvalidValue;
}

size_t score_lds(int d, int group, bool paged, int omax, int nblk, int tile, int block_size, int single) {
  // two score buffers (one in the single-buffer mode), the region shared by the
  // tile's block ids and (the mean) the finalisation's histogram, the units' lengths
  // and tile prefix, and for the maximum over offsets the staged offset blocks, whose
  // region also holds the histogram
  const size_t used = (size_t)(single ? 1 : 2) * group * (tile + 16) +
                      (size_t)score_scratch(omax, paged, tile, block_size) + (size_t)(2 * kListUnits + 1);
  if (!omax) return used * 4;
  // the blocks, then the lanes' reference magnitudes (d/64 16-byte operands a lane)
  const size_t blocks = (size_t)nblk * (d / 32) * 64 * 16 + (size_t)(d / 64) * 64 * 16;
  return ((used + 3) & ~(size_t)3) * 4 + (blocks > (size_t)kBins * 4 ? blocks : (size_t)kBins * 4);
}

namespace {
// Resident-capacity answers, kept per device: a pass asks up to three times per
// tria_score call, and each answer costs an occupancy query and a device-attribute
// query of host time, which a launch-bound pass (few, short kernels) pays in full.
// An answer depends only on the device, the kernel variant and its LDS bytes.
struct CapEntry {
  int dev, d, pairing, paged, omax, single;
  size_t lds;
  int cap;
};
constexpr int kCapSlots = 32;
std::mutex g_cap_mu;
CapEntry g_cap[kCapSlots];
int g_cap_used = 0, g_cap_next = 0;
}  // namespace

int score_capacity(int d, int pairing, bool paged, int group, int omax, int nblk, int tile, int block_size,
                   int single) {
  const size_t lds = score_lds(d, group, paged, omax, nblk, tile, block_size, single);
  int per_cu = 0, dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const CapEntry key{dev, d, pairing, paged ? 1 : 0, omax ? 1 : 0, !paged && !omax && single ? 1 : 0, lds, 0};
  {
    std::lock_guard<std::mutex> lock(g_cap_mu);
    for (int i = 0; i < g_cap_used; ++i) {
      const CapEntry& c = g_cap[i];
      if (c.dev == key.dev && c.d == key.d && c.pairing == key.pairing && c.paged == key.paged &&
          c.omax == key.omax && c.single == key.single && c.lds == key.lds)
        return c.cap;
    }
  }
  hipError_t e = hipErrorInvalidValue;
#define TRIA_OCC_CASE(DD, PP, PG, MX)                                                                     \
  if (d == DD && pairing == PP && paged == PG && (omax != 0) == MX)                                       \
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(                                                     \
        &per_cu,                                                                                          \
        MX ? (const void*)k_score_max<DD, PP, PG>                                                        \
           : (!PG && single ? (const void*)k_score_single<DD, PP> : (const void*)k_score<DD, PP, PG>),   \
        256, lds);
#define TRIA_OCC_CASES(MX)        \
  TRIA_OCC_CASE(64, 0, false, MX)  \
  TRIA_OCC_CASE(64, 1, false, MX)  \
  TRIA_OCC_CASE(128, 0, false, MX) \
  TRIA_OCC_CASE(128, 1, false, MX) \
  TRIA_OCC_CASE(256, 0, false, MX) \
  TRIA_OCC_CASE(256, 1, false, MX) \
  TRIA_OCC_CASE(64, 0, true, MX)   \
  TRIA_OCC_CASE(64, 1, true, MX)   \
  TRIA_OCC_CASE(128, 0, true, MX)  \
  TRIA_OCC_CASE(128, 1, true, MX)  \
  TRIA_OCC_CASE(256, 0, true, MX)  \
  TRIA_OCC_CASE(256, 1, true, MX)
  TRIA_OCC_CASES(false)
  TRIA_OCC_CASES(true)
#undef TRIA_OCC_CASES
#undef TRIA_OCC_CASE
  if (e != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  CapEntry entry = key;
  entry.cap = per_cu * cus;
  {
    std::lock_guard<std::mutex> lock(g_cap_mu);
    g_cap[g_cap_next] = entry;
    g_cap_next = (g_cap_next + 1) % kCapSlots;
    if (g_cap_used < kCapSlots) ++g_cap_used;
  }
  return entry.cap;
}

hipError_t launch_score(const ScoreArgs& a, int d, int pairing, int max_wg, hipStream_t s) {
  const long tiles = (long)a.n_units * a.hkv * a.n_tiles;
  if (tiles == 0) return hipSuccess;
  const bool paged = a.k.bt != nullptr;
  int cap = score_capacity(d, pairing, paged, a.group, a.omax, a.ob.nblk, a.tile, a.k.bs, a.single);
  if (max_wg > 0 && max_wg < cap) cap = max_wg;
  if (cap < a.n_tiles) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles < cap ? tiles : cap)), blk(256);
  const size_t lds = score_lds(d, a.group, paged, a.omax, a.ob.nblk, a.tile, a.k.bs, a.single);
#define TRIA_SCORE_CASE(DD, PP, PG, MX)                                                  \
  if (d == DD && pairing == PP && paged == PG && (a.omax != 0) == MX) {                 \
    if (MX) hipLaunchKernelGGL((k_score_max<DD, PP, PG>), grid, blk, lds, s, a);        \
    else if (!PG && a.single) hipLaunchKernelGGL((k_score_single<DD, PP>), grid, blk, lds, s, a); \
    else hipLaunchKernelGGL((k_score<DD, PP, PG>), grid, blk, lds, s, a);              \
    return hipGetLastError();                                                            \
  }
#define TRIA_SCORE_CASES(MX)        \
  TRIA_SCORE_CASE(64, 0, false, MX)  \
  TRIA_SCORE_CASE(64, 1, false, MX)  \
  TRIA_SCORE_CASE(128, 0, false, MX) \
  TRIA_SCORE_CASE(128, 1, false, MX) \
  TRIA_SCORE_CASE(256, 0, false, MX) \
  TRIA_SCORE_CASE(256, 1, false, MX) \
  TRIA_SCORE_CASE(64, 0, true, MX)   \
  TRIA_SCORE_CASE(64, 1, true, MX)   \
  TRIA_SCORE_CASE(128, 0, true, MX)  \
  TRIA_SCORE_CASE(128, 1, true, MX)  \
  TRIA_SCORE_CASE(256, 0, true, MX)  \
  TRIA_SCORE_CASE(256, 1, true, MX)
  TRIA_SCORE_CASES(false)
  TRIA_SCORE_CASES(true)
#undef TRIA_SCORE_CASES
#undef TRIA_SCORE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectArgs& a, int strategy, hipStream_t s) {
  const long groups = (long)a.n_units * a.hkv;
  if (groups == 0) return hipSuccess;
  // one workgroup per group only on request: measured on MI355X it is 2x slower than
  // the tile-parallel kernels (one 512-thread workgroup fills a CU, and its four
  // threshold scans run back to back)
  const bool fits = a.n_max <= kSelGroupMax;
  if (fits && strategy == 1) {
    hipLaunchKernelGGL(k_sel_group, dim3((unsigned)groups), dim3(512), 0, s, a);
    return hipGetLastError();
  }
  const unsigned tiles = (unsigned)(groups * a.n_st);
  hipLaunchKernelGGL(k_sel_thresh, dim3((unsigned)groups), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tiles) {
    hipLaunchKernelGGL(k_sel_collect, dim3(tiles), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_sel_refine, dim3((unsigned)groups), dim3(512), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (tiles) hipLaunchKernelGGL(k_sel_emit, dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const long blocks = (long)a.n_units * a.hkv * a.n_rtiles;
  if (blocks == 0) return hipSuccess;
  const bool sp = a.ks.bt != nullptr, dp = a.kd.bt != nullptr;
  auto same_table = [](const auto& x, const auto& y) {
    return x.bt == y.bt && (x.bt == nullptr || (x.bs == y.bs && x.mb == y.mb && x.npb == y.npb));
  };
  if (same_table(a.ks, a.vs) && same_table(a.kd, a.vd)) {
#define TRIA_COMPACT_CASE(DD, SP, DP)                                                  \
    if (a.d == DD && sp == SP && dp == DP) {                                           \
      hipLaunchKernelGGL((k_compact_fast<DD, SP, DP>), dim3((unsigned)blocks), dim3(256), 0, s, a); \
      return hipGetLastError();                                                        \
    }
    TRIA_COMPACT_CASE(64, false, false)
    TRIA_COMPACT_CASE(64, false, true)
    TRIA_COMPACT_CASE(64, true, false)
    TRIA_COMPACT_CASE(64, true, true)
    TRIA_COMPACT_CASE(128, false, false)
    TRIA_COMPACT_CASE(128, false, true)
    TRIA_COMPACT_CASE(128, true, false)
    TRIA_COMPACT_CASE(128, true, true)
    TRIA_COMPACT_CASE(256, false, false)
    TRIA_COMPACT_CASE(256, false, true)
    TRIA_COMPACT_CASE(256, true, false)
    TRIA_COMPACT_CASE(256, true, true)
#undef TRIA_COMPACT_CASE
  }
  // K and V in different layouts: one row at a time
  hipLaunchKernelGGL(k_compact, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s) {
  if (a.n_layers == 0 || a.hq == 0 || a.n_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_chunks, (unsigned)(a.n_layers * a.hq));
#define TRIA_CALIB_CASE(DD, PP)                                                 \
  if (a.d == DD && a.pairing == PP) {                                          \
    hipLaunchKernelGGL((k_calib<DD, PP>), grid, dim3(256), 0, s, a);           \
    hipError_t e = hipGetLastError();                                          \
    if (e != hipSuccess) return e;                                             \
    hipLaunchKernelGGL(k_calib_final, dim3((unsigned)(a.n_layers * a.hq)), dim3(256), 0, s, a); \
    return hipGetLastError();                                                  \
  }
  TRIA_CALIB_CASE(64, 0)
  TRIA_CALIB_CASE(64, 1)
  TRIA_CALIB_CASE(128, 0)
  TRIA_CALIB_CASE(128, 1)
  TRIA_CALIB_CASE(256, 0)
  TRIA_CALIB_CASE(256, 1)
#undef TRIA_CALIB_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_compact_inplace(const InplaceArgs& a, hipStream_t s) {
  if (a.n_units == 0 || a.hkv == 0) return hipSuccess;
  const dim3 grid((unsigned)(a.n_units * a.hkv));
  if (a.d == 64) hipLaunchKernelGGL(k_compact_inplace<64>, grid, dim3(256), 0, s, a);
  else if (a.d == 128) hipLaunchKernelGGL(k_compact_inplace<128>, grid, dim3(256), 0, s, a);
  else if (a.d == 256) hipLaunchKernelGGL(k_compact_inplace<256>, grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_set_len, dim3((unsigned)((a.n_units + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ============================================================================ no-allocation pass
// The workspace of tria_pass_noalloc: a device array of the library's own, so that
// callers that cannot allocate device memory can run the pass.  Each device holds
// its own copy at its own address, found once per device with hipGetSymbolAddress;
// host code passes only that address to kernels (the array's name in host code is
// not a device address).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* scratch_address(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

namespace {
__global__ void k_set_word(int32_t* dst, int32_t v) { *dst = v; }
__global__ void k_copy_word(int32_t* dst, const int32_t* src) { *dst = *src; }
}  // namespace

hipError_t launch_set_word(int32_t* dst, int32_t v, hipStream_t s) {
  hipLaunchKernelGGL(k_set_word, dim3(1), dim3(1), 0, s, dst, v);
  return hipGetLastError();
}

hipError_t launch_copy_word(int32_t* dst, const int32_t* src, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(1), 0, s, dst, src);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.n_units == 0 || a.hkv == 0 || a.t_new == 0) return hipSuccess;
  const int rpp = 256 / (a.d / 8);
  const unsigned gy = (unsigned)min((a.t_new + rpp - 1) / rpp, 64);
  hipLaunchKernelGGL(k_append, dim3((unsigned)(a.n_units * a.hkv), gy), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_append_advance, dim3((unsigned)((a.n_units + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tria
