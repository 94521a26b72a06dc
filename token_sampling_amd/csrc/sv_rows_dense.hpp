// sv_rows_dense.hpp -- one pass over a bf16 logits row for the profiles whose
// support is not limited to a few best tokens: temperature alone, or
// temperature with top-k above 64 and/or top-p (SDCP Sec. 4.1).
//
// One wave64 streams one row through a ring of 1 KiB tiles (as the top-k
// kernel does) and computes, in that single pass:
//  - the largest logit lmax;
//  - Z = sum over the row of 2^((l - lmax) * s), s = log2(e) / T.  Every
//    weight, mass and probability of the row is taken in binary64 at this s
//    (the profile is the softmax at T itself).  The one pass sums in binary32
//    at sf, s rounded to binary32: each lane keeps an integer exponent offset
//    q and its sum of 2^(l*sf - q) (one fma and one exp2 per logit); a
//    vector's 8 terms are summed pairwise in binary32 and added to the lane's
//    binary64 sum.  q is set at the lane's first finite logit and moves up (by
//    an exact power-of-two rescale) when a logit passes it by one octave, so
//    the rounded exponent of the lane's largest terms stays below 2 in
//    magnitude; the lanes combine in binary64 in a fixed order.  Z then drops
//    the scale's rounding: rows with a histogram (below) replace the window's
//    share of the sum by its exact binary64 mass at s (the window holds the
//    row's largest logits, the tokens below it weigh at least 2^-8 octaves
//    less); untruncated rows also sum w * l per lane, and add the first-order
//    term ln2 (s - sf) sum w (l - lmax) (|s - sf| <= 2^-24 s, so the second
//    order is below 1e-11 for every term above 2^-60 of the row's largest).
//    A NaN anywhere makes Z NaN; +inf makes it NaN or infinite.
//  - with top-k or top-p: a count histogram of the kWin keys at and below the
//    running maximum, in LDS, indexed by key mod kWin.  When the maximum
//    rises, the bins of the keys that leave the window are cleared for the
//    keys that enter; the window's bottom only rises, so every token whose key
//    lies in the final window has been counted.  After the pass, top-k counts
//    K tokens down from the top: the key where the count reaches K keeps the
//    K - (tokens above it) smallest ids, and Z_k is the sum of the kept
//    counts times their keys' weights.  Top-p then walks the kept masses from
//    the top until 1000 * C >= P * Z_k (Z_k = Z without top-k).  Either gives
//    the cut key kc and the number j of its tokens that stay (those with the j
//    smallest ids, profile order being logit desc, id asc).  A cut below the
//    window (fewer than K tokens in it, or top-p's mass not reached) hands
//    the row back: the caller profiles it exactly.
//  - the drafted token's rank among the tokens of its key with smaller ids (its
//    key's bin just before its vector, plus the earlier tokens of that vector):
//    it is in the support iff its key is above kc, or equal to kc with rank < j.
// The cut is recorded as (kc, j); the sampling kernel turns j into a cut id
// when it needs one.  The argmax is not computed: no rule reads it for these
// profiles (greedy and temperature-0 rows take the top-k kernel).
// row_profile_split runs the same pass over S parts of the row, one wave per
// part, and merges the parts' windows, sums and ranks before the cut.
#pragma once

#include "sv_kernels.hpp"
#include "sv_stream.hpp"

namespace sv {
namespace dense {

using namespace stream;

constexpr int kVec = 2;                  // 16-byte loads per lane per tile
#ifndef SV_DENSE_NBUF
#define SV_DENSE_NBUF 4
#endif
constexpr int kNBuf = SV_DENSE_NBUF;     // tiles in the load ring (kNBuf - 1 in flight)
constexpr int kTile = kWave * kVec * 8;  // bf16 logits per tile
constexpr int kWin = 1024;               // keys in the top-p histogram window
constexpr int kPerLane = kWin / kWave;   // bins per lane in the walk
constexpr int kNegInfKey = -0x7F80;

// signed key of a bf16 value (the order of the logits; +0 and -0 are equal)
__device__ inline int skey_of(float f) {
  const uint32_t h = __float_as_uint(f) >> 16;
  const int mag = (int)(h & 0x7FFFu);
  return (h & 0x8000u) ? -mag : mag;
}
__device__ inline float value_of(int key) {
  const uint32_t bits = key >= 0 ? (uint32_t)key : (0x8000u | (uint32_t)(-key));
  return __uint_as_float(bits << 16);
}

// The row's scales: s for every binary64 weight, sf (s rounded to binary32)
// for the one-pass sum.
struct Scales {
  double s;      // log2(e) * 1000 / temperature_milli
  double d;      // s - sf (exact)
  float sf;
  float inv_sf;  // 1 / sf, rounded: only the lanes' offset thresholds use it
};
// Wave-uniform values kept in scalar registers.
__device__ inline float uni(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ inline double uni(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ inline Scales row_scales(uint32_t t_milli) {
  Scales c;
  c.s = uni(1.4426950408889634074 * 1000.0 / (double)t_milli);
  c.sf = uni((float)c.s);
  c.d = uni(c.s - (double)c.sf);
  c.inv_sf = uni(1.0f / c.sf);
  return c;
}

struct LaneSum {
  float mv;   // this lane's largest logit so far (-inf: none finite yet)
  float q;    // exponent offset: an integer, at most one octave below mv * sf
  float vt;   // logits above vt move q up (-inf until the first finite logit)
  double s;   // sum of 2^(l * sf - q) over this lane's logits so far
  double l1;  // untruncated rows: sum of 2^(l * sf - q) * l (the scale's correction)
  float dep;  // rows with a histogram: mass relative to Hist::dref of the tokens
              // counted in bins that later left the window (this lane's bins)
  bool ovf;   // a logit too large for binary32 exponents: the row falls back
};

constexpr int kNoAnchor = -0x10000;  // no window yet (no finite logit seen)
struct Hist {
  uint32_t* bin;    // kWin counts, index = key mod kWin
  int anchor;       // largest key seen (the window is [anchor - kWin + 1, anchor])
  float anchor_v;   // its value
  float lo_v;       // value of the window's lowest key (never -inf)
  float dref;       // the lanes' departed masses are relative to this value
  int kx;           // key of the drafted token (when it has one)
  int rank_x;       // tokens with key kx and a smaller id
};
__device__ inline Hist hist_init(uint32_t* bins, int kx) {
  return Hist{bins, kNoAnchor, -__builtin_huge_valf(), -__builtin_huge_valf(), 0.0f, kx, 0};
}

// The maximum of two binary32 values, NaN if either is NaN (v_maximum on this
// chip).  fmaxf would skip a NaN but costs a canonicalizing instruction per
// logit; a NaN in the row makes its sums NaN and the row bad either way.
__device__ inline float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Bits 14..25 of x in one v_bfe_u32.
__device__ inline uint32_t bits_14_25(uint32_t x) { return __builtin_amdgcn_ubfe(x, 14, 12); }

// One lane's step over kE logits: its maximum, its offset q, and (kSum: rows
// without a histogram) its binary32 sum of 2^(l sf - q) with the sum of
// those terms times l.  Returns the kE logits' maximum.
template <int kE, bool kSum>
__device__ __attribute__((always_inline)) inline float lane_step(LaneSum& L, const float (&f)[kE],
                                                                 const Scales& sc) {
  float lmv = f[0];
#pragma unroll
  for (int e = 1; e < kE; ++e) lmv = max_nan(lmv, f[e]);
  L.mv = max_nan(L.mv, lmv);
  if (lmv > L.vt && lmv < __builtin_huge_valf()) {  // first finite logit, or an octave up
    const float qn = ceilf(lmv * sc.sf);
    L.ovf |= !(qn < 0x1p22f);
    // a power-of-two rescale is exact; NaN from earlier logits stays NaN
    const bool first = L.vt == -__builtin_huge_valf();
    L.s = first ? (L.s != L.s ? L.s : 0.0) : ldexp(L.s, (int)(L.q - qn));
    if constexpr (kSum) L.l1 = first ? (L.l1 != L.l1 ? L.l1 : 0.0) : ldexp(L.l1, (int)(L.q - qn));
    L.q = qn;
    L.vt = (qn + 1.0f) * sc.inv_sf;
  }
  if constexpr (kSum) {
    float w[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) w[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], sc.sf, -L.q));
    float ts;
    if constexpr (kE == 8) ts = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
    else ts = (w[0] + w[1]) + (w[2] + w[3]);
    L.s += (double)ts;
    // w * l, with -inf logits (weight 0) taken as the largest negative finite
    // value so that they add 0; a NaN logit has a NaN weight and stays NaN
    float tl = w[0] * max_nan(f[0], -__FLT_MAX__);
#pragma unroll
    for (int e = 1; e < kE; ++e) tl = __builtin_fmaf(w[e], max_nan(f[e], -__FLT_MAX__), tl);
    L.l1 += (double)tl;
  }
  return lmv;
}

// One 16-byte vector (8 logits) of a tile: the lane's maximum and running sum,
// then (kHist: top-k and top-p rows) the histogram window and the drafted
// token's rank.  p0 is the window position of the vector's first logit; xvec
// says (wave-uniform) whether the drafted token lies in this vector of the wave.
template <bool kHist>
__device__ __attribute__((always_inline)) inline void dense_vec(LaneSum& L, Hist& H,
                                                                const u32x4& v, int p0, int px,
                                                                bool xvec, const Scales& sc) {
  float f[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = elem(v, d);
    // the two bf16 halves as binary32 (byte permutes: x << 16, x & 0xFFFF0000)
    f[2 * d] = __uint_as_float(__builtin_amdgcn_perm(0u, x, 0x01000C0Cu));
    f[2 * d + 1] = __uint_as_float(__builtin_amdgcn_perm(0u, x, 0x03020C0Cu));
  }
  if constexpr (!kHist) {
    (void)lane_step<8, true>(L, f, sc);
    return;
  }
  // rows with a histogram: the offset q is the wave's, moved with the window
  // (below), so the lanes need only their maximum here
  float lmv = f[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) lmv = max_nan(lmv, f[e]);
  L.mv = max_nan(L.mv, lmv);
  if (__ballot(lmv > H.anchor_v)) {  // the window moves up (wave-uniform)
    int tk = skey_of(lmv);
    tk = wave_reduce(tk, OpMax());
    const int lane = __lane_id();
    const int d = tk - H.anchor;  // keys anchor+1 .. tk take the bins of the keys leaving
    const float nref = uni(value_of(tk));
    const bool had = H.anchor != kNoAnchor;
    // the wave's offset: q = ceil(lmax sf) keeps every term at or below 2; a
    // power-of-two rescale of the sums is exact (NaN stays NaN).  A maximum
    // beyond binary32 exponents (or +inf, or NaN) hands the row back.
    const float qn = ceilf(nref * sc.sf);
    if (qn < 0x1p22f) {
      if (had) L.s = ldexp(L.s, (int)(L.q - qn));
      L.q = qn;
      L.vt = __builtin_huge_valf();  // the lane's sum is relative to the wave's q
    } else {
      L.ovf = true;
    }
    // the leaving bins' tokens are in no sum: their mass goes to dep.  They lie
    // at least kWin keys (eight octaves of magnitude) below the new maximum, so
    // binary32 suffices: an error of a few 1e-7 of a mass far below Z's
    if (had) L.dep *= __builtin_amdgcn_exp2f((H.dref - nref) * sc.sf);
    if (!had || d >= kWin) {  // every bin (the first window: clears them)
      for (int i = lane; i < kWin; i += kWave) {
        const int ko = H.anchor - ((H.anchor - i) & (kWin - 1));  // the key leaving bin i
        const uint32_t c = had ? H.bin[i] : 0u;
        if (c && ko > kNegInfKey)
          L.dep += (float)c * __builtin_amdgcn_exp2f((value_of(ko) - nref) * sc.sf);
        H.bin[i] = 0u;
      }
    } else {  // the d keys leaving: key anchor - (kWin - 1) + j sits in bin anchor + 1 + j
      for (int j = lane; j < d; j += kWave) {
        const int ko = H.anchor - (kWin - 1) + j;
        const int i = (H.anchor + 1 + j) & (kWin - 1);
        const uint32_t c = H.bin[i];
        if (c && ko > kNegInfKey)
          L.dep += (float)c * __builtin_amdgcn_exp2f((value_of(ko) - nref) * sc.sf);
        H.bin[i] = 0u;
      }
    }
    H.dref = uni(nref);
    H.anchor = __builtin_amdgcn_readfirstlane(tk);
    H.anchor_v = uni(nref);
    H.lo_v = uni(value_of(max(tk - (kWin - 1), kNegInfKey + 1)));
  }
  const int lo = H.anchor - (kWin - 1);
  if (xvec) {  // the drafted token's rank: its key's bin before this vector, plus
               // this vector's tokens (in every lane) of that key at smaller ids
    int before = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) before += (p0 + e < px && skey_of(f[e]) == H.kx) ? 1 : 0;
    before = wave_reduce(before, OpAdd());
    H.rank_x = (H.kx >= lo ? (int)H.bin[H.kx & (kWin - 1)] : 0) + before;
  }
  // tokens in the window are counted; the binary32 sum takes only the others.
  // One test per token selects both.  The count is an LDS atomic from the
  // lanes whose token is in the window only (measured: atomics from every
  // lane, the others into a dummy word, cost more than the branch saves).
  float w[8];
  if (lo > 0) {
    // a window of positive keys: the key is the upper half of the bits, and the
    // unpacked value's low 16 bits are zero, so bits 14..25 are the bin's byte
    // offset
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = f[e] >= H.lo_v;
      if (in) atomicAdd((uint32_t*)((char*)H.bin + bits_14_25(__float_as_uint(f[e]))), 1u);
      const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], sc.sf, -L.q));
      w[e] = in ? 0.0f : t;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = f[e] >= H.lo_v;
      if (in) atomicAdd(&H.bin[skey_of(f[e]) & (kWin - 1)], 1u);
      const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], sc.sf, -L.q));
      w[e] = in ? 0.0f : t;
    }
  }
  L.s += (double)(((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7])));
}

// The row's layout for the pass: a 16-byte aligned window over the row, in
// which positions [head, head + V) are the row.
struct RowWin {
  const u32x4* vbase;
  int head, npos, nvec, ntiles;
};
__device__ inline RowWin row_window(const uint16_t* row, int V) {
  RowWin W;
  W.head = (int)(((uintptr_t)row & 15u) >> 1);
  W.vbase = (const u32x4*)(row - W.head);
  W.npos = W.head + V;
  W.nvec = (W.npos + 7) / 8;
  W.ntiles = (W.npos + kTile - 1) / kTile;
  return W;
}

// The pass over tiles [t0, t1) of the window, by one wave: its lanes' running
// maxima and sums (L), and with kHist its histogram window (H) and, when the
// drafted token lies in these tiles, the token's rank among the tokens of its
// key before it in these tiles.  Positions from t1's first on read as -inf.
template <bool kHist>
__device__ __attribute__((always_inline)) inline void stream_part(const RowWin& W, int t0, int t1,
                                                                  int px, const Scales& sc,
                                                                  LaneSum& L, Hist& H) {
  const int lane = __lane_id();
  const int hi = min(W.npos, t1 * kTile);
  const int xv = px >= 0 ? px / (kWave * 8) : -1;  // the drafted token's vector index
  u32x4 ring[kNBuf][kVec];
#pragma unroll
  for (int u = 0; u < kNBuf - 1; ++u) {
    load_tile<kVec>(ring[u], W.vbase, t0 + u, W.nvec - 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nround = (t1 - t0 + kNBuf - 1) / kNBuf;
  for (int r = 0; r < nround; ++r) {
    set_priority(nround - r, nround);
#pragma unroll
    for (int u = 0; u < kNBuf; ++u) {
      const int tt = t0 + r * kNBuf + u;
      load_tile<kVec>(ring[(u + kNBuf - 1) % kNBuf], W.vbase, tt + kNBuf - 1, W.nvec - 1);
      if ((tt == 0 && W.head > 0) || (tt + 1) * kTile > hi) mask_tile<kVec>(ring[u], tt, W.head, hi);
#pragma unroll
      for (int j = 0; j < kVec; ++j)
        dense_vec<kHist>(L, H, ring[u][j], tt * kTile + j * (kWave * 8) + lane * 8, px,
                         tt * kVec + j == xv, sc);
    }
  }
}

__device__ inline LaneSum lane_sum_init() {
  return LaneSum{-__builtin_huge_valf(), 0.0f, -__builtin_huge_valf(), 0.0, 0.0, 0.0f, false};
}

// This wave's sums relative to lmax (lanes combined in a fixed order):
// z = sum of 2^((l - lmax) sf) over the tokens the binary32 pass summed (rows
// with a histogram: those below the window when they were read); c
// (untruncated rows) = sum of 2^((l - lmax) sf) (l - lmax), the first-order
// term of the scale's rounding; dep (rows with a histogram) = the exact mass
// at s of the tokens whose bins left the window.
struct WaveZ {
  double z, c, dep;
};
template <bool kHist>
__device__ inline WaveZ wave_z(const LaneSum& L, const Hist& H, float lmax, const Scales& sc) {
  const double ref = (double)lmax * (double)sc.sf;  // exact: both factors are binary32
  const bool none = L.vt == -__builtin_huge_valf();  // no finite logit in this lane
  const double f = none ? 1.0 : exp2((double)L.q - ref);
  double z = L.s * f;
  double c = kHist ? 0.0 : (none ? L.l1 : (L.l1 - (double)lmax * L.s) * f);
  double dep = (kHist && L.dep != 0.0f)
                   ? (double)L.dep * exp2(((double)H.dref - (double)lmax) * sc.s) : 0.0;
  z = wave_reduce(z, OpAdd());
  c = wave_reduce(c, OpAdd());
  dep = wave_reduce(dep, OpAdd());
  return WaveZ{z, c, dep};
}

__device__ inline float wave_max(float v) {
  v = fmaxf(v, lane_xor<32>(v));
  v = fmaxf(v, lane_xor<16>(v));
  v = fmaxf(v, lane_xor<8>(v));
  v = fmaxf(v, lane_xor<4>(v));
  v = fmaxf(v, lane_xor<2>(v));
  v = fmaxf(v, lane_xor<1>(v));
  return v;
}

template <bool kHist, class Tr = Bf16>
__device__ __attribute__((always_inline)) inline bool finish(const sv_sampling& smp, int V,
                                                             int32_t x, float xval, float lmax,
                                                             WaveZ z, bool ovf, const Hist& H,
                                                             RowRec* rec);

__device__ inline bool row_has_hist(const sv_sampling& smp, int V) {
  return smp.top_p_milli < 1000 || (smp.top_k > 0 && smp.top_k < (uint32_t)V);
}

// The profile of one row of the dense class, by one wave: temperature > 0,
// top-k off or above 64, with or without top-p.  bins is the wave's LDS
// histogram of kWin counts.  Returns true if the row is handed back.
template <bool kHist>
__device__ __attribute__((always_inline)) inline bool row_profile_t(
    const uint16_t* row, int V, const sv_sampling& smp, int32_t x, RowRec* rec, uint32_t* bins) {
  const Scales sc = row_scales(smp.temperature_milli);
  const RowWin W = row_window(row, V);
  const float xval = x >= 0 ? __uint_as_float((uint32_t)row[x] << 16) : 0.0f;
  LaneSum L = lane_sum_init();
  Hist H = hist_init(bins, x >= 0 ? skey_of(xval) : 0);
  stream_part<kHist>(W, 0, W.ntiles, x >= 0 ? x + W.head : -1, sc, L, H);
  const float lmax = wave_max(L.mv);
  return finish<kHist>(smp, V, x, xval, lmax, wave_z<kHist>(L, H, lmax, sc),
                       __ballot(L.ovf) != 0, H, rec);
}
__device__ __attribute__((always_inline)) inline bool row_profile(
    const uint16_t* row, int V, const sv_sampling& smp, int32_t x, RowRec* rec, uint32_t* bins) {
  return row_has_hist(smp, V) ? row_profile_t<true>(row, V, smp, x, rec, bins)
                              : row_profile_t<false>(row, V, smp, x, rec, bins);
}

// What each wave of a split row leaves for the merge.
struct PartRec {
  float lmax;
  int anchor;  // the part's histogram window is [anchor - kWin + 1, anchor]
  int nx;      // tokens of the drafted token's key: before it (its own part), or all
  int ovf;
  double z, c, dep;  // the part's sums relative to the row's lmax (see WaveZ)
};

// The same profile with the row split over the S waves of a workgroup, for
// launches with few rows: wave w streams tiles [w T / S, (w + 1) T / S) into
// its own histogram window (bins + w kWin), and wave 0 merges them.  Every
// part's window ends at its own maximum, at or below the row's, so each holds
// every token of the keys in the row's window [A - kWin + 1, A] (A the row's
// largest key) that lie at or below its maximum: the row's counts there are
// the sums of those bins.  Z is the parts' sums relative to the row's maximum,
// added in part order.  Called by every wave of the workgroup (it has
// workgroup barriers); returns true (in wave 0) if the row is handed back.
template <int S, bool kHist>
__device__ __attribute__((always_inline)) inline bool row_profile_split_t(
    const uint16_t* row, int V, const sv_sampling& smp, int32_t x, RowRec* rec, uint32_t* bins_all,
    PartRec* parts, int wid) {
  const int lane = __lane_id();
  const Scales sc = row_scales(smp.temperature_milli);
  const RowWin W = row_window(row, V);
  const float xval = x >= 0 ? __uint_as_float((uint32_t)row[x] << 16) : 0.0f;
  const int kx = x >= 0 ? skey_of(xval) : 0;
  const int px = x >= 0 ? x + W.head : -1;
  const int t0 = wid * W.ntiles / S, t1 = (wid + 1) * W.ntiles / S;
  const bool x_here = px >= 0 && px / kTile >= t0 && px / kTile < t1;
  LaneSum L = lane_sum_init();
  Hist H = hist_init(bins_all + wid * kWin, kx);
  stream_part<kHist>(W, t0, t1, x_here ? px : -1, sc, L, H);
  const float lm = wave_max(L.mv);
  const bool ovf = __ballot(L.ovf) != 0;
  // tokens of the drafted token's key: before it in its part, all of them in
  // a part before it (when the key lies in the part's window)
  int nx = 0;
  if (x_here) nx = H.rank_x;
  else if (x >= 0 && kHist && kx <= H.anchor && kx > H.anchor - kWin)
    nx = (int)H.bin[kx & (kWin - 1)];
  if (lane == 0) {
    parts[wid].lmax = lm;
    parts[wid].anchor = H.anchor;
    parts[wid].nx = nx;
    parts[wid].ovf = ovf ? 1 : 0;
  }
  __syncthreads();
  float lmax = parts[0].lmax;
#pragma unroll
  for (int w = 1; w < S; ++w) lmax = fmaxf(lmax, parts[w].lmax);
  const WaveZ zw = wave_z<kHist>(L, H, lmax, sc);
  if (lane == 0) {
    parts[wid].z = zw.z;
    parts[wid].c = zw.c;
    parts[wid].dep = zw.dep;
  }
  __syncthreads();  // every part's sum and histogram are complete
  if (wid != 0) return false;
  WaveZ z{parts[0].z, parts[0].c, parts[0].dep};
  int anc = parts[0].anchor, any_ovf = parts[0].ovf;
#pragma unroll
  for (int w = 1; w < S; ++w) {
    z.z += parts[w].z;
    z.c += parts[w].c;
    z.dep += parts[w].dep;
    anc = max(anc, parts[w].anchor);
    any_ovf |= parts[w].ovf;
  }
  Hist M = hist_init(bins_all, kx);
  M.anchor = anc;
  M.anchor_v = value_of(anc);
  M.lo_v = value_of(max(anc - (kWin - 1), kNegInfKey + 1));
  if constexpr (kHist) {
    // the row's window: bin i holds key k = anc - ((anc - i) mod kWin).  Part
    // w's bin i holds key kw = a_w - ((a_w - i) mod kWin) (a_w <= anc, its own
    // anchor): the same key when kw lies in the row's window; else a key below
    // it, whose tokens are in no sum yet and add their exact mass to dep
    double below = 0.0;
    for (int i = lane; i < kWin; i += kWave) {
      const int k = anc - ((anc - i) & (kWin - 1));
      uint32_t c = 0;
#pragma unroll
      for (int w = 0; w < S; ++w) {
        const int aw = parts[w].anchor;
        const uint32_t cw = aw == kNoAnchor ? 0u : bins_all[w * kWin + i];
        const int kw = aw - ((aw - i) & (kWin - 1));
        if (kw == k) c += cw;
        else if (cw && kw > kNegInfKey)
          below += (double)cw * exp2(((double)value_of(kw) - (double)lmax) * sc.s);
      }
      bins_all[i] = c;
    }
    below = wave_reduce(below, OpAdd());
    z.dep += below;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (px >= 0) {  // the drafted token's rank: the parts before its own, then its own
      const int tx = px / kTile;
      for (int w = 0; w < S; ++w) {
        M.rank_x += parts[w].nx;
        if (tx < (w + 1) * W.ntiles / S) break;
      }
    }
  }
  return finish<kHist>(smp, V, x, xval, lmax, z, any_ovf != 0, M, rec);
}

template <int S>
__device__ __attribute__((always_inline)) inline bool row_profile_split(
    const uint16_t* row, int V, const sv_sampling& smp, int32_t x, RowRec* rec, uint32_t* bins_all,
    PartRec* parts, int wid) {
  return row_has_hist(smp, V)
             ? row_profile_split_t<S, true>(row, V, smp, x, rec, bins_all, parts, wid)
             : row_profile_split_t<S, false>(row, V, smp, x, rec, bins_all, parts, wid);
}

// After the pass: the row's record from its maximum, the one-pass sums, the
// overflow flag and the histogram window H (with the drafted token's key and
// rank).  Every weight here is binary64 at the row's true scale s.  Returns
// true if the row is handed back.
template <bool kHist, class Tr>
__device__ __attribute__((always_inline)) inline bool finish(const sv_sampling& smp, int V,
                                                             int32_t x, float xval, float lmax,
                                                             WaveZ zc, bool ovf, const Hist& H,
                                                             RowRec* rec) {
  const int lane = __lane_id();
  const bool top_p = smp.top_p_milli < 1000;
  const bool top_k = smp.top_k > 0 && smp.top_k < (uint32_t)V;
  const Scales sc = row_scales(smp.temperature_milli);
  const uint32_t* bins = H.bin;
  if (ovf) {  // logits beyond binary32 exponent range: handed back
    return true;
  }

  RowRec rr{};
  rr.argmax = -1;
  rr.lmax = lmax;
  rr.scale = sc.s;
  rr.ptok = -1.0;
  const bool bad = !(zc.z == zc.z) || zc.z == __builtin_huge_val() || !(zc.c == zc.c) ||
                   lmax == __builtin_huge_valf() || lmax == -__builtin_huge_valf();
  if (bad) {
    rr.status = SV_S_BAD_LOGITS;
    rr.zsum = 1.0;
    if (lane == 0) *rec = rr;
    return false;
  }
  const double wx = x >= 0 ? weight64(xval, lmax, sc.s) : 0.0;
  if constexpr (!kHist) {  // the support is every finite logit
    // Z at s: the one-pass sum at sf and its first-order correction
    const double z = zc.z + 0.69314718055994530942 * sc.d * zc.c;
    rr.kcut = Tr::kNegInfKey + 1;
    rr.idcut = 0x7FFFFFFF;
    rr.zsum = z;
    if (x >= 0) rr.ptok = wx / z;
    if (lane == 0) *rec = rr;
    return false;
  }

  // the window's counts: lane q holds the bins of keys anchor - kPerLane*q - e;
  // and the window's exact mass at s
  uint32_t cnt[kPerLane];
  double win = 0.0;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) {
    const int k = H.anchor - kPerLane * lane - e;
    cnt[e] = k > kNegInfKey ? bins[k & (kWin - 1)] : 0u;
    if (cnt[e]) win += (double)cnt[e] * weight64(value_of(k), lmax, sc.s);
  }
  win = wave_reduce(win, OpAdd());
  // Z at s: the window's and the departed bins' exact masses, and the binary32
  // sum of the tokens below the window when they were read
  const double z = win + zc.dep + zc.z;
  int kc = 0, j = 0;  // the cut: key kc keeps its j smallest ids
  // top-k: the first K tokens of the order, counted from the top.  Counts
  // after the cut are cleared, so that the masses below are those of the kept
  // tokens.
  if (top_k) {
    const uint32_t K = smp.top_k;
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) tot += cnt[e];
    const uint32_t cincl = wave_incl_scan(tot);
    const uint64_t hitk = __ballot(cincl >= K);
    if (!hitk) {  // fewer than K tokens in the window
      return true;
    }
    const int qk = __builtin_ctzll(hitk);
    uint32_t above = lane_read(cincl - tot, qk);  // tokens in the lanes before qk
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      // every lane walks lane qk's counts (wave-uniform): the cut is the last
      // key that keeps a token
      const uint32_t c = lane_read(cnt[e], qk);
      const uint32_t keep = above >= K ? 0u : (K - above < c ? K - above : c);
      if (keep) {
        kc = H.anchor - kPerLane * qk - e;
        j = (int)keep;
      }
      if (lane == qk) cnt[e] = keep;
      above += c;
    }
    if (lane > qk) {
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) cnt[e] = 0u;
    }
  }

  // masses of the kept counts, summed from the top
  double part = 0.0;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e)
    if (cnt[e]) part += (double)cnt[e] * weight64(value_of(H.anchor - kPerLane * lane - e), lmax, sc.s);
  const double incl = wave_incl_scan(part);
  // Z_k: the mass of the top-k set (the last lane's prefix), else the row's Z
  double zsum = top_k ? lane_read(incl, kWave - 1) : z;

  if (top_p) {  // over the top-k distribution: stop at 1000 * C >= P * Z_k
    const double tgt = (double)smp.top_p_milli * zsum;
    const uint64_t hit = __ballot(1000.0 * incl >= tgt);
    if (!hit) {  // the cut lies below the window (never with top-k: C reaches Z_k)
      return true;
    }
    const int q = __builtin_ctzll(hit);
    double c_above = 0.0, wc = 0.0;
    if (lane == q) {
      double c = incl - part;
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) {
        if (!cnt[e]) continue;
        const int k = H.anchor - kPerLane * lane - e;
        const double w = weight64(value_of(k), lmax, sc.s);
        // this lane's last key with tokens, all kept, unless a key below crosses
        kc = k;
        j = (int)cnt[e];
        c_above = c;
        wc = w;
        if (1000.0 * (c + (double)cnt[e] * w) >= tgt) {
          // the smallest j with 1000 * (c + j * w) >= tgt
          int jj = (int)ceil((tgt / 1000.0 - c) / w);
          jj = max(1, min((int)cnt[e], jj));
          while (jj > 1 && 1000.0 * (c + (double)(jj - 1) * w) >= tgt) --jj;
          while (jj < (int)cnt[e] && 1000.0 * (c + (double)jj * w) < tgt) ++jj;
          j = jj;
          break;
        }
        c += (double)cnt[e] * w;
      }
    }
    kc = lane_read(kc, q);
    j = lane_read(j, q);
    c_above = lane_read(c_above, q);
    wc = lane_read(wc, q);
    zsum = c_above + (double)j * wc;
  }
  rr.kcut = (uint32_t)(kc + 0x8000);
  rr.idcut = -1;
  rr.ntie = j;
  rr.zsum = zsum;
  if (x >= 0) {
    const bool member = H.kx > kc || (H.kx == kc && H.rank_x < j);
    rr.ptok = member ? wx / zsum : 0.0;
  }
  if (lane == 0) *rec = rr;
  return false;
}


// A binary32 row of the dense class without a histogram (temperature alone:
// top-k and top-p off), by one wave: one pass through a ring of 2 KiB tiles
// (4 logits per 16-byte vector), the lanes' maxima and sums as for bf16 rows.
// Rows with top-p or top-k above 64 take the exact profile.  Returns true if
// the row is handed back.
__device__ __attribute__((always_inline)) inline bool row_profile_f32_untruncated(
    const uint32_t* row, int V, const sv_sampling& smp, int32_t x, RowRec* rec) {
  constexpr int kT = kWave * kVec * 4;  // binary32 logits per tile
  const Scales sc = row_scales(smp.temperature_milli);
  const int head = (int)(((uintptr_t)row & 15u) >> 2);
  const u32x4* vbase = (const u32x4*)(row - head);
  const int npos = head + V;
  const int nvec = (npos + 3) / 4;
  const int ntiles = (npos + kT - 1) / kT;
  const float xval = x >= 0 ? __uint_as_float(row[x]) : 0.0f;
  LaneSum L = lane_sum_init();
  u32x4 ring[kNBuf][kVec];
#pragma unroll
  for (int u = 0; u < kNBuf - 1; ++u) {
    load_tile<kVec>(ring[u], vbase, u, nvec - 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nround = (ntiles + kNBuf - 1) / kNBuf;
  for (int r = 0; r < nround; ++r) {
    set_priority(nround - r, nround);
#pragma unroll
    for (int u = 0; u < kNBuf; ++u) {
      const int tt = r * kNBuf + u;
      load_tile<kVec>(ring[(u + kNBuf - 1) % kNBuf], vbase, tt + kNBuf - 1, nvec - 1);
      if ((tt == 0 && head > 0) || (tt + 1) * kT > npos) mask_tile_f32<kVec>(ring[u], tt, head, npos);
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        float f[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) f[d] = __uint_as_float(elem(ring[u][j], d));
        (void)lane_step<4, true>(L, f, sc);
      }
    }
  }
  const float lmax = wave_max(L.mv);
  const Hist H = hist_init(nullptr, 0);
  return finish<false, F32>(smp, V, x, xval, lmax, wave_z<false>(L, H, lmax, sc),
                            __ballot(L.ovf) != 0, H, rec);
}

}  // namespace dense
}  // namespace sv
