// sv_rows_dense32.hpp -- binary32 logits rows of the dense class with a cut
// (top-p, or top-k above 64; SDCP Sec. 4.1), one wave64 per row.
//
// A binary32 key has 2^32 values, so the bf16 path's count histogram (one
// bin per key, every bin holding tokens of one value) does not carry over.
// Instead:
//  1. One streaming pass, as the bf16 dense pass, over coarse keys.  The
//     coarse key of a logit is the bf16 key of its upper 16 bits (the logit
//     truncated toward zero to 7 mantissa bits), so coarse keys are in the
//     order of the logits and each spans 1/128 of an octave.  The window
//     holds the kWin coarse keys at and below the running maximum's, and
//     each bin keeps its count and its mass relative to its own reference
//     r (the truncated value): the sum over its logits l of 2^((l - r) s),
//     l - r exact in binary32, the exponent (l - r) sf + (l - r) (s - sf)
//     rounded once, one exp2 per logit, added in binary64 (LDS atomics).
//     The bin's mass relative to lmax is 2^((r - lmax) s) times that.
//     Tokens below the window go to the binary32 sum as in the bf16 pass,
//     and bins that leave the window give their mass to a departed sum.
//  2. A walk over the window's counts (top-k) and masses (top-p) finds the
//     coarse key the cut lies in.  A second pass over the row lists that
//     coarse key's tokens (their number is known) in LDS as (key, id) with
//     their binary64 weights, and bitwise searches over those keys settle
//     the cut key and its tie count as the exact profile does.  Top-k and
//     top-p cutting in different coarse keys take a third pass.
// Rows handed back to the caller (which profiles them exactly): the cut below
// the window, more tokens in the cut's coarse key than the list holds, a
// maximum with |lmax| s > 256 (where the rounding of a bin-relative exponent
// would pass 2^-23), or logits beyond binary32 exponents.
//
// Precision: a window token's weight carries the exp2 error (about one ulp)
// and the rounding of its exponent, at most 2^-24 |(l - r) s| <= 2^-31 |r| s
// (|l - r| < 2^-7 |r|).  For bins at or below lmax with |r| s <= 256 that is
// at most 2^-23 (binary64 sums add no more), so Z, the cut masses and p are
// within about 2e-7 of the exact sums; a bin with |r| s > 256 lies below a
// negative lmax by more than |r| - 256 / s, and its tokens weigh less than
// 2^-(|r| s - 256) each.  Weights of listed tokens and of the drafted token
// are exact binary64.
#pragma once

#include "sv_rows_dense.hpp"

namespace sv {
namespace dense32 {

using namespace stream;
using dense::kNegInfKey;
using dense::kNoAnchor;
using dense::kWin;
using dense::max_nan;
using dense::Scales;
using dense::skey_of;
using dense::uni;
using dense::value_of;

constexpr int kVec = 2;                  // 16-byte loads per lane per tile
constexpr int kNBuf = 5;                 // tiles in the load ring (kNBuf - 1 in flight)
constexpr int kTile = kWave * kVec * 4;  // binary32 logits per tile
constexpr int kPerLane = kWin / kWave;   // bins per lane in the walk
// LDS of one wave: kWin binary64 masses, then kWin counts; the listed tokens
// of a coarse key reuse it as composites, then weights.
constexpr int kLdsBytes = kWin * (8 + 4);
constexpr int kMemberCap = kLdsBytes / 16;
constexpr float kMaxLS = 256.0f;  // |lmax| s above this: handed back

// Bin reference of a logit: its upper 16 bits (the coarse key's value).
__device__ inline float cref(float f) {
  return __uint_as_float(__float_as_uint(f) & 0xFFFF0000u);
}
// The largest and the smallest value of coarse key c (c > kNegInfKey).
// Coarse key 0 holds +0, -0 and the denormals of both signs below 2^-133.
__device__ inline float top_of(int c) {
  return c >= 0 ? __uint_as_float(((uint32_t)c << 16) | 0xFFFFu) : value_of(c);
}
__device__ inline float bottom_of(int c) {
  return c > 0 ? value_of(c) : __uint_as_float(((0x8000u | (uint32_t)(-c)) << 16) | 0xFFFFu);
}
// composite (key desc, id asc) of a listed token: the 32-bit key of sv::F32
__device__ inline uint64_t composite(uint32_t bits, uint32_t id) {
  return ((uint64_t)F32::key(bits) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ inline uint32_t comp_key(uint64_t c) { return (uint32_t)(c >> 32); }

struct Window {
  double* mass;    // kWin masses relative to each bin's reference, index = key mod kWin
  uint32_t* cnt;   // kWin counts
  int anchor;      // largest coarse key seen (kNoAnchor: no finite logit yet)
  float edge;      // largest value of coarse key anchor: a larger logit moves the window
  float lo_v;      // smallest value of the window's lowest coarse key
  float dref;      // the lanes' departed masses are relative to this value
  int lo;          // the window's lowest coarse key
};
struct Lane {
  float mv;    // this lane's largest logit
  float q;     // the wave's exponent offset of the binary32 sum (an integer)
  double s;    // sum of 2^(l sf - q) over this lane's tokens below the window
  double dep;  // mass relative to Window::dref of tokens in bins that left the window
  bool ovf;    // a maximum too large: the row is handed back
};

// The window moves up to coarse key tk (wave-uniform, above anchor).
__device__ inline void window_move(Lane& L, Window& W, int tk, const Scales& sc) {
  const int lane = __lane_id();
  const bool had = W.anchor != kNoAnchor;
  const float nref = uni(value_of(tk));
  // the binary32 sum's offset: every term of a token below the window is at
  // most 1; a power-of-two rescale is exact (NaN stays NaN)
  const float qn = ceilf(top_of(tk) * sc.sf);
  if (qn < 0x1p22f) {
    if (had) L.s = ldexp(L.s, (int)(L.q - qn));
    L.q = qn;
  } else {
    L.ovf = true;
  }
  if (had) L.dep *= exp2(((double)W.dref - (double)nref) * sc.s);
  // bins that leave: their mass moves to dep (relative to nref)
  const int d = had ? tk - W.anchor : kWin;
  if (d >= kWin) {  // every bin (the first window: clears them)
    for (int i = lane; i < kWin; i += kWave) {
      if (had) {
        const int ko = W.anchor - ((W.anchor - i) & (kWin - 1));  // the key leaving bin i
        const uint32_t c = W.cnt[i];
        if (c && ko > kNegInfKey)
          L.dep += W.mass[i] * exp2(((double)value_of(ko) - (double)nref) * sc.s);
      }
      W.cnt[i] = 0u;
      W.mass[i] = 0.0;
    }
  } else {  // key anchor - (kWin - 1) + j sits in bin anchor + 1 + j
    for (int j = lane; j < d; j += kWave) {
      const int ko = W.anchor - (kWin - 1) + j;
      const int i = (W.anchor + 1 + j) & (kWin - 1);
      const uint32_t c = W.cnt[i];
      if (c && ko > kNegInfKey)
        L.dep += W.mass[i] * exp2(((double)value_of(ko) - (double)nref) * sc.s);
      W.cnt[i] = 0u;
      W.mass[i] = 0.0;
    }
  }
  W.dref = nref;
  W.anchor = __builtin_amdgcn_readfirstlane(tk);
  W.edge = uni(top_of(tk));
  W.lo = __builtin_amdgcn_readfirstlane(max(tk - (kWin - 1), kNegInfKey + 1));
  W.lo_v = uni(bottom_of(W.lo));
}

// The 4 logits of a vector: counted and weighed in their bins (in the
// window), else added to the binary32 sum.
template <bool kPos>
__device__ __attribute__((always_inline)) inline void pass1_tokens(Lane& L, Window& W,
                                                                   const float (&f)[4],
                                                                   const Scales& sc, float df) {
  float w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // in the window: 2^((l - r) s) relative to the bin's reference r (l - r
    // exact: the same sign and exponent); below it: 2^(l sf - q).  Selects of
    // operands, not of two expressions, so that no branch is taken per logit.
    const bool in = f[e] >= W.lo_v;
    const float dl = f[e] - (in ? cref(f[e]) : 0.0f);
    const float ex = __builtin_fmaf(dl, sc.sf, in ? dl * df : -L.q);
    const float t = __builtin_amdgcn_exp2f(ex);
    if (in) {
      const int i = kPos ? (int)__builtin_amdgcn_ubfe(__float_as_uint(f[e]), 16, 10)
                         : skey_of(f[e]) & (kWin - 1);
      atomicAdd(&W.cnt[i], 1u);
      atomicAdd(&W.mass[i], (double)t);
    }
    w[e] = in ? 0.0f : t;
  }
  L.s += (double)((w[0] + w[1]) + (w[2] + w[3]));
}

// One 16-byte vector (4 logits) of the first pass.
__device__ __attribute__((always_inline)) inline void pass1_vec(Lane& L, Window& W, const u32x4& v,
                                                                const Scales& sc, float df) {
  float f[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(elem(v, e));
  const float lmv = max_nan(max_nan(f[0], f[1]), max_nan(f[2], f[3]));
  L.mv = max_nan(L.mv, lmv);
  const bool up = lmv > W.edge;  // false for NaN
  if (__ballot(up)) {
    const int tk = wave_reduce(up ? skey_of(lmv) : INT32_MIN, OpMax());
    window_move(L, W, tk, sc);
  }
  // a window of positive keys: a logit's bin is bits 16..25 of its bits
  if (W.lo > 0) pass1_tokens<true>(L, W, f, sc, df);
  else pass1_tokens<false>(L, W, f, sc, df);
}

// The row's layout: a 16-byte aligned window in which [head, head + V) is the row.
struct RowWin {
  const u32x4* vbase;
  int head, npos, nvec, ntiles;
};
__device__ inline RowWin row_window(const uint32_t* row, int V) {
  RowWin R;
  R.head = (int)(((uintptr_t)row & 15u) >> 2);
  R.vbase = (const u32x4*)(row - R.head);
  R.npos = R.head + V;
  R.nvec = (R.npos + 3) / 4;
  R.ntiles = (R.npos + kTile - 1) / kTile;
  return R;
}

// Stream the row through the ring; fn(tile vector, first position of the
// lane's 4 logits) for every vector, positions outside the row as -inf.
template <class Fn>
__device__ __attribute__((always_inline)) inline void stream_row(const RowWin& R, Fn fn) {
  const int lane = __lane_id();
  u32x4 ring[kNBuf][kVec];
#pragma unroll
  for (int u = 0; u < kNBuf - 1; ++u) {
    load_tile<kVec>(ring[u], R.vbase, u, R.nvec - 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nround = (R.ntiles + kNBuf - 1) / kNBuf;
  for (int r = 0; r < nround; ++r) {
    set_priority(nround - r, nround);
#pragma unroll
    for (int u = 0; u < kNBuf; ++u) {
      const int tt = r * kNBuf + u;
      load_tile<kVec>(ring[(u + kNBuf - 1) % kNBuf], R.vbase, tt + kNBuf - 1, R.nvec - 1);
      if ((tt == 0 && R.head > 0) || (tt + 1) * kTile > R.npos)
        mask_tile_f32<kVec>(ring[u], tt, R.head, R.npos);
#pragma unroll
      for (int j = 0; j < kVec; ++j)
        fn(ring[u][j], tt * kTile + j * (kWave * 4) + lane * 4 - R.head);
    }
  }
}

// The tokens of coarse key c (the first pass counted at most kMemberCap),
// listed in LDS by a pass over the row, with their weights at s relative to
// lmax.
struct List {
  uint64_t* comp;  // composites, in row order
  double* w;       // weights
  int n;
};
__device__ inline List list_key(const RowWin& R, int c, float lmax, const Scales& sc, void* lds) {
  List Ls{(uint64_t*)lds, (double*)((char*)lds + kMemberCap * 8), 0};
  int k = 0;
  // the upper 16 bits of the key's logits (either sign for key 0); c is above
  // -inf's key, so no masked position matches
  const uint32_t cmask = c == 0 ? 0x7FFFu : 0xFFFFu;
  const uint32_t cbits = c >= 0 ? (uint32_t)c : (0x8000u | (uint32_t)(-c));
  stream_row(R, [&](const u32x4& v, int p0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t bits = elem(v, e);
      const bool hit = ((bits >> 16) & cmask) == cbits;
      const uint64_t mk = __ballot(hit);
      if (mk) {
        const int at = k + lanes_below(mk);
        if (hit && at < kMemberCap) Ls.comp[at] = composite(bits, (uint32_t)(p0 + e));
        k += popc64(mk);
      }
    }
  });
  Ls.n = min(k, kMemberCap);
  for (int i = __lane_id(); i < Ls.n; i += kWave)
    Ls.w[i] = weight64(F32::value(F32::unkey(comp_key(Ls.comp[i]))), lmax, sc.s);
  return Ls;
}
// Count and mass of the listed tokens with key >= t.
__device__ inline uint32_t list_count_ge(const List& Ls, uint32_t t) {
  uint32_t c = 0;
  for (int i = __lane_id(); i < Ls.n; i += kWave) c += comp_key(Ls.comp[i]) >= t ? 1u : 0u;
  return wave_reduce(c, OpAdd());
}
__device__ inline double list_mass_ge(const List& Ls, uint32_t t) {
  double s = 0.0;
  for (int i = __lane_id(); i < Ls.n; i += kWave) s += comp_key(Ls.comp[i]) >= t ? Ls.w[i] : 0.0;
  return wave_reduce(s, OpAdd());
}
// the largest key t with count(key >= t) >= need (need >= 1, at most n)
__device__ inline uint32_t list_kth_key(const List& Ls, uint32_t need) {
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    if (list_count_ge(Ls, cand) >= need) t = cand;
  }
  return t;
}

// The profile of one binary32 row with a cut, by one wave; lds is the wave's
// kLdsBytes.  Returns true if the row is handed back.
__device__ __attribute__((always_inline)) inline bool row_profile(
    const uint32_t* row, int V, const sv_sampling& smp, int32_t x, RowRec* rec, void* lds) {
  const int lane = __lane_id();
  const Scales sc = dense::row_scales(smp.temperature_milli);
  const float df = uni((float)sc.d);
  const RowWin R = row_window(row, V);
  Window W{(double*)lds, (uint32_t*)((char*)lds + kWin * 8), kNoAnchor, -__builtin_huge_valf(),
           __builtin_huge_valf(), 0.0f, kNoAnchor};
  Lane L{-__builtin_huge_valf(), 0.0f, 0.0, 0.0, false};
  stream_row(R, [&](const u32x4& v, int) { pass1_vec(L, W, v, sc, df); });
  const float lmax = dense::wave_max(L.mv);
  if (__ballot(L.ovf)) return true;

  // the lanes' sums relative to lmax, combined in a fixed order
  const double zb = wave_reduce(L.s * exp2((double)L.q - (double)lmax * (double)sc.sf), OpAdd());
  const double zd =
      wave_reduce(L.dep != 0.0 ? L.dep * exp2(((double)W.dref - (double)lmax) * sc.s) : 0.0,
                  OpAdd());
  RowRec rr{};
  rr.argmax = -1;
  rr.lmax = lmax;
  rr.scale = sc.s;
  rr.ptok = -1.0;
  if (!(zb == zb) || zb == __builtin_huge_val() || lmax == __builtin_huge_valf() ||
      lmax == -__builtin_huge_valf()) {
    rr.status = SV_S_BAD_LOGITS;
    rr.zsum = 1.0;
    if (lane == 0) *rec = rr;
    return false;
  }
  if (fabsf(lmax) * sc.sf >= kMaxLS) return true;

  // the window: lane q holds the bins of keys anchor - kPerLane q - e, with
  // their counts and masses relative to lmax
  uint32_t cnt[kPerLane];
  double ms[kPerLane];
  double win = 0.0;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) {
    const int k = W.anchor - kPerLane * lane - e;
    const int i = k & (kWin - 1);
    cnt[e] = k > kNegInfKey ? W.cnt[i] : 0u;
    ms[e] = cnt[e] ? W.mass[i] * exp2(((double)value_of(k) - (double)lmax) * sc.s) : 0.0;
    win += ms[e];
  }
  win = wave_reduce(win, OpAdd());
  const double z = win + zd + zb;
  const bool top_p = smp.top_p_milli < 1000;
  const bool top_k = smp.top_k > 0 && smp.top_k < (uint32_t)V;

  int ck_key = 0;     // coarse key of the listed tokens (top-k: the cut's)
  List Ls{nullptr, nullptr, 0};
  uint32_t kk = 0, ckk = 0;  // top-k: cut key and its ties kept
  double zsum = z;
  uint32_t kcut = 0, j = 0;
  if (top_k) {
    const uint32_t K = smp.top_k;
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) tot += cnt[e];
    const uint32_t cincl = wave_incl_scan(tot);
    const uint64_t hitk = __ballot(cincl >= K);
    if (!hitk) return true;  // fewer than K tokens in the window
    const int qk = __builtin_ctzll(hitk);
    // lane qk's bins, from its top: the first where the count reaches K
    uint32_t above = lane_read(cincl - tot, qk);
    int ek = 0;
    uint32_t nk = 0;
    bool fk = false;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const uint32_t c = lane_read(cnt[e], qk);
      if (!fk && above + c >= K) {
        ek = e;
        nk = c;
        fk = true;
      } else if (!fk) {
        above += c;
      }
    }
    // above: tokens in the bins before the cut's, whose coarse key is ck_key
    ck_key = W.anchor - kPerLane * qk - ek;
    if (nk > (uint32_t)kMemberCap) return true;
    Ls = list_key(R, ck_key, lmax, sc, lds);
    const uint32_t need = K - above;  // 1 <= need <= nk
    kk = list_kth_key(Ls, need);
    ckk = need - list_count_ge(Ls, kk + 1);
    // the kept mass of the cut's coarse key, in place of its bin's; bins below are dropped
    const double kept = list_mass_ge(Ls, kk + 1) +
                        (double)ckk * weight64(F32::value(F32::unkey(kk)), lmax, sc.s);
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const bool at = lane == qk && e == ek;
      const bool below = lane > qk || (lane == qk && e > ek);
      ms[e] = at ? kept : (below ? 0.0 : ms[e]);
    }
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) part += ms[e];
    zsum = wave_reduce(part, OpAdd());
    kcut = kk;
    j = ckk;
  }

  if (top_p) {  // over the top-k distribution: stop at 1000 * C >= P * Z_k
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) part += ms[e];
    const double incl = wave_incl_scan(part);
    const double tgt = (double)smp.top_p_milli * zsum;
    const uint64_t hit = __ballot(1000.0 * incl >= tgt);
    if (!hit) return true;  // the cut lies below the window
    const int q = __builtin_ctzll(hit);
    double c = lane_read(incl - part, q);
    int ep = 0;
    uint32_t np = 0;
    bool found = false;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const double me = lane_read(ms[e], q);
      const uint32_t ce = lane_read(cnt[e], q);
      if (!found && me != 0.0 && 1000.0 * (c + me) >= tgt) {
        ep = e;
        np = ce;
        found = true;
      }
      c += found ? 0.0 : me;
    }
    if (!found) return true;  // the lane's sum crossed, its bins in order did not (rounding)
    // c: the mass of the bins before the cut's (kept tokens)
    const int cp_key = W.anchor - kPerLane * q - ep;
    const bool same = top_k && cp_key == ck_key;
    if (!same) {
      if (np > (uint32_t)kMemberCap) return true;
      Ls = list_key(R, cp_key, lmax, sc, lds);
    }
    // the largest key kp with 1000 * (c + mass(kept, key >= kp)) >= tgt
    uint32_t t = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      bool ok;
      if (same && cand <= kk) ok = true;  // the whole top-k support lies at or above cand
      else ok = 1000.0 * (c + list_mass_ge(Ls, cand)) >= tgt;
      if (ok) t = cand;
    }
    const uint32_t kp = t;
    // the coarse key's kept mass must reach the target at kp (the walk's and
    // the list's sums agree but for rounding): else handed back
    uint32_t ntie;
    double above;
    if (same && kp == kk) {
      above = c + list_mass_ge(Ls, kk + 1);
      ntie = ckk;
    } else {
      const uint32_t nge = list_count_ge(Ls, kp), ngt = list_count_ge(Ls, kp + 1);
      if (nge == ngt) return true;  // no listed token at kp
      above = c + list_mass_ge(Ls, kp + 1);
      ntie = nge - ngt;
    }
    const double wt = weight64(F32::value(F32::unkey(kp)), lmax, sc.s);
    if (!(1000.0 * (above + (double)ntie * wt) >= tgt)) return true;
    const double need = (tgt / 1000.0 - above) / wt;
    int64_t cc = (int64_t)ntie;
    if (wt > 0.0 && need < (double)ntie) cc = need <= 1.0 ? 1 : (int64_t)ceil(need);
    while (cc > 1 && 1000.0 * (above + (double)(cc - 1) * wt) >= tgt) --cc;
    while (cc < (int64_t)ntie && !(1000.0 * (above + (double)cc * wt) >= tgt)) ++cc;
    kcut = kp;
    j = (uint32_t)cc;
    zsum = above + (double)cc * wt;
  }

  rr.kcut = kcut;
  rr.idcut = -1;
  rr.ntie = (int32_t)j;
  rr.zsum = zsum;
  if (x >= 0) {
    const uint32_t bx = row[x];
    const uint32_t kx = F32::key(bx);
    bool member = kx > kcut;
    if (kx == kcut) {  // its rank among the listed tokens of its key
      const uint64_t cx = composite(bx, (uint32_t)x);
      uint32_t r = 0;
      for (int i = lane; i < Ls.n; i += kWave) r += (comp_key(Ls.comp[i]) == kx && Ls.comp[i] > cx) ? 1u : 0u;
      member = wave_reduce(r, OpAdd()) < j;
    }
    rr.ptok = member ? weight64(__uint_as_float(bx), lmax, sc.s) / zsum : 0.0;
  }
  if (lane == 0) *rec = rr;
  return false;
}

}  // namespace dense32
}  // namespace sv
