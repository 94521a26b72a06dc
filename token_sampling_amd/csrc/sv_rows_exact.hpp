// sv_rows_exact.hpp -- exact profile of one logits row by repeated passes
// over the row (any element type, any V), by NT threads: a workgroup of the
// generic kernel, or the one wave of a single-pass kernel that hands a row
// back to itself.
//
// SDCP Sec. 4.1: the distribution after temperature, top-k and top-p in that
// order; temperature 0 selects the argmax with ties to the smallest id.  The
// support is found on ordered integer keys:
//   top-k: the key kk of the k-th token in (key desc, id asc) order, by a
//          bitwise search on count(key >= t) >= k; c_k ties at kk are kept;
//   top-p: the largest key kp with 1000 * mass(key >= kp) >= P * Z_k, by a
//          bitwise search; then the smallest count c of tied tokens at kp with
//          1000 * (mass(key > kp) + c * w(kp)) >= P * Z_k;
//   the c-th smallest id among the ties is the cut id, by a bitwise search.
// Masses are binary64 sums of binary64 weights.
#pragma once

#include "sv_kernels.hpp"

namespace sv {
namespace exact {

template <int NT>
struct Smem {
  uint32_t u32[NT / kWave];
  int32_t i32[NT / kWave];
  uint64_t u64[NT / kWave];
  double f64[NT / kWave];
};

// This thread's index among the NT threads: a wave of a larger workgroup
// counts from its own first lane.
template <int NT>
__device__ inline int tid() {
  return (int)threadIdx.x & (NT - 1);
}

// Reduction over the NT threads: a wave alone needs no barrier (the other
// waves of its workgroup may have left).
template <int NT, typename T, typename Op, typename S>
__device__ inline T row_reduce(T v, Op op, S* smem) {
  if constexpr (NT == kWave) {
    (void)smem;
    return wave_reduce(v, op);
  } else {
    return block_reduce<NT>(v, op, smem);
  }
}

template <class Tr, int NT>
struct RowPasses {
  const typename Tr::elem_t* row;
  int V;
  Smem<NT>* sm;

  template <typename Pred>
  __device__ uint64_t count(Pred pred) const {
    uint64_t c = 0;
    for (int y = tid<NT>(); y < V; y += NT) c += pred(y, Tr::key(Tr::bits(row[y]))) ? 1 : 0;
    return row_reduce<NT>(c, OpAdd(), sm->u64);
  }

  // sum of 2^((l - lmax) * scale) over tokens with key >= kmin (binary64)
  __device__ double mass_ge(uint32_t kmin, float lmax, double scale) const {
    double s = 0.0;
    for (int y = tid<NT>(); y < V; y += NT) {
      const uint32_t u = Tr::bits(row[y]);
      if (Tr::key(u) >= kmin) s += weight64(Tr::value(u), lmax, scale);
    }
    return row_reduce<NT>(s, OpAdd(), sm->f64);
  }
};

template <class Tr, int NT>
__device__ __attribute__((always_inline)) void profile_row(const typename Tr::elem_t* row, int V,
                                                          const sv_sampling& smp, bool argmax_only,
                                                          int32_t x, RowRec* rec, Smem<NT>* sm) {
  RowPasses<Tr, NT> ps{row, V, sm};

  // largest / smallest key: bad logits and the row maximum
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
  for (int y = tid<NT>(); y < V; y += NT) {
    const uint32_t k = Tr::key(Tr::bits(row[y]));
    kmax = k > kmax ? k : kmax;
    kmin = k < kmin ? k : kmin;
  }
  kmax = row_reduce<NT>(kmax, OpMax(), sm->u32);
  kmin = row_reduce<NT>(kmin, OpMin(), sm->u32);
  const bool bad = kmax >= Tr::kInfKey || kmin < Tr::kNegInfKey || kmax <= Tr::kNegInfKey;

  int32_t amax = V;
  for (int y = tid<NT>(); y < V; y += NT)
    if (Tr::key(Tr::bits(row[y])) == kmax) amax = y < amax ? y : amax;
  amax = row_reduce<NT>(amax, OpMin(), sm->i32);

  RowRec r;
  r.ntie = 0;
  r.pad = 0;
  r.status = bad ? SV_S_BAD_LOGITS : 0;
  r.argmax = amax;
  r.nsup = 0;
  r.lmax = Tr::value(Tr::unkey(kmax));
  r.ptok = -1.0;

  if (bad || argmax_only || smp.temperature_milli == 0) {
    // one-hot support {argmax}, weight 1
    r.kcut = kmax;
    r.idcut = amax;
    r.scale = 0.0;
    r.zsum = 1.0;
    if (x >= 0 && !bad) r.ptok = (x == amax) ? 1.0 : 0.0;
    if (tid<NT>() == 0) *rec = r;
    return;
  }

  const double scale = 1.4426950408889634074 * 1000.0 / (double)smp.temperature_milli;
  const float lmax = r.lmax;
  const uint32_t kNeg = Tr::kNegInfKey;

  // finite tokens (no +inf / NaN remain): key > key(-inf)
  const uint64_t nfin = ps.count([=](int, uint32_t k) { return k > kNeg; });
  uint32_t kfmin = 0xFFFFFFFFu;
  for (int y = tid<NT>(); y < V; y += NT) {
    const uint32_t k = Tr::key(Tr::bits(row[y]));
    if (k > kNeg && k < kfmin) kfmin = k;
  }
  kfmin = row_reduce<NT>(kfmin, OpMin(), sm->u32);

  // top-k: exactly k tokens in (key desc, id asc) order
  const uint64_t keff =
      (smp.top_k > 0 && (uint64_t)smp.top_k < nfin) ? (uint64_t)smp.top_k : nfin;
  uint32_t kk = kfmin;
  if (keff < nfin) {
    uint32_t t = 0;
    for (int bit = Tr::kKeyBits - 1; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      if (ps.count([=](int, uint32_t k) { return k >= cand; }) >= keff) t = cand;
    }
    kk = t;
  }
  const uint64_t cgt_k = ps.count([=](int, uint32_t k) { return k > kk; });
  const uint64_t ck = keff - cgt_k;  // ties kept at kk (smallest ids)
  const double wk = weight64(Tr::value(Tr::unkey(kk)), lmax, scale);
  const double above_k = ps.mass_ge(kk + 1, lmax, scale);
  const double Zk = above_k + (double)ck * wk;

  uint32_t kcut = kk;
  uint64_t ccut = ck;
  double zsum = Zk;
  if (smp.top_p_milli < 1000) {
    const double tgt = (double)smp.top_p_milli * Zk;  // keep while 1000*C < tgt
    uint32_t t = 0;
    for (int bit = Tr::kKeyBits - 1; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      bool ok;
      if (cand > kmax) {
        ok = false;  // the kept prefix is never empty
      } else if (cand <= kk) {
        ok = true;  // the whole top-k support lies at or above cand
      } else {
        ok = 1000.0 * ps.mass_ge(cand, lmax, scale) >= tgt;
      }
      if (ok) t = cand;
    }
    const uint32_t kp = t;
    double above;
    uint64_t ntie;
    if (kp == kk) {
      above = above_k;
      ntie = ck;
    } else {
      above = ps.mass_ge(kp + 1, lmax, scale);
      ntie = ps.count([=](int, uint32_t k) { return k == kp; });
    }
    const double wt = weight64(Tr::value(Tr::unkey(kp)), lmax, scale);
    // first estimate of the tie count, then settle it on the exact predicate
    const double need = (tgt / 1000.0 - above) / wt;
    int64_t c = (int64_t)ntie;
    if (wt > 0.0 && need < (double)ntie) c = need <= 1.0 ? 1 : (int64_t)ceil(need);
    while (c > 1 && 1000.0 * (above + (double)(c - 1) * wt) >= tgt) --c;
    while (c < (int64_t)ntie && !(1000.0 * (above + (double)c * wt) >= tgt)) ++c;
    kcut = kp;
    ccut = (uint64_t)c;
    zsum = above + (double)c * wt;
  }

  // the ccut-th smallest id among the tokens whose key is kcut
  const uint64_t nat = ps.count([=](int, uint32_t k) { return k == kcut; });
  int32_t idcut;
  if (ccut >= nat) {
    int32_t last = -1;
    for (int y = tid<NT>(); y < V; y += NT)
      if (Tr::key(Tr::bits(row[y])) == kcut) last = y > last ? y : last;
    idcut = row_reduce<NT>(last, OpMax(), sm->i32);
  } else {
    uint32_t t = 0;
    for (int bit = 24; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      if (cand > (uint32_t)V) continue;
      const uint64_t n =
          ps.count([=](int y, uint32_t k) { return k == kcut && (uint32_t)y < cand; });
      if (n < ccut) t = cand;
    }
    idcut = (int32_t)t;
  }

  r.kcut = kcut;
  r.idcut = idcut;
  r.scale = scale;
  r.zsum = zsum;
  if (x >= 0) {
    const uint32_t u = Tr::bits(row[x]);
    const uint32_t kx = Tr::key(u);
    const bool member = kx > kcut || (kx == kcut && x <= idcut);
    r.ptok = member ? weight64(Tr::value(u), lmax, scale) / zsum : 0.0;
  }
  if (tid<NT>() == 0) *rec = r;
}


}  // namespace exact
}  // namespace sv
