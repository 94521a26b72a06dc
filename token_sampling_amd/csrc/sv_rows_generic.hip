// sv_rows_generic.hip -- exact profile of one logits row per workgroup, by
// repeated passes over the row (any element type, any V).
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
#include <algorithm>

#include "sv_kernels.hpp"

namespace sv {

namespace {

constexpr int kNT = 256;

struct Smem {
  uint32_t u32[kNT / kWave];
  int32_t i32[kNT / kWave];
  uint64_t u64[kNT / kWave];
  double f64[kNT / kWave];
};

template <class Tr>
struct RowPasses {
  const typename Tr::elem_t* row;
  int V;
  Smem* sm;

  template <typename Pred>
  __device__ uint64_t count(Pred pred) const {
    uint64_t c = 0;
    for (int y = threadIdx.x; y < V; y += kNT) c += pred(y, Tr::key(Tr::bits(row[y]))) ? 1 : 0;
    return block_reduce<kNT>(c, OpAdd(), sm->u64);
  }

  // sum of 2^((l - lmax) * scale) over tokens with key >= kmin (binary64)
  __device__ double mass_ge(uint32_t kmin, float lmax, double scale) const {
    double s = 0.0;
    for (int y = threadIdx.x; y < V; y += kNT) {
      const uint32_t u = Tr::bits(row[y]);
      if (Tr::key(u) >= kmin) s += weight64(Tr::value(u), lmax, scale);
    }
    return block_reduce<kNT>(s, OpAdd(), sm->f64);
  }
};

template <class Tr>
__device__ void profile_generic(const typename Tr::elem_t* row, int V, const sv_sampling& smp,
                                bool argmax_only, int32_t x, RowRec* rec, Smem* sm) {
  RowPasses<Tr> ps{row, V, sm};

  // largest / smallest key: bad logits and the row maximum
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu;
  for (int y = threadIdx.x; y < V; y += kNT) {
    const uint32_t k = Tr::key(Tr::bits(row[y]));
    kmax = k > kmax ? k : kmax;
    kmin = k < kmin ? k : kmin;
  }
  kmax = block_reduce<kNT>(kmax, OpMax(), sm->u32);
  kmin = block_reduce<kNT>(kmin, OpMin(), sm->u32);
  const bool bad = kmax >= Tr::kInfKey || kmin < Tr::kNegInfKey || kmax <= Tr::kNegInfKey;

  int32_t amax = V;
  for (int y = threadIdx.x; y < V; y += kNT)
    if (Tr::key(Tr::bits(row[y])) == kmax) amax = y < amax ? y : amax;
  amax = block_reduce<kNT>(amax, OpMin(), sm->i32);

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
    if (threadIdx.x == 0) *rec = r;
    return;
  }

  const double scale = 1.4426950408889634074 * 1000.0 / (double)smp.temperature_milli;
  const float lmax = r.lmax;
  const uint32_t kNeg = Tr::kNegInfKey;

  // finite tokens (no +inf / NaN remain): key > key(-inf)
  const uint64_t nfin = ps.count([=](int, uint32_t k) { return k > kNeg; });
  uint32_t kfmin = 0xFFFFFFFFu;
  for (int y = threadIdx.x; y < V; y += kNT) {
    const uint32_t k = Tr::key(Tr::bits(row[y]));
    if (k > kNeg && k < kfmin) kfmin = k;
  }
  kfmin = block_reduce<kNT>(kfmin, OpMin(), sm->u32);

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
    for (int y = threadIdx.x; y < V; y += kNT)
      if (Tr::key(Tr::bits(row[y])) == kcut) last = y > last ? y : last;
    idcut = block_reduce<kNT>(last, OpMax(), sm->i32);
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
  if (threadIdx.x == 0) *rec = r;
}

// Does row slot slot_g need this kernel?  Rows of the other row kernels only
// when they handed the row back.
template <class Tr>
__device__ bool generic_row(int slot_g, const int32_t* m, const int32_t* rule,
                            const sv_sampling* sampling, const int32_t* sess_status, int M, int V,
                            const RowRec* rows, bool draft_logits) {
  const int R = 2 * M + 1;
  const int b = slot_g / R;
  const int slot = slot_g - b * R;
  if (sess_status[b] != 0) return false;
  const int mb = m[b];
  const int rl = rule[b];
  const bool is_target = slot <= M;
  const int i = is_target ? slot + 1 : slot - M;  // 1-based position
  // draft rows are profiled only when draft logits are given (not with q rows)
  if (is_target ? (i > mb + 1) : (rl != SV_RULE_SPECULATIVE || i > mb || !draft_logits))
    return false;
  const sv_sampling smp = sampling[b];
  if (row_uses_topk_kernel(Tr::kDtype, rl, smp) || row_uses_dense_kernel(Tr::kDtype, rl, smp, V))
    return rows[slot_g].status == kRowFallback;
  return true;
}

// A grid of at most kMaxBlocks workgroups scans the row slots: each workgroup
// takes an equal share of consecutive slots, kNT at a time; each thread checks
// one slot, the slots that need this kernel are listed in LDS, and the
// workgroup profiles them one after another.
constexpr int kMaxBlocks = 1024;
template <class Tr>
__global__ __launch_bounds__(kNT) void k_rows_generic(
    const typename Tr::elem_t* __restrict__ target, const typename Tr::elem_t* __restrict__ draft,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling,
    const int32_t* __restrict__ sess_status, int B, int M, int V, RowRec* __restrict__ rows,
    uint32_t* __restrict__ draw_flag, uint32_t draw_token) {
  __shared__ Smem sm;
  __shared__ int32_t todo[kNT];
  __shared__ int32_t wave_cnt[kNT / kWave];
  const int R = 2 * M + 1;
  const int slots = B * R;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  // this workgroup's slots: an equal share, so that few rows spread over many groups
  const int per = (slots + (int)gridDim.x - 1) / (int)gridDim.x;
  const int end = min(slots, ((int)blockIdx.x + 1) * per);
  for (int base = (int)blockIdx.x * per; base < end; base += kNT) {
    const int slot_g = base + (int)threadIdx.x;
    const bool need = slot_g < end &&
                      generic_row<Tr>(slot_g, m, rule, sampling, sess_status, M, V, rows,
                                      draft != nullptr);
    if (need) draw_flag[slot_g / R] = draw_token;  // a row without a listed support
    const uint64_t mask = __ballot(need);
    __syncthreads();  // the previous round's list is consumed
    if (lane == 0) wave_cnt[wid] = __builtin_popcountll(mask);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kNT / kWave; ++w) {
      before += w < wid ? wave_cnt[w] : 0;
      total += wave_cnt[w];
    }
    if (need)
      todo[before + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0))] = slot_g;
    __syncthreads();
    for (int t = 0; t < total; ++t) {
      const int sg = todo[t];
      const int b = sg / R;
      const int slot = sg - b * R;
      const bool is_target = slot <= M;
      const int i = is_target ? slot + 1 : slot - M;
      const int mb = m[b];
      const int32_t x = i <= mb ? tokens[(size_t)b * M + (i - 1)] : -1;
      const typename Tr::elem_t* row =
          is_target ? target + ((size_t)b * (M + 1) + (i - 1)) * (size_t)V
                    : draft + ((size_t)b * M + (i - 1)) * (size_t)V;
      profile_generic<Tr>(row, V, sampling[b], rule[b] == SV_RULE_GREEDY, x, rows + sg, &sm);
    }
  }
}

}  // namespace

void launch_rows_generic(const LaunchArgs& a, hipStream_t st) {
  const size_t slots = (size_t)a.B * (2 * a.M + 1);
  const unsigned grid = (unsigned)std::min<size_t>(slots, kMaxBlocks);
  if (a.dtype == SV_BF16) {
    hipLaunchKernelGGL(k_rows_generic<Bf16>, dim3(grid), dim3(kNT), 0, st,
                       (const uint16_t*)a.target, (const uint16_t*)a.draft, a.tokens, a.m, a.rule,
                       a.sampling, a.sess_status, a.B, a.M, a.V, a.rows, a.draw_flag,
                       a.draw_token);
  } else {
    hipLaunchKernelGGL(k_rows_generic<F32>, dim3(grid), dim3(kNT), 0, st,
                       (const uint32_t*)a.target, (const uint32_t*)a.draft, a.tokens, a.m, a.rule,
                       a.sampling, a.sess_status, a.B, a.M, a.V, a.rows, a.draw_flag,
                       a.draw_token);
  }
}

}  // namespace sv
