// sv_session.hip -- the per-session kernel of libspecverify, one workgroup
// per session:
//   its first wave (lane i = position i+1) takes the acceptance rule, with a
//   64-bit ballot for the first rejection, and draws the additional token
//   from listed supports;
//   the whole workgroup draws the additional token, as an inverse CDF over
//   ascending token ids, when the rows have no listed support.
#include "sv_kernels.hpp"

namespace sv {

namespace {

// Inverse CDF over a listed support (ids ascending): the additional token is
// the smallest id whose running mass exceeds u * S (the largest id with mass
// if rounding leaves none).  With a q list (qid_g) or a published q row (qrow)
// the weights are the residual max(0, p - q), zero where p is zero; a residual
// without mass falls back to p.  A published row is read only at the listed ids
// with p > 0, and *bad is set if such an entry is not a finite non-negative
// number.  One wave; lane j holds entry j.
__device__ int32_t listed_draw(const int32_t* p_id, const double* p_pr, int np,
                               const int32_t* qid_g, const double* qp_g, int nq,
                               const float* qrow, double u, int32_t* q_id, double* q_p,
                               bool* bad) {
  const int lane = __lane_id();
  const int32_t y = lane < np ? p_id[lane] : 0x7FFFFFFF;
  const double p = lane < np ? p_pr[lane] : 0.0;
  double w = p;
  if (qid_g || qrow) {
    double q = 0.0;
    if (qrow) {
      const bool read = lane < np && p > 0.0;
      q = read ? (double)qrow[y] : 0.0;
      if (__any(read && !(q >= 0.0 && q < INFINITY))) *bad = true;
    } else {
      if (lane < nq) {
      q_id[lane] = qid_g[lane];
      q_p[lane] = qp_g[lane];
    }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      // q(y): binary search of y in the q list
      int lo = 0, hi = nq;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (q_id[mid] < y) lo = mid + 1;
        else hi = mid;
      }
      q = (lane < np && lo < nq && q_id[lo] == y) ? q_p[lo] : 0.0;
    }
    const double d = p - q;
    w = (p > 0.0 && d > 0.0) ? d : 0.0;
    double S = w;
    for (int off = kWave / 2; off > 0; off >>= 1) S += __shfl_xor(S, off, kWave);
    if (S == 0.0) w = p;  // rounding only
  }
  double C = w;
  for (int off = 1; off < kWave; off <<= 1) {
    const double t = __shfl_up(C, off, kWave);
    if (lane >= off) C += t;
  }
  const double S = __shfl(C, kWave - 1, kWave);
  const double tgt = u * S;
  const uint64_t hit = __ballot(lane < np && C > tgt);
  const uint64_t pos = __ballot(lane < np && w > 0.0);
  const int j = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : 0);
  return __shfl(y, j, kWave);
}

// A failed session's outputs, by one wave: status, no tokens, no probes.  The
// per-session kernel's first wave writes these and the session's other
// outputs with the same lane-to-address mapping, so a later failure
// overwrites them in each lane's program order.
__device__ void write_failed(int b, int st, int M, int32_t* __restrict__ accepted_len,
                             int32_t* __restrict__ out_tokens, double* __restrict__ p_tok,
                             double* __restrict__ q_tok) {
  const int lane = threadIdx.x;
  int32_t* out = out_tokens + (size_t)b * (M + 1);
  if (lane == 0) accepted_len[b] = st;
  for (int j = lane; j <= M; j += kWave) out[j] = -1;
  for (int j = lane; j < M; j += kWave) {
    if (p_tok) p_tok[(size_t)b * M + j] = -1.0;
    if (q_tok) q_tok[(size_t)b * M + j] = -1.0;
  }
}

// SDCP Sec. 6.4, for session b, by one wave: lane i examines position i+1.
// With published q rows (qrows != null) q_i(x_i) is read from them and no
// draft row record exists.
// Writes accepted_len, out_tokens and the probes; returns the draw left for
// the whole workgroup (kJobNone when the extra token is already written).
__device__ Job finalize_session(int b, const int32_t* __restrict__ tokens,
                                const int32_t* __restrict__ m, const int32_t* __restrict__ rule,
                                const sv_sampling* __restrict__ sampling, int M, int V,
                                const float* __restrict__ qrows, uint64_t seed,
                                uint32_t round, const int32_t* __restrict__ sess_status,
                                const RowRec* __restrict__ rows, int32_t* __restrict__ accepted_len,
                                int32_t* __restrict__ out_tokens, double* __restrict__ p_tok,
                                double* __restrict__ q_tok, const int32_t* __restrict__ sup_id,
                                const double* __restrict__ sup_p, const double* __restrict__ unif,
                                int32_t* q_id, double* q_p) {
  const int lane = threadIdx.x;
  const int R = 2 * M + 1;
  Job job{kJobNone, 0, 0, 0, 0.0};
  const RowRec* rr = rows + (size_t)b * R;
  int32_t* out = out_tokens + (size_t)b * (M + 1);
  int st = sess_status[b];
  const int mb = m[b];
  const int rl = rule[b];
  const int32_t x = (st == 0 && lane < mb) ? tokens[(size_t)b * M + lane] : -1;

  // every row the rule reads must be usable (target rows 1..m+1, draft rows 1..m)
  if (st == 0) {
    bool bad = false;
    for (int j = lane; j <= mb; j += kWave) bad |= rr[j].status != 0;
    if (rl == SV_RULE_SPECULATIVE && !qrows && lane < mb) bad |= rr[M + 1 + lane].status != 0;
    if (__any(bad)) st = SV_S_BAD_LOGITS;
  }
  // Sec. 6.3 step 5: q_i(x_i) != 0 at every position, before any draw
  // (x is in [0, V) once the session's checks passed); a q value that is not a
  // positive finite number (only a published row can hold one) is unusable
  double qx = 1.0, px = -1.0;
  if (st == 0 && rl == SV_RULE_SPECULATIVE) {
    if (lane < mb) {
      qx = qrows ? (double)qrows[((size_t)b * M + lane) * (size_t)V + x] : rr[M + 1 + lane].ptok;
      px = rr[lane].ptok;
    }
    if (__any(lane < mb && !(qx > 0.0 && qx < INFINITY))) st = SV_S_BAD_PROPOSAL;
  }
  if (st == 0 && rl == SV_RULE_RELAXED && lane < mb) px = rr[lane].ptok;

  if (st < 0) {
    write_failed(b, st, M, accepted_len, out_tokens, p_tok, q_tok);
    return job;
  }

  int a;
  int32_t extra = -1;
  if (rl == SV_RULE_GREEDY) {
    // Rule 1: accept while x_i == argmax p_i; additional token argmax p_{a+1}
    const bool acc = lane < mb && x == rr[lane].argmax;
    const uint64_t rej = ~(uint64_t)__ballot(acc);
    a = rej == 0 ? kWave : __builtin_ctzll(rej);
    a = a < mb ? a : mb;
    extra = rr[a].argmax;
  } else if (rl == SV_RULE_RELAXED) {
    // relaxed rule (private use 192): accept x_i while p_i(x_i) > 0; the
    // additional token is drawn from p_{a+1} with the purpose-1 value of
    // position a+1, from the listed support or by the whole workgroup
    const bool acc = lane < mb && px > 0.0;
    const uint64_t rej = ~(uint64_t)__ballot(acc);
    a = rej == 0 ? kWave : __builtin_ctzll(rej);
    a = a < mb ? a : mb;
    double ua, ud;
    if (unif) ud = unif[(size_t)b * R + M + a];
    else verifier_uniforms(seed, sampling[b].session_key, round, (uint32_t)(a + 1), &ua, &ud);
    const RowRec& P = rr[a];
    if (P.nsup > 0) {
      bool bad = false;
      extra = listed_draw(sup_id + ((size_t)b * R + a) * kSupMax,
                          sup_p + ((size_t)b * R + a) * kSupMax, P.nsup, nullptr, nullptr, 0,
                          nullptr, ud, q_id, q_p, &bad);
    } else {
      job = Job{kJobBonus, a, a, -1, ud};
    }
  } else {
    // Rule 2: accept x_i if u_acc(i) < min(1, p_i(x_i) / q_i(x_i)); the values
    // are SDCP's (computed by the row kernel into unif) or Philox's
    const double* uv = unif ? unif + (size_t)b * R : nullptr;
    double u_acc = 1.0, u_add = 0.0;
    if (uv) u_acc = lane < mb ? uv[lane] : 1.0;
    else verifier_uniforms(seed, sampling[b].session_key, round, (uint32_t)(lane + 1), &u_acc, &u_add);
    const double ratio = px / qx;
    const bool acc = lane < mb && u_acc < (ratio < 1.0 ? ratio : 1.0);
    const uint64_t rej = ~(uint64_t)__ballot(acc);
    a = rej == 0 ? kWave : __builtin_ctzll(rej);
    a = a < mb ? a : mb;
    double ua, ud;
    if (uv) ud = uv[M + a];
    else verifier_uniforms(seed, sampling[b].session_key, round, (uint32_t)(a + 1), &ua, &ud);
    // additional token: residual at the first rejection, else the bonus row;
    // drawn here when the rows' supports are listed, else by the sampler
    const RowRec& P = rr[a];
    const RowRec* Q = (a < mb && !qrows) ? &rr[M + 1 + a] : nullptr;
    const float* qrow = (a < mb && qrows) ? qrows + ((size_t)b * M + a) * (size_t)V : nullptr;
    if (P.nsup > 0 && (Q == nullptr || Q->nsup > 0)) {
      bool bad = false;
      extra = listed_draw(sup_id + ((size_t)b * R + a) * kSupMax,
                          sup_p + ((size_t)b * R + a) * kSupMax, P.nsup,
                          Q ? sup_id + ((size_t)b * R + M + 1 + a) * kSupMax : nullptr,
                          Q ? sup_p + ((size_t)b * R + M + 1 + a) * kSupMax : nullptr,
                          Q ? Q->nsup : 0, qrow, ud, q_id, q_p, &bad);
      if (bad) {  // an unusable entry of the published residual row
        write_failed(b, SV_S_BAD_PROPOSAL, M, accepted_len, out_tokens, p_tok, q_tok);
        return job;
      }
    } else {
      job = a < mb ? Job{kJobResidual, a, a, a, ud} : Job{kJobBonus, a, mb, -1, ud};
    }
  }
  if (lane == 0) accepted_len[b] = a;
  for (int j = lane; j <= M; j += kWave) {
    int32_t v = -1;
    if (j < a) v = x;  // j < a <= 64 means j == lane
    else if (j == a) v = extra;  // -1: written by the sampling kernel
    out[j] = v;
  }
  for (int j = lane; j < M; j += kWave) {
    const bool have_p = (rl == SV_RULE_SPECULATIVE || rl == SV_RULE_RELAXED) && j < mb;
    const bool have_q = rl == SV_RULE_SPECULATIVE && j < mb;
    if (p_tok) p_tok[(size_t)b * M + j] = have_p ? px : -1.0;
    if (q_tok) q_tok[(size_t)b * M + j] = have_q ? qx : -1.0;
  }
  return job;
}

constexpr int kSampleNT = 1024;                  // threads per session
constexpr int kSampleWaves = kSampleNT / kWave;  // waves per session
constexpr int kSub = kWave * 4;                  // ids per sub-block: 4 consecutive per lane
constexpr int kMaxGroups = kSampleNT;            // groups of whole sub-blocks (one per thread)
constexpr int kLut = 2048;                       // probabilities tabled per row (by key)

// One row's profile as the sampler sees it: p(y) = w(y) / Z' on the support.
// A row whose cut is recorded as (kcut, ntie) keeps the ntie smallest ids among
// the tokens of key kcut; the sampler counts those ties in id order.  The
// probabilities of the kLut keys below the row's largest key are tabled in
// LDS (a top-p support lies there); other keys evaluate the weight.
template <class Tr>
struct SampleRow {
  const typename Tr::elem_t* row;
  RowRec r;
  uint32_t ktop;      // key of the row's largest logit
  const double* lut;  // lut[ktop - k] = p of key k, for ktop - kLut < k <= ktop
  __device__ bool tie_mode() const { return r.idcut < 0; }
  // probability of token y with bits u; rank = ties of key kcut before y (tie mode)
  __device__ double prob(int y, uint32_t u, int rank) const {
    const uint32_t k = Tr::key(u);
    const bool member = k > r.kcut || (k == r.kcut && (r.idcut >= 0 ? y <= r.idcut : rank < r.ntie));
    if (!member) return 0.0;
    if (ktop - k < (uint32_t)kLut) return lut[ktop - k];
    return weight64(Tr::value(u), r.lmax, r.scale) / r.zsum;
  }
};

// Fill a row's table: p of the keys ktop, ktop - 1, ... (keys at or below
// -inf get 0).  Entries are the same expression the direct path evaluates.
template <class Tr>
__device__ void fill_lut(SampleRow<Tr>& S, double* lut) {
  S.ktop = Tr::key(__float_as_uint(S.r.lmax) >> (32 - Tr::kKeyBits));
  S.lut = lut;
  for (int i = threadIdx.x; i < kLut; i += blockDim.x) {
    const long k = (long)S.ktop - i;
    double p = 0.0;
    if (k > (long)Tr::kNegInfKey)
      p = weight64(Tr::value(Tr::unkey((uint32_t)k)), S.r.lmax, S.r.scale) / S.r.zsum;
    lut[i] = p;
  }
}

// Block-wide exclusive scan in thread order (fixed combination order).
template <typename T>
__device__ T block_exclusive_scan(T v, T* wsum, T* total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  T inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const T t = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += t;
  }
  T exc = __shfl_up(inc, 1, kWave);
  if (lane == 0) exc = T(0);
  __syncthreads();
  if (lane == kWave - 1) wsum[wid] = inc;
  __syncthreads();
  T base = T(0), tot = T(0);
#pragma unroll
  for (int w = 0; w < kSampleNT / kWave; ++w) {
    if (w < wid) base += wsum[w];
    tot += wsum[w];
  }
  *total = tot;
  return base + exc;
}

struct SampleSmem {
  double lut_p[kLut];         // p of the keys below p's largest key
  double lut_q[kLut];         // q of the keys below q's largest key
  double mass[kMaxGroups];    // weight of each group
  uint64_t ties[kMaxGroups];  // the cut keys' ties in each group (p low word, q high), then before it
  double dsum[kSampleWaves];
  uint64_t usum[kSampleWaves];
  int32_t ired[kSampleWaves];
  double base;
};

// The draw of one session's additional token: weights w(y) = max(0, p(y) -
// q(y)) (zero where p is zero) for the residual, or p(y); the smallest id
// whose running weight exceeds u * S.
template <class Tr, bool kQ>
struct Draw {
  SampleRow<Tr> P, Q;  // Q unused with kQ
  const float* qrow;   // the published q row (kQ)
  bool resid;
  int V;
};

// Bits of this lane's 4 consecutive ids of the sub-block starting at y0.
template <class Tr, bool kQ>
__device__ inline void sub_load(const Draw<Tr, kQ>& d, int y0, uint32_t (&up)[4],
                                uint32_t (&uq)[4]) {
  const int y = y0 + 4 * __lane_id();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool in = y + e < d.V;
    up[e] = in ? Tr::bits(d.P.row[y + e]) : Tr::kNegInfBits;
    if constexpr (kQ) uq[e] = (in && d.resid) ? __float_as_uint(d.qrow[y + e]) : 0u;
    else uq[e] = (in && d.resid) ? Tr::bits(d.Q.row[y + e]) : Tr::kNegInfBits;
  }
}

// Which of the 4 ids hold a cut key whose ties are kept by rank: bit e for p,
// bit 4 + e for q.
template <class Tr, bool kQ>
__device__ inline uint32_t sub_tie_bits(const Draw<Tr, kQ>& d, const uint32_t (&up)[4],
                                        const uint32_t (&uq)[4]) {
  uint32_t f = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (d.P.tie_mode() && Tr::key(up[e]) == d.P.r.kcut) f |= 1u << e;
    if (!kQ && d.resid && d.Q.tie_mode() && Tr::key(uq[e]) == d.Q.r.kcut) f |= 16u << e;
  }
  return f;
}

// Exclusive prefix over the wave's lanes of a small count (0..7), and the
// wave total, from one ballot per bit.
__device__ inline int wave_excl_small(int c, int* total) {
  int r = 0, t = 0;
#pragma unroll
  for (int bit = 0; bit < 3; ++bit) {
    const uint64_t bm = __ballot((c >> bit) & 1);
    r += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0)) << bit;
    t += __builtin_popcountll(bm) << bit;
  }
  *total = t;
  return r;
}

// Weights of this lane's 4 ids of a sub-block.  rp, rq: the cut keys' ties
// before the sub-block (wave-uniform); on return they count its ties too.
template <class Tr, bool kQ>
__device__ inline void sub_weights(const Draw<Tr, kQ>& d, int y0, const uint32_t (&up)[4],
                                   const uint32_t (&uq)[4], uint32_t& rp, uint32_t& rq,
                                   double (&w)[4], bool& bad) {
  const uint32_t f = sub_tie_bits<Tr, kQ>(d, up, uq);
  int tp, tq;
  const int bp = wave_excl_small(__builtin_popcount(f & 15u), &tp);
  const int bq = wave_excl_small(__builtin_popcount(f >> 4), &tq);
  int cp = (int)rp + bp, cq = (int)rq + bq;
  const int y = y0 + 4 * __lane_id();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double p = d.P.prob(y + e, up[e], cp);
    if (!d.resid) {
      w[e] = p;
    } else {
      double q;
      if constexpr (kQ) {
        q = (double)__uint_as_float(uq[e]);
        bad |= p > 0.0 && !(q >= 0.0 && q < INFINITY);
      } else {
        q = d.Q.prob(y + e, uq[e], cq);
      }
      const double df = p - q;
      w[e] = (p > 0.0 && df > 0.0) ? df : 0.0;
    }
    cp += (f >> e) & 1u;
    cq += (f >> (4 + e)) & 1u;
  }
  rp += (uint32_t)tp;
  rq += (uint32_t)tq;
}

// Calls fn(y0, up, uq) for the sub-blocks of [lo, hi) in order (lo and hi on
// sub-block boundaries, or hi = V).  (Loading four sub-blocks ahead measured
// slower: the registers it needs push the kernel to its limit.)
template <class Tr, bool kQ, class F>
__device__ inline void stream_subs(const Draw<Tr, kQ>& d, int lo, int hi, F&& fn) {
  for (int y0 = lo; y0 < hi; y0 += kSub) {
    uint32_t up[4], uq[4];
    sub_load<Tr, kQ>(d, y0, up, uq);
    fn(y0, up, uq);
  }
}

__device__ inline double wave_incl_scan(double v) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// Textbook "The acceptance rule" / SDCP Sec. 6.4 Rule 2: additional token from
// norm(max(0, p_j - q_j)) at the first rejection j, or from p_{m+1}; the
// smallest id whose running weight exceeds u * S.  One workgroup per session:
// its first wave takes the acceptance decisions (finalize_session); a draw
// from rows without listed supports then takes the whole workgroup.
// The row is cut into at most kMaxGroups groups of whole sub-blocks; each wave
// owns a run of consecutive groups and streams them with no workgroup barrier:
// a first pass counts the cut keys' ties per group when they are kept by rank
// (a workgroup scan then gives each group its ties before it), a second pass
// weighs every group; a scan over the group weights finds the group holding
// u * S, which one wave weighs again with a wave scan.
template <class Tr, bool kQ>
__global__ __launch_bounds__(kSampleNT) void k_finalize(
    const typename Tr::elem_t* __restrict__ target, const typename Tr::elem_t* __restrict__ draft,
    const float* __restrict__ qrows, const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling, int B, int M, int V,
    uint64_t seed, uint32_t round, const int32_t* __restrict__ sess_status,
    const RowRec* __restrict__ rows, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, double* __restrict__ p_tok, double* __restrict__ q_tok,
    const int32_t* __restrict__ sup_id, const double* __restrict__ sup_p,
    const double* __restrict__ unif) {
  __shared__ SampleSmem sm;
  __shared__ int32_t q_id[kSupMax];
  __shared__ double q_p[kSupMax];
  __shared__ Job job_s;
  const int b = blockIdx.x;
  if (b >= B) return;
  if (threadIdx.x < kWave) {
    const Job j = finalize_session(b, tokens, m, rule, sampling, M, V, kQ ? qrows : nullptr, seed,
                                   round, sess_status, rows,
                                   accepted_len, out_tokens, p_tok, q_tok, sup_id, sup_p, unif,
                                   q_id, q_p);
    if (threadIdx.x == 0) job_s = j;
  }
  __syncthreads();
  const Job job = job_s;
  if (job.kind == kJobNone) return;
  const int R = 2 * M + 1;
  Draw<Tr, kQ> d;
  d.P = SampleRow<Tr>{target + ((size_t)b * (M + 1) + job.trow) * (size_t)V,
                      rows[(size_t)b * R + job.trow], 0, nullptr};
  d.Q = d.P;
  d.qrow = nullptr;
  d.resid = job.kind == kJobResidual;
  d.V = V;
  if (d.resid) {
    if constexpr (kQ) d.qrow = qrows + ((size_t)b * M + job.drow) * (size_t)V;
    else d.Q = SampleRow<Tr>{draft + ((size_t)b * M + job.drow) * (size_t)V,
                             rows[(size_t)b * R + M + 1 + job.drow], 0, nullptr};
  }
  fill_lut<Tr>(d.P, sm.lut_p);
  if (!kQ) fill_lut<Tr>(d.Q, sm.lut_q);

  // groups: at most kMaxGroups runs of Lg ids (whole sub-blocks); wave w owns
  // groups [g0, g1)
  const int nsub = (V + kSub - 1) / kSub;
  const int sub_per_group = (nsub + kMaxGroups - 1) / kMaxGroups;
  const int Lg = sub_per_group * kSub;
  const int ng = (V + Lg - 1) / Lg;
  const int wid = (int)threadIdx.x / kWave, lane = __lane_id();
  const int g0 = wid * ng / kSampleWaves, g1 = (wid + 1) * ng / kSampleWaves;
  const bool ties = d.P.tie_mode() || (!kQ && d.resid && d.Q.tie_mode());

  // the ties of each group, then of all groups before it
  const int lo = g0 * Lg, hi = min(g1 * Lg, V);  // this wave's ids
  if (ties) {
    uint32_t cp = 0, cq = 0;
    stream_subs<Tr, kQ>(d, lo, hi, [&](int y0, const uint32_t(&up)[4], const uint32_t(&uq)[4]) {
      const uint32_t f = sub_tie_bits<Tr, kQ>(d, up, uq);
      cp += __builtin_popcount(f & 15u);
      cq += __builtin_popcount(f >> 4);
      const int g = y0 / Lg;
      if (y0 + kSub >= min((g + 1) * Lg, V)) {  // the group's last sub-block
        const uint64_t c = wave_reduce((uint64_t)cp | ((uint64_t)cq << 32), OpAdd());
        if (lane == 0) sm.ties[g] = c;
        cp = cq = 0;
      }
    });
    __syncthreads();
    uint64_t tot;
    const uint64_t c = (int)threadIdx.x < ng ? sm.ties[threadIdx.x] : 0ull;
    const uint64_t before = block_exclusive_scan<uint64_t>(c, sm.usum, &tot);
    if ((int)threadIdx.x < ng) sm.ties[threadIdx.x] = before;
  }
  __syncthreads();  // tables and tie counts are ready

  // every group's weight, and the last id with weight
  int32_t last = -1;
  bool bad = false;
  for (int attempt = 0; attempt < 2; ++attempt) {
    last = -1;
    uint32_t rp = 0, rq = 0;
    double acc = 0.0;
    stream_subs<Tr, kQ>(d, lo, hi, [&](int y0, const uint32_t(&up)[4], const uint32_t(&uq)[4]) {
      const int g = y0 / Lg;
      if (ties && y0 == g * Lg) {  // the ties before the group
        rp = (uint32_t)sm.ties[g];
        rq = (uint32_t)(sm.ties[g] >> 32);
      }
      double w[4];
      sub_weights<Tr, kQ>(d, y0, up, uq, rp, rq, w, bad);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += w[e];
        if (w[e] > 0.0) last = y0 + 4 * lane + e;
      }
      if (y0 + kSub >= min((g + 1) * Lg, V)) {  // the group's last sub-block
        const double gm = wave_reduce(acc, OpAdd());
        if (lane == 0) sm.mass[g] = gm;
        acc = 0.0;
      }
    });
    last = block_reduce<kSampleNT>(last, OpMax(), sm.ired);
    if (kQ && d.resid && attempt == 0) {
      // an unusable entry of the published residual row fails the session; the
      // first wave rewrites its outputs as it wrote them
      if (block_reduce<kSampleNT>(bad ? 1 : 0, OpMax(), sm.ired) != 0) {
        if (threadIdx.x < kWave)
          write_failed(b, SV_S_BAD_PROPOSAL, M, accepted_len, out_tokens, p_tok, q_tok);
        return;
      }
    }
    if (!d.resid || last >= 0) break;
    d.resid = false;  // residual without mass (rounding only): draw from p
    __syncthreads();  // the group weights are written again
  }

  // the group holding u * S (thread g holds group g)
  __syncthreads();
  const double gm = (int)threadIdx.x < ng ? sm.mass[threadIdx.x] : 0.0;
  double S;
  const double before = block_exclusive_scan<double>(gm, sm.dsum, &S);
  const double tgt = job.u * S;
  const int32_t mine_g = ((int)threadIdx.x < ng && before + gm > tgt) ? (int32_t)threadIdx.x : 0x7FFFFFFF;
  const int32_t gstar = block_reduce<kSampleNT>(mine_g, OpMin(), sm.ired);
  if (gstar == 0x7FFFFFFF) {
    if (threadIdx.x == 0) out_tokens[(size_t)b * (M + 1) + job.pos] = last;
    return;
  }
  if ((int)threadIdx.x == gstar) sm.base = before;
  __syncthreads();
  if (wid != 0) return;
  // the first wave weighs the group again, sub-block by sub-block, and goes on
  // past it if rounding moved the point
  double run = sm.base;
  int32_t pick = last;
  bool found = false;
  for (int g = gstar; g < ng && !found; ++g) {
    uint32_t rp = ties ? (uint32_t)sm.ties[g] : 0u, rq = ties ? (uint32_t)(sm.ties[g] >> 32) : 0u;
    for (int y0 = g * Lg; y0 < min((g + 1) * Lg, V); y0 += kSub) {
      uint32_t up[4], uq[4];
      sub_load<Tr, kQ>(d, y0, up, uq);
      double w[4];
      sub_weights<Tr, kQ>(d, y0, up, uq, rp, rq, w, bad);
      const double ls = (w[0] + w[1]) + (w[2] + w[3]);
      const double incl = wave_incl_scan(ls);
      double a = run + (incl - ls);
      int32_t mine = 0x7FFFFFFF;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a += w[e];
        if (mine == 0x7FFFFFFF && a > tgt) mine = y0 + 4 * lane + e;
      }
      const int32_t first = wave_reduce(mine, OpMin());
      if (first != 0x7FFFFFFF) {
        pick = first;
        found = true;
        break;
      }
      run += __shfl(incl, kWave - 1, kWave);
    }
  }
  if (lane == 0) out_tokens[(size_t)b * (M + 1) + job.pos] = pick;
}

}  // namespace

template <class Tr, bool kQ>
static void launch_finalize_t(const LaunchArgs& a, hipStream_t st) {
  using E = typename Tr::elem_t;
  hipLaunchKernelGGL((k_finalize<Tr, kQ>), dim3(a.B), dim3(kSampleNT), 0, st, (const E*)a.target,
                     (const E*)a.draft, a.qrows, a.tokens, a.m, a.rule, a.sampling, a.B, a.M, a.V,
                     a.seed, a.round, a.sess_status, a.rows, a.accepted_len, a.out_tokens, a.p_tok,
                     a.q_tok, a.sup_id, a.sup_p, a.unif);
}

void launch_finalize(const LaunchArgs& a, hipStream_t st) {
  const bool q = a.qrows != nullptr;
  if (a.dtype == SV_BF16) {
    if (q) launch_finalize_t<Bf16, true>(a, st);
    else launch_finalize_t<Bf16, false>(a, st);
  } else {
    if (q) launch_finalize_t<F32, true>(a, st);
    else launch_finalize_t<F32, false>(a, st);
  }
}

}  // namespace sv
