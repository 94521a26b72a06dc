// sv_session.hip -- the per-session kernels of libspecverify.
// k_finalize: a session takes C workgroups (one per chunk of its vocabulary):
//   the first wave of each takes the acceptance rule (lane i = position i+1,
//   a 64-bit ballot for the first rejection); chunk 0's workgroup draws the
//   additional token from listed supports and writes the session's outputs;
//   when the rows have no listed support, the additional token is an inverse
//   CDF over ascending token ids: each workgroup weighs its chunk, and the
//   session's last workgroup picks the token and writes the outputs.
// k_advance (the in-order reading, between windows of positions): one wave
//   per undecided session finds the position that ends its round, if the
//   rows read so far hold it.
#include "sv_kernels.hpp"
#include "sv_stream.hpp"

namespace sv {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
    const double S = wave_reduce(w, OpAdd());
    if (S == 0.0) w = p;  // rounding only
  }
  const double C = wave_incl_scan(w);
  const double S = lane_read(C, kWave - 1);
  const double tgt = u * S;
  const uint64_t hit = __ballot(lane < np && C > tgt);
  const uint64_t pos = __ballot(lane < np && w > 0.0);
  const int j = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : 0);
  return lane_read(y, j);
}

// A failed session's outputs, by one wave: status, no tokens, no probes.  The
// per-session kernel's first wave writes these and the session's other
// outputs with the same lane-to-address mapping, so a later failure
// overwrites them in each lane's program order.
__device__ __attribute__((always_inline)) void write_failed(
    int b, int st, int M, int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    double* __restrict__ p_tok, double* __restrict__ q_tok) {
  const int lane = threadIdx.x;
  int32_t* out = out_tokens + (size_t)b * (M + 1);
  if (lane == 0) accepted_len[b] = st;
  for (int j = lane; j <= M; j += kWave) out[j] = -1;
  for (int j = lane; j < M; j += kWave) {
    if (p_tok) p_tok[(size_t)b * M + j] = -1.0;
    if (q_tok) q_tok[(size_t)b * M + j] = -1.0;
  }
}

// One session's acceptance verdict, held by the lanes of one wave (lane i:
// position i+1).
struct Verdict {
  int st;         // 0, or the session's failure status
  int a;          // accepted drafted tokens
  int rl, mb;     // rule, drafted tokens
  int np;         // positions with probe values: mb, or fewer when read in order
  int32_t x;      // this lane's drafted token (-1 past m)
  double px, qx;  // this lane's p_i(x_i) and q_i(x_i)
  int32_t extra;  // the additional token, when already drawn
  Job job;        // the draw left to the chunked sampler (kJobNone: none)
};

// What lane i of a session's wave knows of position i+1 once its rows are
// profiled: the drafted token, p_i(x_i) and q_i(x_i) where the rule reads
// them (-1 and 1 elsewhere), and the acceptance value of rule 2 (1 elsewhere).
// Only positions before lim are read.
struct LanePos {
  int32_t x;
  double px, qx, u;
};

__device__ __attribute__((always_inline)) LanePos lane_position(
    int b, int lane, int mb, int lim, int rl, const int32_t* __restrict__ tokens, int M, int V,
    const float* __restrict__ qrows, const RowRec* __restrict__ rr,
    const double* __restrict__ unif, uint64_t seed, uint64_t session_key, uint32_t round) {
  LanePos P{-1, -1.0, 1.0, 1.0};
  if (lane >= mb || lane >= lim) return P;
  P.x = tokens[(size_t)b * M + lane];  // in [0, V) once the session's checks passed
  if (rl == SV_RULE_SPECULATIVE || rl == SV_RULE_RELAXED) P.px = rr[lane].ptok;
  if (rl == SV_RULE_SPECULATIVE) {
    P.qx = qrows ? (double)qrows[((size_t)b * M + lane) * (size_t)V + P.x] : rr[M + 1 + lane].ptok;
    double ud;
    if (unif) P.u = unif[(size_t)b * (2 * M + 1) + lane];
    else verifier_uniforms(seed, session_key, round, (uint32_t)(lane + 1), &P.u, &ud);
  }
  return P;
}

// The in-order reading of a session (textbook "The acceptance rule": the
// proposals are checked one after another, and the first rejection ends the
// round): the first of positions 1..n (lane j: position j+1) at which the
// round ends, as a 1-based position, or 0 if none does.  A position ends it
// with a bad target row (or bad draft row), an unusable q_i(x_i), or a failed
// test; position m+1 (the additional token's row) with a bad row only.
__device__ __attribute__((always_inline)) int inorder_end(int n, int mb, int rl, bool draft_rows,
                                                          const RowRec* __restrict__ rr, int M,
                                                          const LanePos& P) {
  const int lane = threadIdx.x & (kWave - 1);
  bool end = false;
  if (lane < n) {
    end = rr[lane].status != 0;
    if (lane < mb) {
      if (rl == SV_RULE_GREEDY) {
        end |= P.x != rr[lane].argmax;
      } else if (rl == SV_RULE_RELAXED) {
        end |= !(P.px > 0.0);
      } else {
        if (draft_rows) end |= rr[M + 1 + lane].status != 0;
        const double ratio = P.px / P.qx;
        end |= !(P.qx > 0.0 && P.qx < INFINITY) || !(P.u < (ratio < 1.0 ? ratio : 1.0));
      }
    }
  }
  const uint64_t e = __ballot(end);
  // position 65 (m = 64, lane 64 does not exist): its row alone
  if (e == 0 && n > kWave && rr[kWave].status != 0) return kWave + 1;
  return e ? __builtin_ctzll(e) + 1 : 0;
}

// What lane j reads of position j+1's rows, loaded at once before the
// session's checks: every address is in bounds for any m (target rows 0..M,
// draft rows and drafted tokens 0..M-1), so no load waits for m, the rule or
// the status.  Lane j holds the target row record's status, argmax, listed
// support size and p of the drafted token; below M the draft row record's
// status, support size and q of the drafted token, and the drafted token;
// and the verifier values of position j+1 (both words of one Philox call, or
// the SDCP table's entries).  Position M+1 = 65 (M = 64) has no lane: the
// callers read its row record where they need it.
struct LaneRows {
  int32_t ts, targ, tn;  // target row: status, argmax, nsup
  double tp;             // target row: ptok
  int32_t ds, dn;        // draft row: status, nsup
  double dp;             // draft row: ptok
  int32_t x;             // drafted token
  double ua, ud;         // acceptance and additional-token values
};
__device__ __attribute__((always_inline)) LaneRows lane_rows(
    int b, int lane, int M, const int32_t* __restrict__ tokens, const RowRec* __restrict__ rr,
    const double* __restrict__ unif, uint64_t seed, uint64_t session_key, uint32_t round) {
  LaneRows r{0, -1, 0, -1.0, 0, 0, 1.0, -1, 1.0, 1.0};
  if (lane <= M) {
    const RowRec& t = rr[lane];
    r.ts = t.status;
    r.targ = t.argmax;
    r.tn = t.nsup;
    r.tp = t.ptok;
  }
  if (lane < M) {
    const RowRec& d = rr[M + 1 + lane];
    r.ds = d.status;
    r.dn = d.nsup;
    r.dp = d.ptok;
    r.x = tokens[(size_t)b * M + lane];
  }
  if (unif) {
    const int R = 2 * M + 1;
    if (lane < M) r.ua = unif[(size_t)b * R + lane];
    if (lane <= M) r.ud = unif[(size_t)b * R + M + lane];
  } else {
    verifier_uniforms(seed, session_key, round, (uint32_t)(lane + 1), &r.ua, &r.ud);
  }
  return r;
}

// lane_position from a lane's loaded rows (see lane_position).
__device__ __attribute__((always_inline)) LanePos lane_position_lr(
    const LaneRows& Lr, int b, int lane, int mb, int lim, int rl, int M, int V,
    const float* __restrict__ qrows) {
  LanePos P{-1, -1.0, 1.0, 1.0};
  if (lane >= mb || lane >= lim) return P;
  P.x = Lr.x;  // in [0, V) once the session's checks passed
  if (rl == SV_RULE_SPECULATIVE || rl == SV_RULE_RELAXED) P.px = Lr.tp;
  if (rl == SV_RULE_SPECULATIVE) {
    P.qx = qrows ? (double)qrows[((size_t)b * M + lane) * (size_t)V + P.x] : Lr.dp;
    P.u = Lr.ua;
  }
  return P;
}

// inorder_end from a lane's loaded rows (see inorder_end).
__device__ __attribute__((always_inline)) int inorder_end_lr(int n, int mb, int rl,
                                                             bool draft_rows, const LaneRows& Lr,
                                                             const RowRec* __restrict__ rr,
                                                             const LanePos& P) {
  const int lane = threadIdx.x & (kWave - 1);
  bool end = false;
  if (lane < n) {
    end = Lr.ts != 0;
    if (lane < mb) {
      if (rl == SV_RULE_GREEDY) {
        end |= P.x != Lr.targ;
      } else if (rl == SV_RULE_RELAXED) {
        end |= !(P.px > 0.0);
      } else {
        if (draft_rows) end |= Lr.ds != 0;
        const double ratio = P.px / P.qx;
        end |= !(P.qx > 0.0 && P.qx < INFINITY) || !(P.u < (ratio < 1.0 ? ratio : 1.0));
      }
    }
  }
  const uint64_t e = __ballot(end);
  // position 65 (m = 64, lane 64 does not exist): its row alone
  if (e == 0 && n > kWave && rr[kWave].status != 0) return kWave + 1;
  return e ? __builtin_ctzll(e) + 1 : 0;
}

// The additional token's value (purpose 1) for position a+1: lane a's, or
// for a = 64 (position 65, no lane) the table's entry or a Philox call.
__device__ __attribute__((always_inline)) double additional_value(
    const LaneRows& Lr, int a, int b, int M, const double* __restrict__ unif, uint64_t seed,
    const sv_sampling* __restrict__ sampling, uint32_t round) {
  if (a < kWave) return lane_read(Lr.ud, a);
  if (unif) return unif[(size_t)b * (2 * M + 1) + M + a];
  double ua, ud;
  verifier_uniforms(seed, sampling[b].session_key, round, (uint32_t)(a + 1), &ua, &ud);
  return ud;
}

// SDCP Sec. 6.4, for session b, by one wave: lane i examines position i+1.
// With published q rows (qrows != null) q_i(x_i) is read from them and no
// draft row record exists.  Writes nothing.  A draw from listed supports is
// taken here when listed is set; otherwise such a session only reports that
// no chunked draw is left (job kind none).  decided != null: the in-order
// reading, whose rows are read up to the position decided[b] (0: up to m+1),
// and statuses and decisions come from those rows alone.
__device__ __attribute__((always_inline)) Verdict accept_session(
    int b, const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling, int M, int V,
    const float* __restrict__ qrows, uint64_t seed, uint32_t round,
    const int32_t* __restrict__ sess_status, const RowRec* __restrict__ rows,
    const int32_t* __restrict__ sup_id, const double* __restrict__ sup_p,
    const double* __restrict__ unif, const int32_t* __restrict__ decided, bool listed,
    int32_t* q_id, double* q_p) {
  const int lane = threadIdx.x;
  const int R = 2 * M + 1;
  Verdict v;
  v.job = Job{kJobNone, 0, 0, 0, 0.0};
  v.a = 0;
  v.extra = -1;
  const RowRec* rr = rows + (size_t)b * R;
  const LaneRows Lr = lane_rows(b, lane, M, tokens, rr, unif, seed, sampling[b].session_key, round);
  int st = sess_status[b];
  const int mb = m[b];
  const int rl = rule[b];
  v.rl = rl;
  v.mb = mb;
  const bool draft_rows = rl == SV_RULE_SPECULATIVE && !qrows;
  // target rows read: 1..L (the SDCP reading: every row, m+1 of them); in
  // order, up to the decided position (all m+1 rows if still undecided)
  const int e = (st == 0 && decided) ? decided[b] : 0;
  const int n = e > 0 ? e : mb + 1;
  LanePos pos{-1, -1.0, 1.0, 1.0};
  if (st == 0) pos = lane_position_lr(Lr, b, lane, mb, n, rl, M, V, qrows);
  int L = mb + 1;
  if (st == 0 && decided) {
    const int f = inorder_end_lr(n, mb, rl, draft_rows, Lr, rr, pos);
    L = f > 0 ? f : n;
  }
  const int np = L < mb ? L : mb;  // positions whose drafted token is examined
  v.np = np;
  const int32_t x = lane < np ? pos.x : -1;
  v.x = x;

  // every row the rule reads must be usable (target rows 1..L, draft rows 1..np)
  if (st == 0) {
    bool bad = lane < L && Lr.ts != 0;
    if (L > kWave && lane == 0) bad |= rr[kWave].status != 0;  // row 65 (M = 64)
    if (draft_rows && lane < np) bad |= Lr.ds != 0;
    if (__any(bad)) st = SV_S_BAD_LOGITS;
  }
  // Sec. 6.3 step 5: q_i(x_i) != 0 at every position examined, before any
  // draw; a q value that is not a positive finite number (only a published
  // row can hold one) is unusable
  double qx = 1.0, px = -1.0;
  if (st == 0 && rl == SV_RULE_SPECULATIVE) {
    if (lane < np) {
      qx = pos.qx;
      px = pos.px;
    }
    if (__any(lane < np && !(qx > 0.0 && qx < INFINITY))) st = SV_S_BAD_PROPOSAL;
  }
  if (st == 0 && rl == SV_RULE_RELAXED && lane < np) px = pos.px;
  v.px = px;
  v.qx = qx;
  v.st = st;
  if (st < 0) return v;

  int a;
  if (rl == SV_RULE_GREEDY) {
    // Rule 1: accept while x_i == argmax p_i; additional token argmax p_{a+1}
    const bool acc = lane < np && x == Lr.targ;
    const uint64_t rej = ~(uint64_t)__ballot(acc);
    a = rej == 0 ? kWave : __builtin_ctzll(rej);
    a = a < mb ? a : mb;
    v.extra = a < kWave ? lane_read(Lr.targ, a) : rr[a].argmax;
  } else if (rl == SV_RULE_RELAXED) {
    // relaxed rule (private use 192): accept x_i while p_i(x_i) > 0; the
    // additional token is drawn from p_{a+1} with the purpose-1 value of
    // position a+1, from the listed support or by the chunked sampler
    const bool acc = lane < np && px > 0.0;
    const uint64_t rej = ~(uint64_t)__ballot(acc);
    a = rej == 0 ? kWave : __builtin_ctzll(rej);
    a = a < mb ? a : mb;
    const double ud = additional_value(Lr, a, b, M, unif, seed, sampling, round);
    const int pn = a < kWave ? lane_read(Lr.tn, a) : rr[a].nsup;
    if (pn > 0) {
      if (listed) {
        bool bad = false;
        v.extra = listed_draw(sup_id + ((size_t)b * R + a) * kSupMax,
                              sup_p + ((size_t)b * R + a) * kSupMax, pn, nullptr, nullptr, 0,
                              nullptr, ud, q_id, q_p, &bad);
      }
    } else {
      v.job = Job{kJobBonus, a, a, -1, ud};
    }
  } else {
    // Rule 2: accept x_i if u_acc(i) < min(1, p_i(x_i) / q_i(x_i)); the values
    // are SDCP's (computed by the row kernel into unif) or Philox's
    const double ratio = px / qx;
    const bool acc = lane < np && pos.u < (ratio < 1.0 ? ratio : 1.0);
    const uint64_t rej = ~(uint64_t)__ballot(acc);
    a = rej == 0 ? kWave : __builtin_ctzll(rej);
    a = a < mb ? a : mb;
    const double ud = additional_value(Lr, a, b, M, unif, seed, sampling, round);
    // additional token: residual at the first rejection, else the bonus row;
    // drawn here when the rows' supports are listed, else by the chunks
    const int pn = a < kWave ? lane_read(Lr.tn, a) : rr[a].nsup;
    const bool draft = a < mb && !qrows;  // a < mb <= 64: lane a exists
    const int qn = draft ? lane_read(Lr.dn, a) : 0;
    const float* qrow = (a < mb && qrows) ? qrows + ((size_t)b * M + a) * (size_t)V : nullptr;
    if (pn > 0 && (!draft || qn > 0)) {
      if (listed) {
        bool bad = false;
        v.extra = listed_draw(sup_id + ((size_t)b * R + a) * kSupMax,
                              sup_p + ((size_t)b * R + a) * kSupMax, pn,
                              draft ? sup_id + ((size_t)b * R + M + 1 + a) * kSupMax : nullptr,
                              draft ? sup_p + ((size_t)b * R + M + 1 + a) * kSupMax : nullptr,
                              qn, qrow, ud, q_id, q_p, &bad);
        if (bad) v.st = SV_S_BAD_PROPOSAL;  // an unusable entry of the published residual row
      }
    } else {
      v.job = a < mb ? Job{kJobResidual, a, a, a, ud} : Job{kJobBonus, a, mb, -1, ud};
    }
  }
  v.a = a;
  return v;
}

// A session's outputs from its verdict and additional token, by one wave.
__device__ __attribute__((always_inline)) void write_verdict(
    int b, const Verdict& v, int32_t extra, int M, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, double* __restrict__ p_tok, double* __restrict__ q_tok) {
  if (v.st < 0) {
    write_failed(b, v.st, M, accepted_len, out_tokens, p_tok, q_tok);
    return;
  }
  const int lane = threadIdx.x;
  int32_t* out = out_tokens + (size_t)b * (M + 1);
  if (lane == 0) accepted_len[b] = v.a;
  for (int j = lane; j <= M; j += kWave) {
    int32_t t = -1;
    if (j < v.a) t = v.x;  // j < a <= 64 means j == lane
    else if (j == v.a) t = extra;
    out[j] = t;
  }
  for (int j = lane; j < M; j += kWave) {
    const bool have_p = (v.rl == SV_RULE_SPECULATIVE || v.rl == SV_RULE_RELAXED) && j < v.np;
    const bool have_q = v.rl == SV_RULE_SPECULATIVE && j < v.np;
    if (p_tok) p_tok[(size_t)b * M + j] = have_p ? v.px : -1.0;
    if (q_tok) q_tok[(size_t)b * M + j] = have_q ? v.qx : -1.0;
  }
}

// ------------------------------------------------------------ chunked draw
// Textbook "The acceptance rule" / SDCP Sec. 6.4 Rule 2 (and the relaxed
// rule's draw from p): the additional token is the smallest id whose running
// weight exceeds u * S, over ascending ids, with weights max(0, p - q) (zero
// where p is zero) for the residual, or p.  A session's row is cut into groups
// of kGroup ids; C workgroups per session each take a run of groups, each
// wave a run inside it, and record every group (GroupRec).  The session's
// last workgroup to finish adds the records up, finds the group holding
// u * S and weighs that group again id by id.

constexpr int kDrawNT = 256;                 // threads per workgroup
constexpr int kDrawWaves = kDrawNT / kWave;
constexpr int kPer = 8;                      // consecutive ids per lane per step
constexpr int kWStep = kWave * kPer;         // ids per wave step
constexpr int kSteps = kGroup / kWStep;      // wave steps per group
constexpr int kTabBits = 9;                  // 2^(i / kTab) tabled per row
constexpr int kTab = 1 << kTabBits;
constexpr int kDeg = 4;                      // degree of the polynomial for 2^(f / kTab)
static_assert(kSteps == 4, "the load ring holds one group");

// Weights in binary64 by Tang's table-driven method (P. T. P. Tang, "Table-
// driven implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989), base 2: with x = (l - lmax) * scale and
// kTab x = n + f (n integer, 0 <= f < 1),
//   2^x = 2^(n >> kTabBits) * 2^((n & (kTab - 1)) / kTab) * 2^(f / kTab),
// the middle factor (divided by the row's Z) tabled per row, the last the
// Taylor polynomial of exp(f ln2 / kTab) to degree kDeg (with kTab = 512 and
// degree 4 the truncation is below 4e-17 relative; measured faster than 256
// entries and degree 5, and than 16 to 64 entries with degrees 8 to 6).
struct TaylorCoef {
  double c[kDeg + 1];
  constexpr TaylorCoef() : c() {
    const double r = 0.69314718055994530942 / kTab;  // ln 2 / kTab
    c[0] = 1.0;
    for (int n = 1; n <= kDeg; ++n) c[n] = c[n - 1] * r / n;
  }
};
constexpr TaylorCoef kTaylor;

// One row as the draw sees it: p(y) = w(y) / Z on the support.  A row whose
// cut is recorded as (kcut, ntie) keeps the ntie smallest ids among the tokens
// of key kcut (its ties, ranked in id order); other members are decided by
// key (and id, when the cut id is known).
template <class Tr>
struct DrawRow {
  const typename Tr::elem_t* row;
  const double* tab;  // tab[i] = 2^(i / kTab) / Z
  double sk, ck;      // kTab * scale (exact) and kTab * scale * lmax (rounded once)
  double wcut;        // p of each tie (tie mode)
  uint32_t kcut;
  float cv;           // the value of key kcut
  int32_t idcut;
  uint32_t ntie;      // ties kept (tie mode), else 0
  bool vec;           // 16-byte aligned row: vector loads
  __device__ bool tie(uint32_t k) const { return idcut < 0 && k == kcut; }
  __device__ bool fixed_member(uint32_t k, int y) const {
    return k > kcut || (k == kcut && idcut >= 0 && y <= idcut);
  }
  // the same tests on values: for the logits of a row that is drawn from (no
  // NaN) the order of the values is that of the keys, and +0 and -0 compare
  // equal as their keys do; one compare instead of the key transform
  __device__ bool tie_v(float f) const { return (idcut < 0) & (f == cv); }
  __device__ bool fixed_v(float f, int y) const {
    return (f > cv) | ((f == cv) & (idcut >= 0) & (y <= idcut));
  }
  __device__ double w(float l) const {
    // t = kTab (l - lmax) scale: l * sk is exact inside the fma and ck carries
    // one rounding, at most 2^-53 |lmax scale| octaves (a relative weight error
    // of ln2 2^-53 |lmax scale|); far below the binary64 range the integer part
    // saturates and ldexp gives 0
    const double t = __builtin_fma((double)l, sk, -ck);
    const double n = floor(t);
    const double f = t - n;
    const int ni = (int)n;
    double p = kTaylor.c[kDeg];
#pragma unroll
    for (int i = kDeg - 1; i >= 0; --i) p = __builtin_fma(p, f, kTaylor.c[i]);
    return ldexp(tab[ni & (kTab - 1)] * p, ni >> kTabBits);
  }
  // p of a token that is not a tie
  __device__ double p_fixed(uint32_t u, int y) const {
    const uint32_t k = Tr::key(u);
    return fixed_member(k, y) ? w(Tr::value(u)) : 0.0;
  }
};

// 8 consecutive elements' raw bits.
template <int kBytes>
struct Raw8;
template <>
struct Raw8<2> {
  u32x4 v;
  __device__ uint32_t get(int e) const {
    const uint32_t d = v[e >> 1];
    return (e & 1) ? d >> 16 : d & 0xFFFFu;
  }
};
template <>
struct Raw8<4> {
  u32x4 v[2];
  __device__ uint32_t get(int e) const {
    const uint32_t d = v[e >> 2][e & 3];
    return d;
  }
};

// Elements y .. y+7 of a row (fill past V).  Vector loads where the row is
// 16-byte aligned and the 8 elements lie inside it.
template <class E>
__device__ __attribute__((always_inline)) void load8(const E* row, int y, int V, bool vec,
                                                     uint32_t fill, Raw8<sizeof(E)>& r) {
  if (vec && y + kPer <= V) {
    const u32x4* p = (const u32x4*)(row + y);
    if constexpr (sizeof(E) == 2) r.v = p[0];
    else {
      r.v[0] = p[0];
      r.v[1] = p[1];
    }
  } else if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = y + 2 * d < V ? (uint32_t)row[y + 2 * d] : fill;
      const uint32_t hi = y + 2 * d + 1 < V ? (uint32_t)row[y + 2 * d + 1] : fill;
      r.v[d] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) r.v[e >> 2][e & 3] = y + e < V ? (uint32_t)row[y + e] : fill;
  }
}

// Elements y .. y+7 by vector loads only: the row is 16-byte aligned and
// y + 8 <= V (the caller's guarantee).
template <class E>
__device__ __attribute__((always_inline)) void load8_vec(const E* row, int y,
                                                         Raw8<sizeof(E)>& r) {
  const u32x4* p = (const u32x4*)(row + y);
  if constexpr (sizeof(E) == 2) r.v = p[0];
  else {
    r.v[0] = p[0];
    r.v[1] = p[1];
  }
}

template <class Tr, bool kQ>
struct DrawCtx {
  using RawP = Raw8<sizeof(typename Tr::elem_t)>;
  using RawQ = Raw8<kQ ? 4 : sizeof(typename Tr::elem_t)>;
  DrawRow<Tr> P, Q;    // Q: draft row (residual, !kQ)
  const float* qrow;   // published q row (residual, kQ)
  bool qvec;
  int V;
  __device__ __attribute__((always_inline)) void load(int y, bool resid, RawP& rp, RawQ& rq) const {
    load8(P.row, y, V, P.vec, Tr::kNegInfBits, rp);
    if (resid) {
      if constexpr (kQ) load8((const uint32_t*)qrow, y, V, qvec, 0u, rq);
      else load8(Q.row, y, V, Q.vec, Tr::kNegInfBits, rq);
    }
  }
  // the same inside whole vectors of aligned rows: a fixed number of vector
  // loads (kResid: the q row's too), so that a ring of them keeps its wait
  // counts exact
  template <bool kResid>
  __device__ __attribute__((always_inline)) void load_vec(int y, RawP& rp, RawQ& rq) const {
    load8_vec(P.row, y, rp);
    if constexpr (kResid) {
      if constexpr (kQ) load8_vec((const uint32_t*)qrow, y, rq);
      else load8_vec(Q.row, y, rq);
    }
  }
  // whole vectors can be loaded: every row read 16-byte aligned
  __device__ bool aligned(bool resid) const { return P.vec && (!resid || (kQ ? qvec : Q.vec)); }
};

// Exclusive prefix over the wave's lanes of a count in 0..15, and the wave
// total, from one ballot per bit.
__device__ inline uint32_t wave_excl_count(uint32_t c, uint32_t* total) {
  uint32_t r = 0, t = 0;
#pragma unroll
  for (int bit = 0; bit < 4; ++bit) {
    const uint64_t bm = __ballot((c >> bit) & 1u);
    r += (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0)) << bit;
    t += (uint32_t)__builtin_popcountll(bm) << bit;
  }
  *total = t;
  return r;
}

// A group's weights with the ties of each cut both kept and left out (see
// GroupRec), summed over one lane's ids.
struct GroupAcc {
  double a, bp, cq1, cq0, ap;
  uint32_t np, nq, npq, bad;
};

// One token's weights and classes from its binary32 logits (fp, and uq: q's
// logit as binary32 bits, or a published q entry): p's and q's weights are
// computed on every lane and kept where the token is a member (no branch per
// token, so that the binary64 chains and table reads of several tokens
// overlap).
struct IdW {
  double pv, qv;
  bool tp, tq, qbad;
};
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) IdW weigh_id(const DrawCtx<Tr, kQ>& d, bool resid,
                                                       float fp, uint32_t uq, int y) {
  IdW r;
  r.tp = d.P.tie_v(fp);
  const bool mp = !r.tp & d.P.fixed_v(fp, y);
  const double wp = d.P.w(fp);
  r.pv = mp ? wp : 0.0;
  r.qv = 0.0;
  r.tq = false;
  r.qbad = false;
  if (resid) {
    if constexpr (kQ) {
      r.qv = (double)__uint_as_float(uq);
      r.qbad = !(r.qv >= 0.0 && r.qv < INFINITY);
    } else {
      const float fq = __uint_as_float(uq);
      r.tq = d.Q.tie_v(fq);
      const bool mq = !r.tq & d.Q.fixed_v(fq, y);
      const double wq = d.Q.w(fq);
      r.qv = mq ? wq : 0.0;
    }
  }
  return r;
}

// One residual token's share of its group when no lane of the wave holds a
// tie of either row: p is zero off its support, and a draft row's q is never
// negative, so max(p - q, 0) is the residual.
template <bool kQ>
__device__ __attribute__((always_inline)) GroupAcc add_plain(double pv, double qv, bool qbad,
                                                             GroupAcc s) {
  const double df = pv - qv;
  if constexpr (kQ) {
    s.a += ((pv > 0.0) & (df > 0.0)) ? df : 0.0;
    if (pv > 0.0 && qbad) s.bad |= 1u;
  } else {
    s.a += __builtin_fmax(df, 0.0);
  }
  s.ap += pv;
  return s;
}

// One token's share of its group (see GroupAcc), ties included.  Only the
// ties take a branch, on a ballot (one value for the whole wave).
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) GroupAcc add_id(const DrawCtx<Tr, kQ>& d, bool resid,
                                                          double pv, double qv, bool tp, bool tq,
                                                          bool qbad, GroupAcc s) {
  if (!resid) {
    s.a += pv;
    s.np += tp ? 1u : 0u;
    return s;
  }
  const bool plain = !tp & !tq;
  const double df = pv - qv;
  s.a += (plain & (pv > 0.0) & (df > 0.0)) ? df : 0.0;
  s.ap += tp ? 0.0 : pv;
  if (kQ && plain && pv > 0.0 && qbad) s.bad |= 1u;
  if (__builtin_amdgcn_ballot_w64(tp | tq)) {  // ties: rows cut by rank only
    const double dp = d.P.wcut - qv;   // a tie of p (not of q), kept
    s.bp += (tp && !tq && d.P.wcut > 0.0 && dp > 0.0) ? dp : 0.0;
    const double dq = pv - d.Q.wcut;   // a tie of q (not of p), kept
    s.cq1 += (!tp && tq && pv > 0.0 && dq > 0.0) ? dq : 0.0;
    s.cq0 += (!tp && tq) ? pv : 0.0;
    s.np += tp ? 1u : 0u;
    s.nq += tq ? 1u : 0u;
    s.npq += (tp && tq) ? 1u : 0u;
    if (kQ && tp && qbad) s.bad |= 2u;
  }
  return s;
}

// One token's share of its group, in place (see GroupAcc): the branches test
// ballots, so a weight no lane of the wave needs is not computed.
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) GroupAcc weigh1(const DrawCtx<Tr, kQ>& d, bool resid,
                                                          uint32_t up, uint32_t uq, int y,
                                                          GroupAcc s) {
  const float fp = Tr::value(up);
  const bool tp = d.P.tie_v(fp);
  const bool mp = !tp & d.P.fixed_v(fp, y);
  bool tq = false, mq = false;
  float fq = 0.0f;
  if constexpr (!kQ) {
    if (resid) {
      fq = Tr::value(uq);
      tq = d.Q.tie_v(fq);
      mq = !tq & d.Q.fixed_v(fq, y);
    }
  }
  // no member or tie of p and no tie of q in the whole wave: nothing to add
  // (where p is zero, a member of q changes no weight)
  if (!__builtin_amdgcn_ballot_w64(mp | tp | tq)) return s;
  double pv = 0.0, qv = 0.0;
  bool qbad = false;
  if (__builtin_amdgcn_ballot_w64(mp)) {
    const double w = d.P.w(fp);
    pv = mp ? w : 0.0;
  }
  if (resid) {
    if constexpr (kQ) {
      qv = (double)__uint_as_float(uq);
      qbad = !(qv >= 0.0 && qv < INFINITY);
    } else if (__builtin_amdgcn_ballot_w64(mq & (mp | tp))) {
      const double w = d.Q.w(fq);
      qv = mq ? w : 0.0;
    }
  }
  return add_id<Tr, kQ>(d, resid, pv, qv, tp, tq, qbad, s);
}

// A lane's 8 ids of one step, in place: rows where most ids are members.
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) void weigh8(const DrawCtx<Tr, kQ>& d, bool resid, int y,
                                                      const typename DrawCtx<Tr, kQ>::RawP& pr,
                                                      const typename DrawCtx<Tr, kQ>::RawQ& qr,
                                                      GroupAcc& s) {
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    s = weigh1<Tr, kQ>(d, resid, pr.get(e), resid ? qr.get(e) : 0u, y + e, s);
}

// Table mode: a bf16 row cut by rank (idcut < 0) at a key above +0, with at
// most kKeyTab - 1 keys from the cut key to its largest logit, has few
// distinct member logits, and a member's weight depends on its logit alone.
// Its table holds, at entry i, the weight of the logit whose key is kcut + i
// (entry 0, the ties, 0: they are weighed by rank), and at entry n, past the
// largest key, 0.  For logits above +0 the bf16 bits grow with the key by
// one per key, so bits - bits(cut) is the entry; every logit below the cut
// gives, modulo 2^16, a larger value (negative ones too: their bits lie past
// the finite positive range, which holds bits(cut) + n), clamped to n.
constexpr int kKeyTab = 1536;  // entries of a row table, the zero entry included
struct KeyTab {
  bool on;
  const double* t[2];  // p's and q's tables
  uint32_t cut2[2];    // each row's cut logit (bf16 bits) in both halves
  uint32_t n2[2];      // each table's zero entry n in both halves
};
// Keys from a row's cut key to its largest logit when the row can take a
// table (bf16 rows), else 0.
__device__ inline int key_span(const RowRec& r) {
  if (r.idcut >= 0 || r.kcut <= Bf16::kSign) return 0;
  const int n = (int)Bf16::key(__float_as_uint(r.lmax) >> 16) - (int)r.kcut + 1;
  return (n >= 1 && n <= kKeyTab - 1) ? n : 0;
}

// Table mode on the logits as they are loaded, a dword holding two bf16
// logits (the lower id in the low half): with 16-bit halves, key - kcut is
// bits - bits(cut) for logits above +0 (and wraps past n for the others, see
// above), so one packed subtract and one packed minimum give both entries,
// and the sign bit of entry - 1 marks a tie (entry 0).
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
struct PairEntries {
  uint32_t lo, hi;  // byte offsets of the two logits' entries
  uint32_t tie;     // 0x8000 (low) and 0x80000000 (high) for ties
};
__device__ inline PairEntries pair_entries(uint32_t d, uint32_t cut2, uint32_t n2) {
  u16x2 x = __builtin_bit_cast(u16x2, d) - __builtin_bit_cast(u16x2, cut2);
  x = __builtin_elementwise_min(x, __builtin_bit_cast(u16x2, n2));
  const uint32_t off = __builtin_bit_cast(uint32_t, (u16x2)(x << (uint16_t)3));
  const u16x2 xm = x - (u16x2)(uint16_t)1;
  return PairEntries{off & 0xFFFFu, off >> 16, __builtin_bit_cast(uint32_t, xm) & 0x80008000u};
}
__device__ inline double table_at(const double* t, uint32_t off) {
  return *(const double*)((const char*)t + off);
}

// A lane's 8 ids of one step in table mode: the weights of p and q read from
// the key tables (ties and non-members read 0), kTabBatch ids at a time, then
// each id's share in id order.
#ifndef SV_TAB_BATCH
#define SV_TAB_BATCH 2
#endif
constexpr int kTabBatch = SV_TAB_BATCH;
static_assert(kTabBatch % 2 == 0, "whole dwords of bf16 pairs");
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) void weigh8_table(
    const DrawCtx<Tr, kQ>& d, const KeyTab& kt, bool resid,
    const typename DrawCtx<Tr, kQ>::RawP& pr, const typename DrawCtx<Tr, kQ>::RawQ& qr,
    GroupAcc& s) {
  static_assert(sizeof(typename Tr::elem_t) == 2, "bf16 rows");
#pragma unroll
  for (int h = 0; h < kPer; h += kTabBatch) {
    double pv[kTabBatch], qv[kTabBatch];
    uint32_t tp[kTabBatch / 2], tq[kTabBatch / 2];
    uint32_t tie = 0;
#pragma unroll
    for (int j = 0; j < kTabBatch / 2; ++j) {
      const PairEntries ep = pair_entries(pr.v[h / 2 + j], kt.cut2[0], kt.n2[0]);
      pv[2 * j] = table_at(kt.t[0], ep.lo);
      pv[2 * j + 1] = table_at(kt.t[0], ep.hi);
      tp[j] = ep.tie;
      tie |= ep.tie;
      tq[j] = 0;
      if (resid) {
        const PairEntries eq = pair_entries(qr.v[h / 2 + j], kt.cut2[1], kt.n2[1]);
        qv[2 * j] = table_at(kt.t[1], eq.lo);
        qv[2 * j + 1] = table_at(kt.t[1], eq.hi);
        tq[j] = eq.tie;
        tie |= eq.tie;
      }
    }
    if (!resid) {
#pragma unroll
      for (int e = 0; e < kTabBatch; ++e) s.a += pv[e];
#pragma unroll
      for (int j = 0; j < kTabBatch / 2; ++j) s.np += (uint32_t)__popc(tp[j]);
      continue;
    }
    if (!__builtin_amdgcn_ballot_w64(tie != 0)) {
#pragma unroll
      for (int e = 0; e < kTabBatch; ++e) s = add_plain<kQ>(pv[e], qv[e], false, s);
    } else {
#pragma unroll
      for (int e = 0; e < kTabBatch; ++e) {
        const uint32_t bit = (e & 1) ? 0x80000000u : 0x8000u;
        s = add_id<Tr, kQ>(d, true, pv[e], qv[e], (tp[e / 2] & bit) != 0, (tq[e / 2] & bit) != 0,
                           false, s);
      }
    }
  }
}

// Which of a lane's 8 ids can add to a group record: ids at or above p's cut
// key (members or ties of p), and for a residual the ties of q (counted even
// where p is zero).  A member of q where p is zero adds nothing: every
// residual weight, and the p mass of q's ties, is zero there.
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) uint32_t need_bits(
    const DrawCtx<Tr, kQ>& d, bool resid, const typename DrawCtx<Tr, kQ>::RawP& pr,
    const typename DrawCtx<Tr, kQ>::RawQ& qr) {
  uint32_t need = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    bool n = Tr::value(pr.get(e)) >= d.P.cv;
    if constexpr (!kQ)
      if (resid) n |= d.Q.tie_v(Tr::value(qr.get(e)));
    need |= n ? 1u << e : 0u;
  }
  return need;
}

// The wave's 512 ids of one step, compacted: the ids that need weighing are
// queued in LDS and weighed 64 at a time, so that a position whose lanes
// mostly hold non-members does not cost a full wave's binary64 work.  The
// queue is filled one element position at a time (a ballot and its prefix
// count per position), so it holds the ids by position, then lane; a group
// record only sums its ids' weights and counts its ties, so their order is
// free.  qu holds the wave's queue: p's logits and q's (binary32 bits;
// a published q row's entries), ids.
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) GroupAcc weigh_step_queued(
    const DrawCtx<Tr, kQ>& d, bool resid, int y, const typename DrawCtx<Tr, kQ>::RawP& pr,
    const typename DrawCtx<Tr, kQ>::RawQ& qr, GroupAcc s, uint32_t* qu) {
  const int lane = __lane_id();
  uint32_t total = 0;  // wave-uniform
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const float fp = Tr::value(pr.get(e));
    bool n = fp >= d.P.cv;  // at or above p's cut key
    uint32_t uq = 0u;       // q's logit as binary32 bits, or the published entry
    if (resid) {
      if constexpr (kQ) {
        uq = qr.get(e);
      } else {
        const float fq = Tr::value(qr.get(e));
        n |= d.Q.tie_v(fq);
        uq = __float_as_uint(fq);
      }
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(n);
    if (m) {
      const uint32_t j = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, total));
      if (n) {
        qu[j] = __float_as_uint(fp);
        qu[kWStep + j] = uq;
        qu[2 * kWStep + j] = (uint32_t)(y + e);
      }
      total += (uint32_t)__builtin_popcountll(m);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // rounds of 64 queued ids, two at a time; total <= kWStep and rounds start
  // at multiples of 64 below it, so every slot read lies in the queue (slots
  // at or past total hold stale words and are masked)
  auto entry = [&](uint32_t i, uint32_t& up, uint32_t& uq, int& yy) {
    const bool valid = i < total;
    up = qu[i];
    uq = qu[kWStep + i];
    yy = (int)qu[2 * kWStep + i];
    // past the queue: -inf, neither a member nor a tie of either row
    up = valid ? up : 0xFF800000u;
    uq = valid ? uq : (kQ ? 0u : 0xFF800000u);
    yy = valid ? yy : 0;
  };
  uint32_t r = 0;
  for (; r + kWave < total; r += 2 * kWave) {
    uint32_t up0, uq0, up1, uq1;
    int y0, y1;
    entry(r + (uint32_t)lane, up0, uq0, y0);
    entry(r + kWave + (uint32_t)lane, up1, uq1, y1);
    const IdW a0 = weigh_id<Tr, kQ>(d, resid, __uint_as_float(up0), uq0, y0);
    const IdW a1 = weigh_id<Tr, kQ>(d, resid, __uint_as_float(up1), uq1, y1);
    if (resid && !__builtin_amdgcn_ballot_w64(a0.tp | a0.tq | a1.tp | a1.tq)) {
      s = add_plain<kQ>(a0.pv, a0.qv, a0.qbad, s);
      s = add_plain<kQ>(a1.pv, a1.qv, a1.qbad, s);
    } else {
      s = add_id<Tr, kQ>(d, resid, a0.pv, a0.qv, a0.tp, a0.tq, a0.qbad, s);
      s = add_id<Tr, kQ>(d, resid, a1.pv, a1.qv, a1.tp, a1.tq, a1.qbad, s);
    }
  }
  for (; r < total; r += kWave) {
    uint32_t up0, uq0;
    int y0;
    entry(r + (uint32_t)lane, up0, uq0, y0);
    const IdW a0 = weigh_id<Tr, kQ>(d, resid, __uint_as_float(up0), uq0, y0);
    s = add_id<Tr, kQ>(d, resid, a0.pv, a0.qv, a0.tp, a0.tq, a0.qbad, s);
  }
  __builtin_amdgcn_wave_barrier();
  return s;
}

// Group records cross workgroups as six 64-bit words in device-scope atomics
// (the session's workgroups may run on different L2 caches): word i of a
// record is a, bp, cq1, cq0, ap (i = 0..4), and the tie counts np | nq << 16 |
// (npq | bad << 16) << 32 (i = 5).
// A group's sums over the wave, stored as its record (the words above).
// The six 64-bit fields (five weights; the tie counts packed exactly into one
// binary64 integer, each count below 2^12 and each flag count below 2^8) and
// two empty ones are reduced by a transposed butterfly: across 32 and then 16
// lanes a lane keeps half of its fields and takes its partner's share of
// them (v_permlane32_swap, v_permlane16_swap: after a swap of the fields a, b
// that the two halves keep, a + b is the pair's sum in both), across 8 lanes
// one of its two (DPP row mirror), and the 8 lanes that hold field f add it
// up (DPP), so lane 8f stores word f.  The order of the additions is fixed.
__device__ inline void swap_halves(double& a, double& b, bool rows16) {
  const uint64_t ua = (uint64_t)__double_as_longlong(a), ub = (uint64_t)__double_as_longlong(b);
  uint32_t lo0, lo1, hi0, hi1;
  if (rows16) {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)ua, (uint32_t)ub, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32),
                                                     false, false);
    lo0 = lo[0], lo1 = lo[1], hi0 = hi[0], hi1 = hi[1];
  } else {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)ua, (uint32_t)ub, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32),
                                                     false, false);
    lo0 = lo[0], lo1 = lo[1], hi0 = hi[0], hi1 = hi[1];
  }
  a = __longlong_as_double((long long)(((uint64_t)hi0 << 32) | lo0));
  b = __longlong_as_double((long long)(((uint64_t)hi1 << 32) | lo1));
}
template <int kCtrl>
__device__ inline double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, kCtrl, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), kCtrl, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ inline void reduce_store_group(GroupRec* rec, const GroupAcc& s) {
  constexpr int kRowMirror = 0x140, kHalfMirror = 0x141;
  constexpr int kQuadSwap2 = 0x4E, kQuadSwap1 = 0xB1;  // quad_perm [2,3,0,1], [1,0,3,2]
  const int lane = __lane_id();
  const uint32_t c_lo = s.np | (s.nq << 12);
  const uint32_t c_hi = s.npq | ((s.bad & 1u) << 12) | ((s.bad >> 1) << 20);
  double v[8] = {s.a, s.bp, s.cq1, s.cq0, s.ap, (double)c_lo + (double)c_hi * 16777216.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // lanes 0-31 keep fields 0-3, lanes 32-63 fields 4-7
    swap_halves(v[i], v[i + 4], false);
    v[i] = v[i] + v[i + 4];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // within each half, rows 0 and 2 keep the first two
    swap_halves(v[j], v[j + 2], true);
    v[j] = v[j] + v[j + 2];
  }
  const bool up8 = (lane & 8) != 0;  // within a row, lanes 8-15 keep the second
  const double keep = up8 ? v[1] : v[0];
  const double x = keep + dpp_f64<kRowMirror>(up8 ? v[0] : v[1]);
  const double x1 = x + dpp_f64<kHalfMirror>(x);
  const double x2 = x1 + dpp_f64<kQuadSwap2>(x1);
  const double t = x2 + dpp_f64<kQuadSwap1>(x2);  // field lane >> 3, in all 8 of its lanes
  const int f = lane >> 3;
  if ((lane & 7) == 0 && f < 6) {
    uint64_t w = (uint64_t)__double_as_longlong(t);
    if (f == 5) {
      const uint32_t hi = (uint32_t)(t * (1.0 / 16777216.0));
      const uint32_t lo = (uint32_t)(t - (double)hi * 16777216.0);
      const uint32_t np = lo & 0xFFFu, nq = lo >> 12, npq = hi & 0xFFFu;
      const uint32_t bad = (((hi >> 12) & 0xFFu) ? 1u : 0u) | ((hi >> 20) ? 2u : 0u);
      w = (uint64_t)(np | (nq << 16)) | ((uint64_t)(npq | (bad << 16)) << 32);
    }
    __hip_atomic_store((uint64_t*)rec + f, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
__device__ inline GroupAcc decode_group(const uint64_t (&w)[6]) {
  GroupAcc r;
  r.a = __longlong_as_double((long long)w[0]);
  r.bp = __longlong_as_double((long long)w[1]);
  r.cq1 = __longlong_as_double((long long)w[2]);
  r.cq0 = __longlong_as_double((long long)w[3]);
  r.ap = __longlong_as_double((long long)w[4]);
  r.np = (uint32_t)w[5] & 0xFFFFu;
  r.nq = (uint32_t)w[5] >> 16;
  r.npq = (uint32_t)(w[5] >> 32) & 0xFFFFu;
  r.bad = (uint32_t)(w[5] >> 48);
  return r;
}
__device__ inline GroupAcc load_group(const GroupRec* rec) {
  uint64_t w[6];
#pragma unroll
  for (int i = 0; i < 6; ++i)
    w[i] = __hip_atomic_load((const uint64_t*)rec + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return decode_group(w);
}

// One wave records groups [g0, g1): steps of 8 ids per lane through a ring of
// kSteps loads, three steps ahead.  For a row cut to a support, the wave
// weighs queued ids when its first step has 16 to SV_QUEUE_MAX (three rounds
// of 64) ids to weigh, else in place (with fewer, in place skips the empty
// positions anyway; rows with more members keep the 8 unrolled positions,
// which overlap their binary64 chains).  The two loops are kept apart so that
// each has its own registers.
//
// kSteady: groups that lie wholly inside aligned rows.  Every step then issues
// the same vector loads (the ring's last three clamped to the wave's last
// step), so the compiler's wait counts leave three steps in flight; with
// loads that depend on the step (the row's end, a scalar fallback) it waits
// for all of them at each step, and the ring drains.  kResid fixes, at
// compile time, whether the q row is read.
enum RecordMode { kInPlace = 0, kQueued = 1, kTable = 2 };
template <class Tr, bool kQ, int kMode, bool kSteady = false, bool kResid = false>
__device__ __attribute__((always_inline)) void record_loop(const DrawCtx<Tr, kQ>& d, bool resid,
                                                           int g0, int g1,
                                                           GroupRec* __restrict__ recs,
                                                           uint32_t* qu, const KeyTab& kt) {
  if constexpr (kSteady) resid = kResid;
  const int lane = __lane_id();
  const int nk = (g1 - g0) * kSteps;
  const int ybase = g0 * kGroup + lane * kPer;
  typename DrawCtx<Tr, kQ>::RawP p[kSteps];
  typename DrawCtx<Tr, kQ>::RawQ q[kSteps];
  if constexpr (kSteady) {
    // four steps ahead, each slot refilled right after it is weighed, so the
    // loads outstanding at the loop's back edge are those of the prologue, in
    // the same order
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      d.template load_vec<kResid>(ybase + min(u, nk - 1) * kWStep, p[u], q[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    d.load(ybase, resid, p[0], q[0]);
    d.load(ybase + kWStep, resid, p[1], q[1]);
    d.load(ybase + 2 * kWStep, resid, p[2], q[2]);
  }
  for (int k = 0; k < nk; k += kSteps) {
    GroupAcc s{};
    // the waves of a SIMD share it by the share of their groups left (see
    // stream::set_priority): without it the oldest waves finish first and the
    // session whose waves came last on their SIMDs ends the kernel
    stream::set_priority(nk - k, nk);
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
      const int kk = k + u;
      if constexpr (!kSteady)
        if (kk + 3 < nk)
          d.load(ybase + (kk + 3) * kWStep, resid, p[(u + 3) % kSteps], q[(u + 3) % kSteps]);
      const int y = ybase + kk * kWStep;
      if constexpr (kMode == kTable) weigh8_table<Tr, kQ>(d, kt, resid, p[u], q[u], s);
      else if constexpr (kMode == kQueued) s = weigh_step_queued<Tr, kQ>(d, resid, y, p[u], q[u], s, qu);
      else weigh8<Tr, kQ>(d, resid, y, p[u], q[u], s);
      if constexpr (kSteady) {
        __builtin_amdgcn_sched_barrier(0);
        d.template load_vec<kResid>(ybase + min(kk + kSteps, nk - 1) * kWStep, p[u], q[u]);
      }
    }
    reduce_store_group(recs + g0 + k / kSteps, s);
  }
}

#ifndef SV_QUEUE_MAX
#define SV_QUEUE_MAX (3 * kWave)
#endif
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) void record_groups(const DrawCtx<Tr, kQ>& d, bool resid,
                                                             int g0, int g1, bool sparse,
                                                             GroupRec* __restrict__ recs,
                                                             uint32_t* qu, const KeyTab& kt) {
  if (g0 >= g1) return;
  if constexpr (std::is_same<Tr, Bf16>::value && !kQ) {
    if (kt.on) {
      const int gs = d.aligned(resid) ? min(g1, d.V / kGroup) : g0;
      if (g0 < gs) {
        if (resid) record_loop<Tr, kQ, kTable, true, true>(d, resid, g0, gs, recs, qu, kt);
        else record_loop<Tr, kQ, kTable, true, false>(d, resid, g0, gs, recs, qu, kt);
      }
      const int gr = max(g0, gs);
      if (gr < g1) record_loop<Tr, kQ, kTable>(d, resid, gr, g1, recs, qu, kt);
      return;
    }
  }
  bool queued = false;
  if (sparse) {  // the first step's ids to weigh, over the wave
    typename DrawCtx<Tr, kQ>::RawP p0;
    typename DrawCtx<Tr, kQ>::RawQ q0;
    d.load(g0 * kGroup + __lane_id() * kPer, resid, p0, q0);
    uint32_t total;
    (void)wave_excl_count(__builtin_popcount(need_bits<Tr, kQ>(d, resid, p0, q0)), &total);
    queued = total >= 16 && total <= SV_QUEUE_MAX;
  }
  // the groups inside whole vectors of aligned rows take the steady loop; a
  // row's last group (its end, a partial vector) the general one
  const int gs = d.aligned(resid) ? min(g1, d.V / kGroup) : g0;
  if (g0 < gs) {
    if (queued) {
      if (resid) record_loop<Tr, kQ, kQueued, true, true>(d, resid, g0, gs, recs, qu, kt);
      else record_loop<Tr, kQ, kQueued, true, false>(d, resid, g0, gs, recs, qu, kt);
    } else {
      if (resid) record_loop<Tr, kQ, kInPlace, true, true>(d, resid, g0, gs, recs, qu, kt);
      else record_loop<Tr, kQ, kInPlace, true, false>(d, resid, g0, gs, recs, qu, kt);
    }
  }
  const int gr = max(g0, gs);
  if (gr < g1) {
    if (queued) record_loop<Tr, kQ, kQueued>(d, resid, gr, g1, recs, qu, kt);
    else record_loop<Tr, kQ, kInPlace>(d, resid, gr, g1, recs, qu, kt);
  }
}

// A group's weight from its record: the ties of p kept (sp = 1), left out
// (sp = 0); likewise for q.  kept: ties of p kept (draws from p).
__device__ inline double group_mass(const GroupAcc& r, bool resid, int sp, int sq, uint32_t kept,
                                    double Pk, double Qk) {
  if (!resid) return r.a + (double)kept * Pk;
  double m = r.a + (sp ? r.bp : 0.0) + (sq ? r.cq1 : r.cq0);
  if (r.npq) {
    const double df = Pk - Qk;
    m += (double)r.npq * (sp ? (sq ? ((Pk > 0.0 && df > 0.0) ? df : 0.0) : Pk) : 0.0);
  }
  return m;
}

constexpr int kLdsGroups = 512;  // group records staged in LDS for the pick

struct DrawSmem {
  union {
    uint64_t grec[kLdsGroups][6];             // the pick: staged group records
    uint32_t queue[kDrawWaves][3 * kWStep];  // the records: each wave's queue
    double ktab[2][kKeyTab];                  // the records in table mode: p's, q's table
  };
  double tab_p[kTab];
  double tab_q[kTab];
  double dscan[kDrawWaves];
  uint64_t uscan[kDrawWaves];
  int32_t ired[kDrawWaves];
  int32_t red3[kDrawWaves][3];  // group scans: first crossing, last id with weight, unusable
  uint32_t wties[kDrawWaves];  // group scans: ties of each wave's step
  double wsum[kDrawWaves];     // group scans: weight of each wave's step
  int32_t sg[2];            // groups holding the cut of p, of q (-1: none)
  uint32_t stp[2], stq[2];  // their ties before them
  double smass[2];          // their weights, ties ranked
  int32_t sbad[2];
  int32_t gstar;            // the group holding u * S, its weight before, ties before
  double gbase;
  uint32_t gtp, gtq;
  uint32_t ltp, ltq;        // ties before the last group with weight
  int32_t q_id[kSupMax];
  double q_p[kSupMax];
  Job job;
  uint32_t last;
};

// Block-wide exclusive scan in thread order (fixed combination order).
template <int NT, typename T>
__device__ __attribute__((always_inline)) T block_exclusive_scan(T v, T* wsum, T* total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const T inc = wave_incl_scan(v);
  const T exc = inc - v;  // not a one-lane shift: see group_scan
  __syncthreads();
  if (lane == kWave - 1) wsum[wid] = inc;
  __syncthreads();
  T base = T(0), tot = T(0);
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    if (w < wid) base += wsum[w];
    tot += wsum[w];
  }
  *total = tot;
  return base + exc;
}

struct ScanRes {
  double total;
  int32_t first;  // INT32_MAX: not in this group
  int32_t lastpos;
  uint32_t np, nq;
  bool bad;
};

// A thread's 8 ids of group g for group_scan, loaded ahead of it (so that
// the loads of two groups can be in flight together).
template <class Tr, bool kQ>
struct ScanLoad {
  typename DrawCtx<Tr, kQ>::RawP pr;
  typename DrawCtx<Tr, kQ>::RawQ qr;
};
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) ScanLoad<Tr, kQ> scan_load(const DrawCtx<Tr, kQ>& d,
                                                                     bool resid, int g) {
  const int lane = __lane_id(), wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  ScanLoad<Tr, kQ> L;
  d.load(g * kGroup + wid * kWStep + lane * kPer, resid, L.pr, L.qr);
  return L;
}

// Group g weighed id by id by the whole workgroup, ties ranked: wave w takes
// the group's step w (512 ids, loaded by scan_load), the waves exchange their
// tie counts and weights through LDS.  rp, rq are the ties of p and q before
// the group.  Returns the group's weight and tie counts, the last id with
// weight, whether an unusable published q entry was read where p > 0, and
// (find) the first id at which base + running weight exceeds tgt.  All
// threads call it.
// p (r = 0) or q (r = 1) of a token that is not a tie of that row: from the
// row's key table when the tables are still in LDS (table mode; the same
// binary64 weights, see weigh8_table), else computed.
template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) double scan_weight(const DrawRow<Tr>& D,
                                                             const KeyTab& kt, bool tabs, int r,
                                                             uint32_t u, int y) {
  if constexpr (std::is_same<Tr, Bf16>::value && !kQ) {
    if (tabs) {
      const uint32_t cut = kt.cut2[r] & 0xFFFFu, n = kt.n2[r] & 0xFFFFu;
      return table_at(kt.t[r], min((u - cut) & 0xFFFFu, n) * 8u);
    }
  }
  return D.p_fixed(u, y);
}

template <class Tr, bool kQ>
__device__ __attribute__((always_inline)) ScanRes group_scan(const DrawCtx<Tr, kQ>& d, bool resid,
                                                             int g, const ScanLoad<Tr, kQ>& L,
                                                             uint32_t rp, uint32_t rq,
                                                             double base, double tgt, bool find,
                                                             DrawSmem& sm, const KeyTab& kt,
                                                             bool tabs) {
  const int lane = __lane_id(), wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int y = g * kGroup + wid * kWStep + lane * kPer;
  const typename DrawCtx<Tr, kQ>::RawP& pr = L.pr;
  const typename DrawCtx<Tr, kQ>::RawQ& qr = L.qr;
  uint32_t fp = 0, fq = 0;  // which of the 8 ids are ties of p, of q
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if (d.P.tie(Tr::key(pr.get(e)))) fp |= 1u << e;
    if constexpr (!kQ)
      if (resid && d.Q.tie(Tr::key(qr.get(e)))) fq |= 1u << e;
  }
  uint32_t tpw, tqw;
  const uint32_t ep = wave_excl_count(__builtin_popcount(fp), &tpw);
  const uint32_t eq = wave_excl_count(__builtin_popcount(fq), &tqw);
  __syncthreads();  // the previous scan's exchange is read
  if (lane == 0) sm.wties[wid] = tpw | (tqw << 16);  // at most 512 each
  __syncthreads();
  uint32_t bp = 0, bq = 0, np = 0, nq = 0;
#pragma unroll
  for (int w = 0; w < kDrawWaves; ++w) {
    const uint32_t v = sm.wties[w];
    if (w < wid) {
      bp += v & 0xFFFFu;
      bq += v >> 16;
    }
    np += v & 0xFFFFu;
    nq += v >> 16;
  }
  uint32_t cp = rp + bp + ep, cq = rq + bq + eq;
  double w8[kPer];
  double ls = 0.0;
  bool bad = false;
  int32_t lastpos = -1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    double pv;
    if ((fp >> e) & 1u) pv = cp++ < d.P.ntie ? d.P.wcut : 0.0;
    else pv = scan_weight<Tr, kQ>(d.P, kt, tabs, 0, pr.get(e), y + e);
    double wt = pv;
    if (resid) {
      double qv;
      if constexpr (kQ) {
        qv = (double)__uint_as_float(qr.get(e));
        bad |= pv > 0.0 && !(qv >= 0.0 && qv < INFINITY);
      } else {
        if ((fq >> e) & 1u) qv = cq++ < d.Q.ntie ? d.Q.wcut : 0.0;
        else qv = scan_weight<Tr, kQ>(d.Q, kt, tabs, 1, qr.get(e), y + e);
      }
      const double df = pv - qv;
      wt = (pv > 0.0 && df > 0.0) ? df : 0.0;
    }
    w8[e] = wt;
    ls += wt;
    if (wt > 0.0) lastpos = y + e;
  }
  // running weight over the lanes in id order; the exclusive prefix as
  // incl - ls (see block_exclusive_scan)
  const double incl = wave_incl_scan(ls);
  const double excl = incl - ls;
  const double wtot = lane_read(incl, kWave - 1);
  if (lane == 0) sm.wsum[wid] = wtot;
  __syncthreads();
  double before = 0.0, total = 0.0;
#pragma unroll
  for (int w = 0; w < kDrawWaves; ++w) {
    const double v = sm.wsum[w];
    if (w < wid) before += v;
    total += v;
  }
  int32_t mine = INT32_MAX;
  if (find) {
    double acc = base + before + excl;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      acc += w8[e];
      if (mine == INT32_MAX && acc > tgt) mine = y + e;
    }
  }
  // the first crossing, the last id with weight and the unusable entries over
  // the workgroup, in one exchange (the previous scan's reads of sm.red3 are
  // behind the barriers of this scan's exchanges above)
  mine = wave_reduce(mine, OpMin());
  lastpos = wave_reduce(lastpos, OpMax());
  const int32_t anybad = __builtin_amdgcn_ballot_w64(bad) != 0 ? 1 : 0;
  if (lane == 0) {
    sm.red3[wid][0] = mine;
    sm.red3[wid][1] = lastpos;
    sm.red3[wid][2] = anybad;
  }
  __syncthreads();
  ScanRes res{total, INT32_MAX, -1, np, nq, false};
#pragma unroll
  for (int w = 0; w < kDrawWaves; ++w) {
    res.first = min(res.first, sm.red3[w][0]);
    res.lastpos = max(res.lastpos, sm.red3[w][1]);
    res.bad |= sm.red3[w][2] != 0;
  }
  return res;
}

// The kernel: workgroup (b, c) = blockIdx.x = b * C + c; wave w of chunk c
// records groups [(4c + w) * gw, (4c + w + 1) * gw).  Every workgroup's first
// wave takes session b's acceptance rule; chunk 0's workgroup writes the
// outputs of a session left with no whole-row draw.  With such a draw, the
// last workgroup to finish (a counter per session, cleared by the single-pass
// row kernel; C = 1 needs none) picks the token and writes all the session's
// outputs.
template <class Tr, bool kQ>
// The LDS of four workgroups fits a CU (four waves per SIMD); bf16 rows hold
// their registers to the same occupancy.
__global__ __launch_bounds__(kDrawNT)
__attribute__((amdgpu_waves_per_eu(sizeof(typename Tr::elem_t) == 2 ? 4 : 3))) void k_finalize(
    const typename Tr::elem_t* __restrict__ target, const typename Tr::elem_t* __restrict__ draft,
    const float* __restrict__ qrows, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling, int B, int M, int V,
    uint64_t seed, uint32_t round, const int32_t* __restrict__ sess_status,
    const RowRec* __restrict__ rows, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, double* __restrict__ p_tok, double* __restrict__ q_tok,
    const int32_t* __restrict__ sup_id, const double* __restrict__ sup_p,
    const double* __restrict__ unif, GroupRec* __restrict__ groups, uint32_t* __restrict__ ctr,
    const uint32_t* __restrict__ draw_flag, uint32_t draw_token, int C, int gw,
    const int32_t* __restrict__ decided) {
  __shared__ DrawSmem sm;
  const int b = (int)blockIdx.x / C;
  const int c = (int)blockIdx.x - b * C;
  if (b >= B) return;
  const int t = threadIdx.x;
  // the wave's index, as a scalar: the record loops' bounds derive from it
  const int wid = __builtin_amdgcn_readfirstlane(t / kWave);
  // only chunk 0 has work in sessions that draw no token from whole rows
  if (c > 0 && (draw_flag[b] != draw_token || rule[b] == SV_RULE_GREEDY || sess_status[b] != 0))
    return;
  Verdict v{};
  if (t < kWave) {
    v = accept_session(b, tokens, m, rule, sampling, M, V, kQ ? qrows : nullptr, seed, round,
                       sess_status, rows, sup_id, sup_p, unif, decided, c == 0, sm.q_id,
                       sm.q_p);
    if (v.st < 0 || v.job.kind == kJobNone) {
      if (c == 0) write_verdict(b, v, v.extra, M, accepted_len, out_tokens, p_tok, q_tok);
      v.job.kind = kJobNone;
    }
    if (t == 0) sm.job = v.job;
  }
  __syncthreads();
  const Job job = sm.job;
  if (job.kind == kJobNone) return;

  const int R = 2 * M + 1;
  const int G = (V + kGroup - 1) / kGroup;
  const bool resid = job.kind == kJobResidual;
  auto make_row = [&](const typename Tr::elem_t* row, const RowRec& r, double* tab) {
    DrawRow<Tr> D;
    D.row = row;
    D.tab = tab;
    D.sk = r.scale * (double)kTab;
    D.ck = (double)r.lmax * D.sk;
    D.kcut = r.kcut;
    D.cv = Tr::value(Tr::unkey(r.kcut));
    D.idcut = r.idcut;
    D.ntie = r.idcut < 0 ? (uint32_t)r.ntie : 0u;
    D.wcut = weight64(Tr::value(Tr::unkey(r.kcut)), r.lmax, r.scale) / r.zsum;
    D.vec = ((uintptr_t)row & 15u) == 0;
    for (int i = t; i < kTab; i += kDrawNT) tab[i] = exp2((double)i / (double)kTab) / r.zsum;
    return D;
  };
  const DrawRow<Tr> Prow = make_row(target + ((size_t)b * (M + 1) + job.trow) * (size_t)V,
                                    rows[(size_t)b * R + job.trow], sm.tab_p);
  DrawRow<Tr> Qrow = Prow;
  Qrow.idcut = 0;  // no q ties unless a draft row is read
  Qrow.ntie = 0;
  const float* qrow = nullptr;
  if (resid) {
    if constexpr (kQ) qrow = qrows + ((size_t)b * M + job.drow) * (size_t)V;
    else Qrow = make_row(draft + ((size_t)b * M + job.drow) * (size_t)V,
                         rows[(size_t)b * R + M + 1 + job.drow], sm.tab_q);
  }
  const DrawCtx<Tr, kQ> d{Prow, Qrow, qrow, ((uintptr_t)qrow & 15u) == 0, V};
  __syncthreads();  // tables ready

  // rows with few member logits: their key tables, from the weights above
  KeyTab kt{};
  kt.t[0] = sm.ktab[0];  // set on every path: a constant LDS address, folded into the reads
  kt.t[1] = sm.ktab[1];
  if constexpr (std::is_same<Tr, Bf16>::value && !kQ) {
    const RowRec& rp = rows[(size_t)b * R + job.trow];
    const int np = key_span(rp);
    const int nq = resid ? key_span(rows[(size_t)b * R + M + 1 + job.drow]) : 1;
    if (np > 0 && nq > 0) {
      kt.on = true;
      const DrawRow<Tr>* row2[2] = {&d.P, &d.Q};
      const int n2[2] = {np, nq};
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (r == 1 && !resid) break;
        const DrawRow<Tr>& D = *row2[r];
        const uint32_t cut = __float_as_uint(D.cv) >> 16;
        kt.cut2[r] = cut | (cut << 16);
        kt.n2[r] = (uint32_t)n2[r] | ((uint32_t)n2[r] << 16);
        for (int i = t; i <= n2[r]; i += kDrawNT)
          sm.ktab[r][i] = (i == 0 || i == n2[r]) ? 0.0 : D.w(Tr::value(Tr::unkey(D.kcut + (uint32_t)i)));
      }
      __syncthreads();
    }
  }

  // this wave's groups, then (several chunks) the session's counter
  GroupRec* recs = groups + (size_t)b * G;
  {
    const int g0 = (4 * c + wid) * gw;
    // rows cut to a support (top-k, top-p) weigh their members only;
    // untruncated rows, where every id is a member, weigh in place
    const bool sparse = !(d.P.kcut == Tr::kNegInfKey + 1 && d.P.idcut >= 0);
    record_groups<Tr, kQ>(d, resid, min(g0, G), min(g0 + gw, G), sparse, recs, sm.queue[wid],
                          kt);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's records are stored
  __syncthreads();
  if (C > 1) {
    if (t == 0) {
      const uint32_t done =
          __hip_atomic_fetch_add(&ctr[b], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = done == (uint32_t)(C - 1);
      if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      sm.last = last ? 1u : 0u;
    }
    __syncthreads();
    if (!sm.last) return;
  }

  // ---- the session's last workgroup: the pick is the end of the session's
  // critical path, so it takes the SIMD ahead of waves still recording
  __builtin_amdgcn_s_setprio(3);
  // thread t adds up groups [ga, gb)
  const int ga = (int)((long long)t * G / kDrawNT), gb = (int)((long long)(t + 1) * G / kDrawNT);
  // the records, staged in LDS when they fit (else read where they are)
  // the records, staged in LDS when they fit (else read where they are): in
  // table mode after the key tables' entries when there is room, so that the
  // groups weighed again read their weights from the tables
  const bool staged = G <= kLdsGroups;
  constexpr int kUnionBytes = (int)sizeof(sm.grec);
  static_assert(sizeof(sm.ktab) == kUnionBytes, "the key tables fill the staging space");
  bool tabs_kept = false;
  if constexpr (std::is_same<Tr, Bf16>::value && !kQ) {
    const int used = resid ? (int)sizeof(sm.ktab[0]) + 8 * ((int)(kt.n2[1] & 0xFFFFu) + 1)
                           : 8 * ((int)(kt.n2[0] & 0xFFFFu) + 1);
    tabs_kept = kt.on && staged && kUnionBytes - 48 * G >= used;
  }
  uint64_t* grec = tabs_kept ? (uint64_t*)((char*)&sm.grec[0][0] + kUnionBytes - 48 * G)
                             : &sm.grec[0][0];
  if (staged) {
    for (int i = t; i < G * 6; i += kDrawNT)
      grec[i] = __hip_atomic_load((const uint64_t*)(recs + i / 6) + i % 6, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  auto rec = [&](int g) -> GroupAcc {
    if (staged) {
      uint64_t w[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) w[i] = grec[g * 6 + i];
      return decode_group(w);
    }
    return load_group(recs + g);
  };
  const uint32_t jp = d.P.ntie, jq = d.Q.ntie;
  const double Pk = d.P.wcut, Qk = kQ ? 0.0 : d.Q.wcut;
  // a group's ties: all kept (1), none (0), or the cut falls inside it (2)
  auto state = [](uint32_t before, uint32_t n, uint32_t j) -> int {
    return before + n <= j ? 1 : (before >= j ? 0 : 2);
  };
  auto kept = [](int s, uint32_t before, uint32_t n, uint32_t j) -> uint32_t {
    return s == 1 ? n : (s == 0 ? 0u : j - before);
  };
  if (t == 0) sm.sg[0] = sm.sg[1] = -1;
  uint32_t lp = 0, lq = 0;
  for (int g = ga; g < gb; ++g) {
    const GroupAcc r = rec(g);
    lp += r.np;
    lq += r.nq;
  }
  uint64_t ttot;
  const uint64_t tb = block_exclusive_scan<kDrawNT, uint64_t>((uint64_t)lp | ((uint64_t)lq << 32),
                                                             sm.uscan, &ttot);
  const uint32_t tp0 = (uint32_t)tb, tq0 = (uint32_t)(tb >> 32);
  if (resid) {  // the groups holding a cut: their weights need the ties ranked
    uint32_t tp = tp0, tq = tq0;
    for (int g = ga; g < gb; ++g) {
      const GroupAcc r = rec(g);
      if (state(tp, r.np, jp) == 2) {
        sm.sg[0] = g;
        sm.stp[0] = tp;
        sm.stq[0] = tq;
      }
      if (state(tq, r.nq, jq) == 2) {
        sm.sg[1] = g;
        sm.stp[1] = tp;
        sm.stq[1] = tq;
      }
      tp += r.np;
      tq += r.nq;
    }
  }
  __syncthreads();
  {  // the groups holding p's and q's cut, both loaded before either is weighed
    const int ga = sm.sg[0], gq = sm.sg[1];
    const bool has_a = ga >= 0, has_q = gq >= 0 && gq != ga;
    ScanLoad<Tr, kQ> La{}, Lq{};
    if (has_a) La = scan_load<Tr, kQ>(d, true, ga);
    if (has_q) Lq = scan_load<Tr, kQ>(d, true, gq);
    if (has_a) {
      const ScanRes sr =
          group_scan<Tr, kQ>(d, true, ga, La, sm.stp[0], sm.stq[0], 0.0, 0.0, false, sm, kt, tabs_kept);
      if (t == 0) {
        sm.smass[0] = sr.total;
        sm.sbad[0] = sr.bad ? 1 : 0;
      }
    }
    if (has_q) {
      const ScanRes sr =
          group_scan<Tr, kQ>(d, true, gq, Lq, sm.stp[1], sm.stq[1], 0.0, 0.0, false, sm, kt, tabs_kept);
      if (t == 0) {
        sm.smass[1] = sr.total;
        sm.sbad[1] = sr.bad ? 1 : 0;
      }
    }
  }
  __syncthreads();
  // every group's weight (the ranked weights for the cut groups)
  auto mass_of = [&](int g, const GroupAcc& r, uint32_t tp, uint32_t tq, bool rs,
                     bool* badp) -> double {
    const int sp = state(tp, r.np, jp), sq = rs ? state(tq, r.nq, jq) : 1;
    if (!rs) return (resid ? r.ap : r.a) + (double)kept(sp, tp, r.np, jp) * Pk;
    if (g == sm.sg[0] || g == sm.sg[1]) {
      const int k = g == sm.sg[0] ? 0 : 1;
      if (badp) *badp |= sm.sbad[k] != 0;
      return sm.smass[k];
    }
    if (badp) *badp |= (r.bad & 1u) || ((r.bad & 2u) && sp == 1 && Pk > 0.0);
    return group_mass(r, true, sp, sq, 0u, Pk, Qk);
  };
  double loc = 0.0;
  bool bad = false;
  {
    uint32_t tp = tp0, tq = tq0;
    for (int g = ga; g < gb; ++g) {
      const GroupAcc r = rec(g);
      loc += mass_of(g, r, tp, tq, resid, &bad);
      tp += r.np;
      tq += r.nq;
    }
  }
  if (kQ && resid && block_reduce<kDrawNT>(bad ? 1 : 0, OpMax(), sm.ired) != 0) {
    // an unusable entry of the published residual row fails the session
    if (t < kWave) write_failed(b, SV_S_BAD_PROPOSAL, M, accepted_len, out_tokens, p_tok, q_tok);
    return;
  }
  double S;
  double before = block_exclusive_scan<kDrawNT, double>(loc, sm.dscan, &S);
  bool rs = resid;
  if (resid && S == 0.0) {  // residual without mass (rounding only): draw from p
    rs = false;
    loc = 0.0;
    uint32_t tp = tp0, tq = tq0;
    for (int g = ga; g < gb; ++g) {
      const GroupAcc r = rec(g);
      loc += mass_of(g, r, tp, tq, false, nullptr);
      tp += r.np;
      tq += r.nq;
    }
    before = block_exclusive_scan<kDrawNT, double>(loc, sm.dscan, &S);
  }
  const double tgt = job.u * S;
  // the group holding u * S, and the last group with weight
  if (t == 0) sm.gstar = -1;
  const int owner = block_reduce<kDrawNT>((gb > ga && before + loc > tgt) ? t : INT32_MAX,
                                          OpMin(), sm.ired);
  int lastg = -1;
  {
    uint32_t tp = tp0, tq = tq0;
    double run = before;
    bool found = false;
    for (int g = ga; g < gb; ++g) {
      const GroupAcc r = rec(g);
      const double mg = mass_of(g, r, tp, tq, rs, nullptr);
      if (t == owner && !found && run + mg > tgt) {
        found = true;
        sm.gstar = g;
        sm.gbase = run;
        sm.gtp = tp;
        sm.gtq = tq;
      }
      if (mg > 0.0) lastg = g;
      run += mg;
      tp += r.np;
      tq += r.nq;
    }
    // rounding kept the point past this range's groups: on from the next one
    if (t == owner && !found && gb < G) {
      sm.gstar = gb;
      sm.gbase = run;
      sm.gtp = tp;
      sm.gtq = tq;
    }
  }
  const int lg = block_reduce<kDrawNT>(lastg, OpMax(), sm.ired);
  if (lg >= 0 && lastg == lg) {  // this thread's range holds it: its ties before
    uint32_t tp = tp0, tq = tq0;
    for (int g = ga; g < lg; ++g) {
      const GroupAcc r = rec(g);
      tp += r.np;
      tq += r.nq;
    }
    sm.ltp = tp;
    sm.ltq = tq;
  }
  __syncthreads();
  // the group holding u * S weighed again id by id, on past it if rounding
  // moved the point, else the largest id with weight
  int32_t pick = INT32_MAX;
  const int gstar = sm.gstar;
  if (gstar >= 0) {
    double run = sm.gbase;
    uint32_t tp = sm.gtp, tq = sm.gtq;
    for (int g = gstar; g < G && pick == INT32_MAX; ++g) {
      const ScanRes sr =
          group_scan<Tr, kQ>(d, rs, g, scan_load<Tr, kQ>(d, rs, g), tp, tq, run, tgt, true, sm, kt, tabs_kept);
      pick = sr.first;
      run += sr.total;
      tp += sr.np;
      tq += sr.nq;
    }
  }
  if (pick == INT32_MAX) {
    pick = -1;
    if (lg >= 0)
      pick = group_scan<Tr, kQ>(d, rs, lg, scan_load<Tr, kQ>(d, rs, lg), sm.ltp, sm.ltq, 0.0, 0.0,
                                false, sm, kt, tabs_kept).lastpos;
  }
  if (wid == 0) write_verdict(b, v, pick, M, accepted_len, out_tokens, p_tok, q_tok);
}

// After a window of the in-order reading (positions up to hi read for every
// undecided session): one wave per session finds the position at which its
// round ends, if any is at or before hi, and records it in decided[b]; a
// session whose every position through m+1 passes ends at m+1.  The next
// window's row kernels skip decided sessions.
constexpr int kAdvanceNT = 256;
__global__ __launch_bounds__(kAdvanceNT) void k_advance(
    const float* __restrict__ qrows, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ m, const int32_t* __restrict__ rule,
    const sv_sampling* __restrict__ sampling, int B, int M, int V, uint64_t seed, uint32_t round,
    const int32_t* __restrict__ sess_status, const RowRec* __restrict__ rows,
    const double* __restrict__ unif, int has_draft_logits, int hi, int32_t* __restrict__ decided) {
  const int b = (int)blockIdx.x * (kAdvanceNT / kWave) + (int)threadIdx.x / kWave;
  if (b >= B || decided[b] != 0 || sess_status[b] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int mb = m[b];
  const int rl = rule[b];
  const RowRec* rr = rows + (size_t)b * (2 * M + 1);
  const int n = hi < mb + 1 ? hi : mb + 1;
  const LanePos pos = lane_position(b, lane, mb, n, rl, tokens, M, V, qrows, rr, unif, seed,
                                    sampling[b].session_key, round);
  const int f = inorder_end(n, mb, rl, rl == SV_RULE_SPECULATIVE && has_draft_logits, rr, M, pos);
  if (lane == 0) {
    if (f > 0) decided[b] = f;
    else if (hi >= mb + 1) decided[b] = mb + 1;
  }
}

}  // namespace

void launch_advance(const LaunchArgs& a, hipStream_t st, int hi) {
  const int per = kAdvanceNT / kWave;
  const unsigned grid = (unsigned)((a.B + per - 1) / per);
  hipLaunchKernelGGL(k_advance, dim3(grid), dim3(kAdvanceNT), 0, st, a.qrows, a.tokens, a.m,
                     a.rule, a.sampling, a.B, a.M, a.V, a.seed, a.round, a.sess_status, a.rows,
                     a.unif, a.draft != nullptr ? 1 : 0, hi, a.decided);
}

template <class Tr, bool kQ>
static void launch_finalize_t(const LaunchArgs& a, hipStream_t st) {
  using E = typename Tr::elem_t;
  const unsigned grid = (unsigned)((size_t)a.B * (size_t)a.draw_C);
  hipLaunchKernelGGL((k_finalize<Tr, kQ>), dim3(grid), dim3(kDrawNT), 0, st, (const E*)a.target,
                     (const E*)a.draft, a.qrows, a.tokens, a.m, a.rule, a.sampling, a.B, a.M, a.V,
                     a.seed, a.round, a.sess_status, a.rows, a.accepted_len, a.out_tokens, a.p_tok,
                     a.q_tok, a.sup_id, a.sup_p, a.unif, a.groups, a.draw_ctr, a.draw_flag,
                     a.draw_token, a.draw_C, a.draw_gw, a.decided);
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
