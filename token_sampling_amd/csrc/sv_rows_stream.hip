// sv_rows_stream.hip -- the single-pass row kernel: one wave64 per row slot
// streams the row once and computes its profile (SDCP Sec. 4.1) by the path
// its profile needs:
//   top-k class (greedy, temperature 0, 1 <= top_k <= 64): topk::row_profile;
//   dense class (temperature > 0, top-k off or above 64, with or without
//     top-p): dense::row_profile.
// A row a path hands back (a top-k region that overflows, a cut below the
// dense histogram's window, logits beyond binary32 exponent range) is profiled
// exactly by the same wave (sv_rows_exact.hpp).  Binary32 rows take the top-k
// path on 32-bit keys (topk32::row_profile) or, with temperature alone, the
// dense pass (dense::row_profile_f32_untruncated); binary32 rows with top-p or
// top-k above 64 are left to k_rows_dense32 (vocabularies above kDense32MinV;
// below, this wave profiles them exactly).  Each wave also takes its
// session's statuses that need no logits (SDCP Table 2, Sec. 6.3 step 5:
// limit, profile, q availability, drafted tokens in range); the wave of a
// session's first row slot records them for the kernels that follow.
//
// With SDCP verifier values (Sec. 6.4) the grid starts with extra workgroups
// that compute them, one value per lane; they depend on no logits, so they
// run while the row waves stream.
#include <stdlib.h>

#include "sv_commit.hpp"
#include "sv_kernels.hpp"
#include "sv_rows_dense.hpp"
#include "sv_rows_exact.hpp"
#include "sv_rows_topk.hpp"
#include "sv_rows_topk32.hpp"
#include "sv_sdcp.hpp"

namespace sv {

namespace {

// A session's status decidable without reading logits, by one wave (lane i
// checks drafted token i; m <= 64).
__device__ inline int session_status(int b, const int32_t* tokens, const int32_t* m,
                                     const int32_t* rule, const sv_sampling* sampling, int M,
                                     int V, bool has_draft) {
  const int lane = __lane_id();
  const int mb = m[b];
  const int rl = rule[b];
  const sv_sampling s = sampling[b];
  if (mb < 1 || mb > M) return SV_S_LIMIT;
  if ((rl != SV_RULE_GREEDY && rl != SV_RULE_SPECULATIVE && rl != SV_RULE_RELAXED) ||
      s.reserved != 0 || s.top_p_milli > 1000)
    return SV_S_BAD_PROFILE;
  if (rl == SV_RULE_SPECULATIVE && !has_draft) return SV_S_Q_UNAVAILABLE;
  const int32_t x = lane < mb ? tokens[(size_t)b * M + lane] : 0;
  if (__ballot(x < 0 || x >= V)) return SV_S_BAD_PROPOSAL;
  return 0;
}

// Verifier value g of the [B, 2M+1] table: j = g mod (2M+1) < M is the
// acceptance value of position j+1, j >= M the additional-token value of
// position j-M+1.  Only speculative-sampling sessions with a valid m use
// them (and relaxed-rule sessions, their additional-token values), and only at
// positions up to m (acceptance) or m+1 (additional token).
__device__ inline void sdcp_value(int64_t g, const sv_sdcp_session* __restrict__ sessions,
                                  const int32_t* __restrict__ m, const int32_t* __restrict__ rule,
                                  int B, int M, double* __restrict__ unif) {
  const int R = 2 * M + 1;
  const int64_t b = g / R;
  if (b >= B) return;
  const int j = (int)(g - b * R);
  const uint32_t purpose = j < M ? 0u : 1u;
  const int pos = j < M ? j + 1 : j - M + 1;
  const int mb = m[b];
  const int rl = rule[b];
  if (rl != SV_RULE_SPECULATIVE && !(rl == SV_RULE_RELAXED && purpose == 1)) return;
  if (mb < 1 || mb > M || pos > mb + (int)purpose) return;
  const uint2* rec = (const uint2*)(sessions + b);  // 32 bytes, 8-byte aligned
  const uint2 id01 = rec[0], id23 = rec[1], sd = rec[2], rd = rec[3];
  const uint32_t id[4] = {__builtin_bswap32(id01.x), __builtin_bswap32(id01.y),
                          __builtin_bswap32(id23.x), __builtin_bswap32(id23.y)};
  const uint64_t seed = ((uint64_t)sd.y << 32) | sd.x;
  const uint64_t bits = sdcp::verifier_bits(seed, id, rd.x, (uint32_t)pos, purpose);
  unif[g] = (double)bits * 0x1p-53;
}

// LDS of one wave: the top-k region, or the dense histogram
constexpr int kDenseBytes = dense::kWin * 4;
constexpr int kLdsWords = (topk::kCap * 8 > kDenseBytes ? topk::kCap * 8 : kDenseBytes) / 8;

#ifndef SV_STREAM_WAVES_PER_EU
#define SV_STREAM_WAVES_PER_EU 5
#endif
template <class Tr>
__global__ __launch_bounds__(kWave)
__attribute__((amdgpu_waves_per_eu(SV_STREAM_WAVES_PER_EU))) void k_rows_stream(
    const typename Tr::elem_t* __restrict__ target, const typename Tr::elem_t* __restrict__ draft,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling, int has_draft,
    int B, int M, int V, int32_t* __restrict__ sess_status, uint32_t* __restrict__ draw_ctr,
    uint32_t* __restrict__ draw_flag, uint32_t draw_token, RowRec* __restrict__ rows,
    int32_t* __restrict__ sup_id, double* __restrict__ sup_p,
    const sv_sdcp_session* __restrict__ sessions, double* __restrict__ unif, int n_value_blocks,
    int32_t* __restrict__ decided, int win_lo, int win_w,
    const sv_contract* __restrict__ contracts, const sv_session_state* __restrict__ states,
    uint32_t* __restrict__ chain, int n_chain_blocks) {
  using E = typename Tr::elem_t;
  __shared__ __align__(16) uint64_t lds[kLdsWords];  // top-k region or dense histogram
  const int lane = __lane_id();
  const int n_front = n_chain_blocks + n_value_blocks;
  if ((int)blockIdx.x < n_front) {
    if ((int)blockIdx.x < n_chain_blocks) {
      __builtin_amdgcn_s_setprio(3);
      commit::chain_drafted((int64_t)blockIdx.x * kWave + lane, contracts, states, tokens, m, B, M,
                            chain);
    } else {
      sdcp_value((int64_t)((int)blockIdx.x - n_chain_blocks) * kWave + lane, sessions, m, rule, B,
                 M, unif);
    }
    return;
  }
  const int R = 2 * M + 1;
  const int slot_g = launch_slot((int)blockIdx.x - n_front, M, win_lo, win_w);
  if (slot_g < 0) return;
  const int b = slot_g / R;
  const int slot = slot_g - b * R;
  if (b >= B) return;
  if (win_lo > 1 && decided[b] != 0) return;  // decided by an earlier window
  const int st = session_status(b, tokens, m, rule, sampling, M, V, has_draft != 0);
  if (slot == 0 && lane == 0) {
    sess_status[b] = st;
    draw_ctr[b] = 0u;  // the draw's chunk counter, for the per-session kernel
    if (decided) decided[b] = 0;
  }
  if (st != 0) return;
  const int mb = m[b];
  const int rl = rule[b];
  const bool is_target = slot <= M;
  const int i = is_target ? slot + 1 : slot - M;  // 1-based position
  // draft rows are profiled only when draft logits are given (not with q rows)
  if (is_target ? (i > mb + 1) : (rl != SV_RULE_SPECULATIVE || i > mb || draft == nullptr))
    return;
  const sv_sampling smp = sampling[b];
  const int32_t x = i <= mb ? tokens[(size_t)b * M + (i - 1)] : -1;
  const E* row = is_target ? target + ((size_t)b * (M + 1) + (i - 1)) * (size_t)V
                           : draft + ((size_t)b * M + (i - 1)) * (size_t)V;
  RowRec* rec = rows + (size_t)slot_g;
  bool back;
  if (row_uses_topk_kernel(Tr::kDtype, rl, smp)) {
    const bool one_hot = rl == SV_RULE_GREEDY || smp.temperature_milli == 0;
    const int k = one_hot ? 1 : (int)smp.top_k;
    const size_t so = (size_t)slot_g * kSupMax;
    if constexpr (Tr::kDtype == SV_BF16)
      back = topk::row_profile(row, V, k, one_hot, smp, x, rec, sup_id + so, sup_p + so, lds);
    else
      back = topk32::row_profile(row, V, k, one_hot, smp, x, rec, sup_id + so, sup_p + so, lds);
  } else if (row_uses_dense_kernel(Tr::kDtype, rl, smp, V)) {
    if (lane == 0) draw_flag[b] = draw_token;  // a row without a listed support
    if constexpr (Tr::kDtype == SV_BF16)
      back = dense::row_profile(row, V, smp, x, rec, (uint32_t*)lds);
    else
      back = dense::row_profile_f32_untruncated(row, V, smp, x, rec);
  } else if (V <= kDense32MinV) {
    back = true;  // a binary32 cut row of a small vocabulary: profiled exactly below
  } else {
    return;  // binary32 rows with top-p or top-k above 64: k_rows_dense32
  }
  if (back) {  // the exact profile, by this wave
    if (lane == 0) draw_flag[b] = draw_token;
    exact::profile_row<Tr, kWave>(row, V, smp, rl == SV_RULE_GREEDY, x, rec, nullptr);
  }
}

// The same row slots with each row split over S waves of one workgroup, for
// launches with few rows: one wave alone needs about 90 us for a 128K-logit
// top-50 row (57 us of it streaming with ten tiles in flight, the rest
// candidate insertion), so a few long rows leave the chip idle.  Wave w streams
// tiles [w T / S, (w + 1) T / S).  Top-k class: with its own first bound (a
// bound from any part of the row bounds the row's k-th best), it cuts its
// region to its k best, and wave 0 merges the S lists (at most S * 64 <= kCap
// entries) and finishes the row.  Dense class: into its own histogram window
// and sums, which wave 0 merges (dense::row_profile_split).
#ifndef SV_SPLIT_WAVES_PER_EU
#define SV_SPLIT_WAVES_PER_EU 4
#endif
template <int S>
__global__ __launch_bounds__(S * kWave)
__attribute__((amdgpu_waves_per_eu(SV_SPLIT_WAVES_PER_EU))) void k_rows_split(
    const uint16_t* __restrict__ target, const uint16_t* __restrict__ draft, int32_t dtype,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling, int has_draft,
    int B, int M, int V, int32_t* __restrict__ sess_status, uint32_t* __restrict__ draw_ctr,
    uint32_t* __restrict__ draw_flag, uint32_t draw_token, RowRec* __restrict__ rows,
    int32_t* __restrict__ sup_id, double* __restrict__ sup_p,
    const sv_sdcp_session* __restrict__ sessions, double* __restrict__ unif, int n_value_blocks,
    int32_t* __restrict__ decided, int win_lo, int win_w,
    const sv_contract* __restrict__ contracts, const sv_session_state* __restrict__ states,
    uint32_t* __restrict__ chain, int n_chain_blocks) {
  // top-k-class rows use the first TS waves (the merged lists fit one region)
  constexpr int TS = S < 4 ? S : 4;
  static_assert(TS * kSupMax <= topk::kCap, "the merged lists fit one region");
  constexpr int kHists = S * dense::kWin / 2;  // S histograms
  constexpr int kRegions = S * topk::kCap > kHists ? S * topk::kCap : kHists;
  constexpr int kWords = kRegions > kLdsWords ? kRegions : kLdsWords;
  __shared__ __align__(16) uint64_t lds[kWords];  // S regions, or S dense histograms
  __shared__ dense::PartRec parts_s[S];
  __shared__ int cnt_s[S], ovf_s[S];
  __shared__ uint32_t mm_s[S], um_s[S];
  const int lane = __lane_id();
  const int wid = (int)threadIdx.x / kWave;
  const int n_front = n_chain_blocks + n_value_blocks;
  if ((int)blockIdx.x < n_front) {
    if ((int)blockIdx.x < n_chain_blocks) {
      __builtin_amdgcn_s_setprio(3);
      commit::chain_drafted((int64_t)blockIdx.x * (S * kWave) + threadIdx.x, contracts, states,
                            tokens, m, B, M, chain);
    } else {
      sdcp_value((int64_t)((int)blockIdx.x - n_chain_blocks) * (S * kWave) + threadIdx.x,
                 sessions, m, rule, B, M, unif);
    }
    return;
  }
  const int R = 2 * M + 1;
  const int slot_g = launch_slot((int)blockIdx.x - n_front, M, win_lo, win_w);
  if (slot_g < 0) return;
  const int b = slot_g / R;
  const int slot = slot_g - b * R;
  if (b >= B) return;
  if (win_lo > 1 && decided[b] != 0) return;  // decided by an earlier window
  const int st = session_status(b, tokens, m, rule, sampling, M, V, has_draft != 0);
  if (wid == 0 && slot == 0 && lane == 0) {
    sess_status[b] = st;
    draw_ctr[b] = 0u;
    if (decided) decided[b] = 0;
  }
  if (st != 0 || dtype != SV_BF16) return;
  const int mb = m[b];
  const int rl = rule[b];
  const bool is_target = slot <= M;
  const int i = is_target ? slot + 1 : slot - M;  // 1-based position
  if (is_target ? (i > mb + 1) : (rl != SV_RULE_SPECULATIVE || i > mb || draft == nullptr))
    return;
  const sv_sampling smp = sampling[b];
  const int32_t x = i <= mb ? tokens[(size_t)b * M + (i - 1)] : -1;
  const uint16_t* row = is_target ? target + ((size_t)b * (M + 1) + (i - 1)) * (size_t)V
                                  : draft + ((size_t)b * M + (i - 1)) * (size_t)V;
  RowRec* rec = rows + (size_t)slot_g;
  if (row_uses_topk_kernel(SV_BF16, rl, smp)) {
    const bool one_hot = rl == SV_RULE_GREEDY || smp.temperature_milli == 0;
    const int k = one_hot ? 1 : (int)smp.top_k;
    const int T = topk::row_tiles(row, V);
    uint64_t* reg = lds + wid * topk::kCap;
    if (wid < TS) {
      topk::WaveState s;
      topk::chunk_scan(row, V, k, wid * T / TS, (wid + 1) * T / TS, s, reg);
      const int n = s.overflow ? 0 : topk::region_cut(reg, s.n, k).n;
      struct PairMax {
        __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return stream::max_u16x2(a, b); }
      };
      const uint32_t mm = wave_reduce(s.magmax, PairMax()), um = wave_reduce(s.umax, PairMax());
      if (lane == 0) {
        cnt_s[wid] = n;
        ovf_s[wid] = s.overflow ? 1 : 0;
        mm_s[wid] = mm;
        um_s[wid] = um;
      }
    }
    __syncthreads();
    if (wid != 0) return;
    int ovf = 0, total = cnt_s[0];
    uint32_t mmax = mm_s[0], umax = um_s[0];
#pragma unroll
    for (int w = 1; w < TS; ++w) {
      ovf |= ovf_s[w];
      mmax = stream::max_u16x2(mmax, mm_s[w]);
      umax = stream::max_u16x2(umax, um_s[w]);
      const int c = cnt_s[w];
      if (lane < c) reg[total + lane] = lds[w * topk::kCap + lane];
      total += c;
    }
    ovf |= ovf_s[0];
    if (ovf) {  // a part overflowed its region: the exact profile, by this wave
      if (lane == 0) draw_flag[b] = draw_token;
      exact::profile_row<Bf16, kWave>(row, V, smp, rl == SV_RULE_GREEDY, x, rec, nullptr);
      return;
    }
    const size_t so = (size_t)slot_g * kSupMax;
    const bool nan = max((int)(mmax & 0xFFFFu), (int)(mmax >> 16)) > 0x7F80 ||
                     max((int)(umax & 0xFFFFu), (int)(umax >> 16)) > 0xFF80;
    topk::row_finish<topk::Key16>(reg, total, k, nan, 0x7F80, one_hot, smp.temperature_milli,
                                  smp.top_p_milli, x, rec, sup_id + so, sup_p + so);
  } else if (row_uses_dense_kernel(SV_BF16, rl, smp, V)) {
    // the S waves stream S parts of the row; wave 0 merges them and finishes
    if (wid == 0 && lane == 0) draw_flag[b] = draw_token;  // a row without a listed support
    if (dense::row_profile_split<S>(row, V, smp, x, rec, (uint32_t*)lds, parts_s, wid))
      exact::profile_row<Bf16, kWave>(row, V, smp, rl == SV_RULE_GREEDY, x, rec, nullptr);
  }
}

}  // namespace

// Waves per top-k-class row.  Measured on b256 rows (bf16, V = 128256): a
// part of a row costs more than its share, since every part starts with a
// low threshold and inserts many candidates, so splitting pays only while the
// launch has under about one row per SIMD: 4 waves per row below 1024 rows
// (272 rows: 91 -> 59 us; 768 rows: 104 -> 91 us), 1 above (2304 rows: 120 us
// with 1 wave, 132 us with 2).  SV_ROWS_SPLIT (1, 2, 4 or 8) overrides the choice.
#ifndef SV_LATE_SPLIT
#define SV_LATE_SPLIT 4
#endif
#ifndef SV_TAIL_SPLIT
#define SV_TAIL_SPLIT 1
#endif
static int rows_split_factor(const LaunchArgs& a) {
  if (a.dtype != SV_BF16) return 1;  // binary32 rows: one wave per row
  const char* env = getenv("SV_ROWS_SPLIT");
  if (env) {
    const int s = atoi(env);
    if (s == 1 || s == 2 || s == 4 || s == 8) return s;
  }
  // In-order windows: the second holds the few sessions the first left
  // undecided (few rows: split); the later ones are either empty, where
  // dispatch dominates and a one-wave workgroup costs least, or hold sessions
  // that accept long runs, with rows enough for one wave each.
  if (a.win_w != 0 && a.win_index >= 2) return SV_TAIL_SPLIT;
  if (a.win_w != 0 && a.win_lo > 1) return SV_LATE_SPLIT;
  const int W = a.win_w == 0 ? a.M + 1 : a.win_w;  // target positions per session
  const size_t rows = (size_t)a.B * W + (a.draft ? (size_t)a.B * (W < a.M ? W : a.M) : 0);
  return rows < 1024 ? 4 : 1;
}

// Row slots of the launch (every slot, or a window's), and the SDCP values'
// workgroups of per_block values each (all values, in the first launch only).
static size_t launch_slots(const LaunchArgs& a) {
  if (a.win_w == 0) return (size_t)a.B * (2 * a.M + 1);
  return (size_t)a.B * 2 * a.win_w;
}
static int value_blocks(const LaunchArgs& a, int per_block) {
  if (!a.sdcp || a.win_lo > 1) return 0;
  const size_t values = (size_t)a.B * (2 * a.M + 1);
  return (int)((values + per_block - 1) / per_block);
}
// The drafted tokens' digest chains, one session per work-item (first launch
// only).
static int chain_blocks(const LaunchArgs& a, int per_block) {
  if (!a.chain || a.win_lo > 1) return 0;
  return (a.B + per_block - 1) / per_block;
}

template <int S>
static void launch_split(const LaunchArgs& a, hipStream_t st, size_t slots) {
  const int per_block = S * kWave;
  const int n_value_blocks = value_blocks(a, per_block);
  const int n_chain_blocks = chain_blocks(a, per_block);
  const unsigned grid = (unsigned)(slots + n_value_blocks + n_chain_blocks);
  hipLaunchKernelGGL((k_rows_split<S>), dim3(grid), dim3(per_block), 0, st,
                     (const uint16_t*)a.target, (const uint16_t*)a.draft, a.dtype, a.tokens, a.m,
                     a.rule, a.sampling, (a.draft != nullptr || a.qrows != nullptr) ? 1 : 0, a.B,
                     a.M, a.V, a.sess_status, a.draw_ctr, a.draw_flag, a.draw_token, a.rows,
                     a.sup_id, a.sup_p, a.sdcp, a.unif, n_value_blocks, a.decided, a.win_lo,
                     a.win_w, a.contracts, a.states, a.chain, n_chain_blocks);
}

void launch_rows_stream(const LaunchArgs& a, hipStream_t st) {
  const size_t slots = launch_slots(a);
  const int split = rows_split_factor(a);
  if (split == 2) return launch_split<2>(a, st, slots);
  if (split == 4) return launch_split<4>(a, st, slots);
  if (split == 8) return launch_split<8>(a, st, slots);
  const int n_value_blocks = value_blocks(a, kWave);
  const int n_chain_blocks = chain_blocks(a, kWave);
  const unsigned grid = (unsigned)(slots + n_value_blocks + n_chain_blocks);
  const int has_draft = (a.draft != nullptr || a.qrows != nullptr) ? 1 : 0;
  if (a.dtype == SV_BF16)
    hipLaunchKernelGGL(k_rows_stream<Bf16>, dim3(grid), dim3(kWave), 0, st,
                       (const uint16_t*)a.target, (const uint16_t*)a.draft, a.tokens, a.m, a.rule,
                       a.sampling, has_draft, a.B, a.M, a.V, a.sess_status, a.draw_ctr,
                       a.draw_flag, a.draw_token, a.rows, a.sup_id, a.sup_p, a.sdcp, a.unif,
                       n_value_blocks, a.decided, a.win_lo, a.win_w, a.contracts, a.states,
                       a.chain, n_chain_blocks);
  else
    hipLaunchKernelGGL(k_rows_stream<F32>, dim3(grid), dim3(kWave), 0, st,
                       (const uint32_t*)a.target, (const uint32_t*)a.draft, a.tokens, a.m, a.rule,
                       a.sampling, has_draft, a.B, a.M, a.V, a.sess_status, a.draw_ctr,
                       a.draw_flag, a.draw_token, a.rows, a.sup_id, a.sup_p, a.sdcp, a.unif,
                       n_value_blocks, a.decided, a.win_lo, a.win_w, a.contracts, a.states,
                       a.chain, n_chain_blocks);
}

}  // namespace sv
