// sv_rows_stream.hip -- the single-pass row kernel: one wave64 per row slot
// streams the row once and computes its profile (SDCP Sec. 4.1) by the path
// its profile needs:
//   top-k class (greedy, temperature 0, 1 <= top_k <= 64): topk::row_profile;
//   dense class (temperature > 0, top-k off, with or without top-p):
//     dense::row_profile.
// Rows of other profiles, and rows a path hands back, are left to the
// generic kernel.  Each wave also takes its session's statuses that need no
// logits (SDCP Table 2, Sec. 6.3 step 5: limit, profile, q availability,
// drafted tokens in range); the wave of a session's first row slot records
// them for the kernels that follow.
#include "sv_kernels.hpp"
#include "sv_rows_dense.hpp"
#include "sv_rows_topk.hpp"

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
  if ((rl != SV_RULE_GREEDY && rl != SV_RULE_SPECULATIVE) || s.reserved != 0 || s.top_p_milli > 1000)
    return SV_S_BAD_PROFILE;
  if (rl == SV_RULE_SPECULATIVE && !has_draft) return SV_S_Q_UNAVAILABLE;
  const int32_t x = lane < mb ? tokens[(size_t)b * M + lane] : 0;
  if (__ballot(x < 0 || x >= V)) return SV_S_BAD_PROPOSAL;
  return 0;
}

constexpr int kLdsWords = (topk::kCap * 8 > dense::kWin * 4 ? topk::kCap * 8 : dense::kWin * 4) / 8;

#ifndef SV_STREAM_WAVES_PER_EU
#define SV_STREAM_WAVES_PER_EU 5
#endif
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(SV_STREAM_WAVES_PER_EU))) void k_rows_stream(
    const uint16_t* __restrict__ target, const uint16_t* __restrict__ draft, int32_t dtype,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling, int has_draft,
    int B, int M, int V, int32_t* __restrict__ sess_status, RowRec* __restrict__ rows,
    int32_t* __restrict__ sup_id, double* __restrict__ sup_p) {
  __shared__ __align__(16) uint64_t lds[kLdsWords];  // top-k region or dense histogram
  const int lane = __lane_id();
  const int R = 2 * M + 1;
  const int slot_g = blockIdx.x;
  const int b = slot_g / R;
  const int slot = slot_g - b * R;
  if (b >= B) return;
  const int st = session_status(b, tokens, m, rule, sampling, M, V, has_draft != 0);
  if (slot == 0 && lane == 0) sess_status[b] = st;
  if (st != 0 || dtype != SV_BF16) return;
  const int mb = m[b];
  const int rl = rule[b];
  const bool is_target = slot <= M;
  const int i = is_target ? slot + 1 : slot - M;  // 1-based position
  if (is_target ? (i > mb + 1) : (rl != SV_RULE_SPECULATIVE || i > mb)) return;
  const sv_sampling smp = sampling[b];
  const int32_t x = i <= mb ? tokens[(size_t)b * M + (i - 1)] : -1;
  const uint16_t* row = is_target ? target + ((size_t)b * (M + 1) + (i - 1)) * (size_t)V
                                  : draft + ((size_t)b * M + (i - 1)) * (size_t)V;
  RowRec* rec = rows + (size_t)slot_g;
  if (row_uses_topk_kernel(SV_BF16, rl, smp)) {
    const bool one_hot = rl == SV_RULE_GREEDY || smp.temperature_milli == 0;
    const int k = one_hot ? 1 : (int)smp.top_k;
    const size_t so = (size_t)slot_g * kSupMax;
    topk::row_profile(row, V, k, one_hot, smp, x, rec, sup_id + so, sup_p + so, lds);
  } else if (row_uses_dense_kernel(SV_BF16, rl, smp, V)) {
    dense::row_profile(row, V, smp, x, rec, (uint32_t*)lds);
  }
}

}  // namespace

void launch_rows_stream(const LaunchArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)a.B * (2 * a.M + 1));
  hipLaunchKernelGGL(k_rows_stream, dim3(grid), dim3(kWave), 0, st, (const uint16_t*)a.target,
                     (const uint16_t*)a.draft, a.dtype, a.tokens, a.m, a.rule, a.sampling,
                     a.draft != nullptr ? 1 : 0, a.B, a.M, a.V, a.sess_status, a.rows, a.sup_id,
                     a.sup_p);
}

}  // namespace sv
