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
//
// With SDCP verifier values (Sec. 6.4) the grid starts with extra workgroups
// that compute them, one value per lane; they depend on no logits, so they
// run while the row waves stream.
#include "sv_kernels.hpp"
#include "sv_rows_dense.hpp"
#include "sv_rows_topk.hpp"
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

constexpr int kLdsWords = (topk::kCap * 8 > dense::kWin * 4 ? topk::kCap * 8 : dense::kWin * 4) / 8;

#ifndef SV_STREAM_WAVES_PER_EU
#define SV_STREAM_WAVES_PER_EU 5
#endif
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(SV_STREAM_WAVES_PER_EU))) void k_rows_stream(
    const uint16_t* __restrict__ target, const uint16_t* __restrict__ draft, int32_t dtype,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling, int has_draft,
    int B, int M, int V, int32_t* __restrict__ sess_status, RowRec* __restrict__ rows,
    int32_t* __restrict__ sup_id, double* __restrict__ sup_p,
    const sv_sdcp_session* __restrict__ sessions, double* __restrict__ unif, int n_value_blocks) {
  __shared__ __align__(16) uint64_t lds[kLdsWords];  // top-k region or dense histogram
  const int lane = __lane_id();
  if ((int)blockIdx.x < n_value_blocks) {
    sdcp_value((int64_t)blockIdx.x * kWave + lane, sessions, m, rule, B, M, unif);
    return;
  }
  const int R = 2 * M + 1;
  const int slot_g = blockIdx.x - n_value_blocks;
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
  // draft rows are profiled only when draft logits are given (not with q rows)
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
    const size_t so = (size_t)slot_g * kSupMax;
    topk::row_profile(row, V, k, one_hot, smp, x, rec, sup_id + so, sup_p + so, lds);
  } else if (row_uses_dense_kernel(SV_BF16, rl, smp, V)) {
    dense::row_profile(row, V, smp, x, rec, (uint32_t*)lds);
  }
}

}  // namespace

void launch_rows_stream(const LaunchArgs& a, hipStream_t st) {
  const size_t slots = (size_t)a.B * (2 * a.M + 1);
  const int n_value_blocks = a.sdcp ? (int)((slots + kWave - 1) / kWave) : 0;
  const unsigned grid = (unsigned)(slots + n_value_blocks);
  hipLaunchKernelGGL(k_rows_stream, dim3(grid), dim3(kWave), 0, st, (const uint16_t*)a.target,
                     (const uint16_t*)a.draft, a.dtype, a.tokens, a.m, a.rule, a.sampling,
                     (a.draft != nullptr || a.qrows != nullptr) ? 1 : 0, a.B, a.M, a.V, a.sess_status, a.rows, a.sup_id,
                     a.sup_p, a.sdcp, a.unif, n_value_blocks);
}

}  // namespace sv
