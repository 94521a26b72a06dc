// sv_rows_dense32.hip -- the binary32 rows that the single-pass kernel leaves
// (top-p, or top-k above 64; sv_rows_dense32.hpp), one wave64 per row slot.
// A row it hands back, the same wave profiles exactly (sv_rows_exact.hpp).
// It runs after the single-pass kernel, which writes the sessions' statuses.
#include "sv_kernels.hpp"
#include "sv_rows_dense32.hpp"
#include "sv_rows_exact.hpp"

namespace sv {

namespace {

__global__ __launch_bounds__(kWave)
__attribute__((amdgpu_waves_per_eu(3))) void k_rows_dense32(
    const uint32_t* __restrict__ target, const uint32_t* __restrict__ draft,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling,
    const int32_t* __restrict__ sess_status, int B, int M, int V, RowRec* __restrict__ rows,
    uint32_t* __restrict__ draw_flag, uint32_t draw_token, const int32_t* __restrict__ decided,
    int win_lo, int win_w) {
  __shared__ __align__(16) unsigned char lds[dense32::kLdsBytes];
  const int lane = __lane_id();
  const int slot_g = launch_slot((int)blockIdx.x, M, win_lo, win_w);
  if (slot_g < 0) return;
  const int R = 2 * M + 1;
  const int b = slot_g / R;
  const int slot = slot_g - b * R;
  if (b >= B) return;
  if (win_lo > 1 && decided[b] != 0) return;  // decided by an earlier window
  if (sess_status[b] != 0) return;
  const int mb = m[b];
  const int rl = rule[b];
  const bool is_target = slot <= M;
  const int i = is_target ? slot + 1 : slot - M;  // 1-based position
  // draft rows are profiled only when draft logits are given (not with q rows)
  if (is_target ? (i > mb + 1) : (rl != SV_RULE_SPECULATIVE || i > mb || draft == nullptr))
    return;
  const sv_sampling smp = sampling[b];
  if (row_uses_topk_kernel(SV_FP32, rl, smp) || row_uses_dense_kernel(SV_FP32, rl, smp, V))
    return;  // the single-pass kernel's row
  if (lane == 0) draw_flag[b] = draw_token;  // a row without a listed support
  const int32_t x = i <= mb ? tokens[(size_t)b * M + (i - 1)] : -1;
  const uint32_t* row = is_target ? target + ((size_t)b * (M + 1) + (i - 1)) * (size_t)V
                                  : draft + ((size_t)b * M + (i - 1)) * (size_t)V;
  RowRec* rec = rows + (size_t)slot_g;
  if (dense32::row_profile(row, V, smp, x, rec, lds))
    exact::profile_row<F32, kWave>(row, V, smp, rl == SV_RULE_GREEDY, x, rec, nullptr);
}

}  // namespace

void launch_rows_dense32(const LaunchArgs& a, hipStream_t st) {
  // bf16 rows, and binary32 rows of small vocabularies, are all profiled by the
  // single-pass kernel: no launch
  if (a.dtype != SV_FP32 || a.V <= kDense32MinV) return;
  const size_t slots =
      a.win_w == 0 ? (size_t)a.B * (2 * a.M + 1) : (size_t)a.B * 2 * (size_t)a.win_w;
  hipLaunchKernelGGL(k_rows_dense32, dim3((unsigned)slots), dim3(kWave), 0, st,
                     (const uint32_t*)a.target, (const uint32_t*)a.draft, a.tokens, a.m, a.rule,
                     a.sampling, a.sess_status, a.B, a.M, a.V, a.rows, a.draw_flag, a.draw_token,
                     a.decided, a.win_lo, a.win_w);
}

}  // namespace sv
