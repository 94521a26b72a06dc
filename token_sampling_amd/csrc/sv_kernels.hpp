// sv_kernels.hpp -- launch interface between the host entry points and the
// kernels of libspecverify.
#pragma once

#include "sv_common.hpp"

namespace sv {

struct LaunchArgs {
  const void* target;
  const void* draft;   // draft logits, or null (no draft logits are read)
  const float* qrows;  // SDCP q_rows [B, M, V] in place of draft logits, or null
  int32_t dtype;
  const int32_t* tokens;
  const int32_t* m;
  const int32_t* rule;
  const sv_sampling* sampling;
  int32_t B, M, V;
  uint64_t seed;
  uint32_t round;
  int32_t* accepted_len;
  int32_t* out_tokens;
  double* p_tok;  // may be null
  double* q_tok;  // may be null
  // workspace carve-up
  RowRec* rows;         // [B, 2M+1]: target rows 1..M+1, then draft rows 1..M
  int32_t* sess_status; // [B], written by the single-pass row kernel
  int32_t* sup_id;      // [B, 2M+1, kSupMax] listed supports (ids ascending)
  double* sup_p;        // [B, 2M+1, kSupMax] their probabilities
  // SDCP Sec. 6.4 verifier values (null: Philox from seed, round)
  const sv_sdcp_session* sdcp;  // [B] per-session seed, id and round
  double* unif;                 // [B, 2M+1]: j < M acceptance value of position j+1,
                                // j >= M additional-token value of position j-M+1
};

// Row status written by a specialised row kernel that could not finish a row;
// the generic kernel then computes that row.
constexpr int32_t kRowFallback = 1;

// Rows whose support lies among the 64 best tokens take the single-pass
// kernel's top-k path (bf16 only): greedy rows, temperature-0 rows,
// 1 <= top_k <= 64.
__host__ __device__ inline bool row_uses_topk_kernel(int32_t dtype, int32_t rule,
                                                     const sv_sampling& s) {
  if (dtype != SV_BF16) return false;
  if (rule == SV_RULE_GREEDY || s.temperature_milli == 0) return true;
  return s.top_k >= 1 && s.top_k <= 64;
}

// Every other bf16 row takes the single-pass kernel's dense path: temperature
// > 0 with top-k off (top_k = 0 or top_k >= V) or above 64, with or without
// top-p.
__host__ __device__ inline bool row_uses_dense_kernel(int32_t dtype, int32_t rule,
                                                      const sv_sampling& s, int32_t V) {
  (void)V;
  return dtype == SV_BF16 && !row_uses_topk_kernel(dtype, rule, s);
}

struct WorkspaceLayout {
  size_t rows_off, status_off, supid_off, supp_off, unif_off, total;
};

WorkspaceLayout workspace_layout(int32_t B, int32_t M, int32_t V);

void launch_rows_stream(const LaunchArgs& a, hipStream_t st);
void launch_rows_generic(const LaunchArgs& a, hipStream_t st);
void launch_finalize(const LaunchArgs& a, hipStream_t st);

}  // namespace sv
