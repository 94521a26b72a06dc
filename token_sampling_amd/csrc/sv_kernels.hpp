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
  // the draw from rows without listed supports: each session's row is cut
  // into groups of kGroup ids, recorded by draw_C workgroups per session,
  // draw_gw groups per wave
  struct GroupRec* groups;  // [B, ceil(V / kGroup)]
  uint32_t* draw_ctr;       // [B] workgroups finished; cleared by the single-pass row kernel
  int32_t draw_C, draw_gw;
  // draw_flag[b] == draw_token: a row of session b has no listed support (set by
  // the row kernels of this call); only then do a session's extra draw
  // workgroups have work.  A value left by an earlier call that equals the
  // token costs them an acceptance pass, nothing more.
  uint32_t* draw_flag;  // [B]
  uint32_t draw_token;
  // In-order reading (null decided: every row of a session is read).  The
  // row kernels then read the positions win_lo .. win_lo + win_w - 1 of the
  // sessions still undecided; decided[b] is the position (1-based) at which
  // session b's round ends, 0 while undecided (cleared by the row kernels'
  // first window).
  int32_t* decided;  // [B]
  int32_t win_lo, win_w;
  int32_t win_index;  // 0 for the first window
  // sv_verify_commit: the first row launch's front workgroups chain the
  // drafted tokens' digests (sv_commit.hpp) from each session's state, for the
  // commit after the verdict (null chain: no commit)
  const sv_contract* contracts;  // [B]
  const sv_session_state* states;  // [B]
  uint32_t* chain;  // [B, M] digests after the first 1..M drafted tokens, 8 words each
};

// Ids per group record of the draw.
constexpr int kGroup = 2048;

// What one group of ids leaves for the draw's last workgroup.  The cut
// keys' ties kept by rank (rows cut by the dense path) all weigh the same,
// so the group's weights are recorded for both cases, kept and left out, and
// the session's tie counts decide which case holds where (only a group
// holding a row's cut needs its ties ranked).  Residual draws: weights
// max(0, p - q) where p > 0; p ties / q ties are tokens of the cut key of p /
// of q in a row cut by rank.  Stored as six 64-bit words.
struct GroupRec {
  double a;    // weight of the tokens that are ties of neither row
  double bp;   // residual: weight of the p ties (not q ties), all kept
  double cq1;  // residual: weight of the q ties (not p ties), all kept
  double cq0;  // residual: the same tokens with no q tie kept (their p)
  double ap;   // residual: p of the tokens that are not p ties (a draw from p)
  uint32_t ties;     // p ties | q ties << 16
  uint32_t npq_bad;  // tokens that are both | published q unusable << 16 (bit
                     // 0 where p > 0 outside the p ties, bit 1 at a p tie)
};
static_assert(sizeof(GroupRec) == 48, "GroupRec layout");

// Workgroups per session for the draw: about kDrawTarget in all (B * C), each
// wave taking gw whole groups.
#ifndef SV_DRAW_TARGET
#define SV_DRAW_TARGET 1024
#endif
constexpr long long kDrawTarget = SV_DRAW_TARGET;
struct DrawChunks {
  int32_t C, gw;
};
__host__ __device__ inline DrawChunks draw_chunks(int32_t B, int32_t V) {
  const long long G = ((long long)V + kGroup - 1) / kGroup;
  long long C = (kDrawTarget + (long long)B - 1) / B;
  const long long cmax = (G + 3) / 4;
  if (C > cmax) C = cmax;
  if (C < 1) C = 1;
  const long long gw = (G + 4 * C - 1) / (4 * C);
  C = (G + 4 * gw - 1) / (4 * gw);
  return DrawChunks{(int32_t)C, (int32_t)gw};
}

// Rows whose support lies among the 64 best tokens take the single-pass
// kernel's top-k path (bf16 or binary32): greedy rows, temperature-0 rows,
// 1 <= top_k <= 64.
__host__ __device__ inline bool row_uses_topk_kernel(int32_t dtype, int32_t rule,
                                                     const sv_sampling& s) {
  (void)dtype;
  if (rule == SV_RULE_GREEDY || s.temperature_milli == 0) return true;
  return s.top_k >= 1 && s.top_k <= 64;
}

// The single-pass kernel's dense path takes every other bf16 row (temperature
// > 0 with top-k off or above 64, with or without top-p), and the binary32
// rows with temperature alone (top-k and top-p off); other binary32 rows take
// k_rows_dense32 (sv_rows_dense32.hip).
__host__ __device__ inline bool row_uses_dense_kernel(int32_t dtype, int32_t rule,
                                                      const sv_sampling& s, int32_t V) {
  if (row_uses_topk_kernel(dtype, rule, s)) return false;
  if (dtype == SV_BF16) return true;
  return s.top_p_milli >= 1000 && (s.top_k == 0 || s.top_k >= (uint32_t)V);
}

// Binary32 rows with top-p or top-k above 64 of a vocabulary at most this
// size are profiled exactly by the single-pass kernel's wave (the exact
// profile's passes over at most 16 KiB, in cache), which spares the launch of
// the cut-row kernel k_rows_dense32 for small vocabularies.
constexpr int kDense32MinV = 4096;

struct WorkspaceLayout {
  size_t rows_off, status_off, supid_off, supp_off, unif_off, chunk_off, ctr_off, flag_off,
      decided_off, chain_off, total;
};

// Row slot g of the launch: every slot of every session (win_w == 0), or the
// positions win_lo .. win_lo + win_w - 1 of each session, its target rows then
// its draft rows.  Returns the slot in the [B, 2M+1] record array, or -1 for
// a draft position past M.
__device__ inline int launch_slot(int g, int M, int win_lo, int win_w) {
  if (win_w == 0) return g;
  const int per = 2 * win_w;
  const int b = g / per;
  const int k = g - b * per;
  const bool is_target = k < win_w;
  const int i = win_lo + (is_target ? k : k - win_w);  // 1-based position
  if (!is_target && i > M) return -1;
  return b * (2 * M + 1) + (is_target ? i - 1 : M + i);
}

WorkspaceLayout workspace_layout(int32_t B, int32_t M, int32_t V);

void launch_rows_stream(const LaunchArgs& a, hipStream_t st);
void launch_rows_dense32(const LaunchArgs& a, hipStream_t st);
void launch_finalize(const LaunchArgs& a, hipStream_t st);
void launch_advance(const LaunchArgs& a, hipStream_t st, int hi);
void launch_commit(const sv_contract* contracts, sv_session_state* states, const int32_t* m,
                   const int32_t* accepted_len, int32_t* out_tokens, const uint8_t* self_decode_ok,
                   int B, int M, int32_t* emitted_len, int32_t* action, const uint32_t* chain,
                   hipStream_t st);

}  // namespace sv
