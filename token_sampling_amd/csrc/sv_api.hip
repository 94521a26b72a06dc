// sv_api.hip -- the C ABI of libspecverify (declared in include/specverify.h).
//
// sv_verify and sv_verify_sdcp check their scalar arguments on the host, carve
// the caller's workspace and enqueue the kernels on the caller's stream:
//   single-pass row kernel (session statuses, then each row by the top-k or
//   the dense path) -> binary32 cut-row kernel (binary32 rows with top-p or
//   top-k above 64) -> finalize
//   (acceptance, and the additional token's draw).
// With SDCP values the single-pass kernel's first workgroups also compute them;
// sv_verify_commit adds workgroups in front of those that chain the drafted
// tokens' digests, and the commit kernel after the finalize.
// sv_verify_early enqueues the row kernels once per window of positions, each
// followed by the advance kernel, and the finalize after the last window.
// Neither call synchronises or allocates.
#include <limits.h>

#include <atomic>
#include <mutex>

#include "sv_kernels.hpp"

namespace sv {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

WorkspaceLayout workspace_layout(int32_t B, int32_t M, int32_t V) {
  WorkspaceLayout L;
  size_t off = 0;
  L.rows_off = off;
  off = align_up(off + (size_t)B * (2 * (size_t)M + 1) * sizeof(RowRec), 256);
  L.status_off = off;
  off = align_up(off + (size_t)B * sizeof(int32_t), 256);
  const size_t slots = (size_t)B * (2 * (size_t)M + 1);
  L.supid_off = off;
  off = align_up(off + slots * kSupMax * sizeof(int32_t), 256);
  L.supp_off = off;
  off = align_up(off + slots * kSupMax * sizeof(double), 256);
  L.unif_off = off;
  off = align_up(off + slots * sizeof(double), 256);
  L.chunk_off = off;
  off = align_up(off + (size_t)B * (((size_t)V + kGroup - 1) / kGroup) * sizeof(GroupRec), 256);
  L.ctr_off = off;
  off = align_up(off + (size_t)B * sizeof(uint32_t), 256);
  L.flag_off = off;
  off = align_up(off + (size_t)B * sizeof(uint32_t), 256);
  L.decided_off = off;
  off = align_up(off + (size_t)B * sizeof(int32_t), 256);
  L.chain_off = off;
  off = align_up(off + (size_t)B * (size_t)M * 32, 256);
  L.total = off;
  return L;
}

static bool sizes_ok(int32_t B, int32_t M, int32_t V, int32_t dtype) {
  if (B < 1 || M < 1 || M > SV_M_MAX || V < 1 || V > SV_V_MAX) return false;
  if (dtype != SV_BF16 && dtype != SV_FP32) return false;
  // launches: one wave per row slot (plus one per 64 SDCP values) and 1024
  // work-items per session must stay within a 32-bit work-item count;
  // element counts must fit a signed 64-bit index
  if (B > SV_B_MAX) return false;
  const unsigned long long slots = (unsigned long long)B * (2ull * (unsigned)M + 1ull);
  if (slots > (unsigned long long)SV_SLOTS_MAX) return false;
  const unsigned long long elems = (unsigned long long)B * ((unsigned)M + 1ull) * (unsigned)V;
  if (elems > (unsigned long long)(LLONG_MAX / 4)) return false;
  return true;
}

}  // namespace sv

extern "C" size_t sv_workspace_bytes(int32_t B, int32_t M, int32_t V) {
  if (!sv::sizes_ok(B, M, V, SV_BF16)) return 0;
  return sv::workspace_layout(B, M, V).total;
}

namespace sv {

// Each window of the in-order reading after the first covers kWindowGrowth
// times the positions of the one before it.
#ifndef SV_WINDOW_GROWTH
#define SV_WINDOW_GROWTH 4
#endif
constexpr int kWindowGrowth = SV_WINDOW_GROWTH;

// The benchmark hook's events (sv_bench_row_events), per host thread.
static thread_local hipEvent_t g_row_ev[3] = {nullptr, nullptr, nullptr};

// A value per call for the rows' draw flags (never 0, so that a cleared
// workspace matches no call).
static uint32_t next_draw_token() {
  static std::atomic<uint32_t> counter{0};
  uint32_t t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  if (t == 0) t = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  return t;
}

// Shared by the entry points: sdcp == null takes the Philox values from
// (seed, round); otherwise the SDCP Sec. 6.4 values of each session's record.
// window0 == 0 reads every row of a session (the SDCP reading); window0 >= 1
// reads them in order, in windows of window0, 4 window0, 16 window0, ...
// positions, each window only for the sessions its predecessors left
// undecided.
static int verify_impl(const void* target_logits, const void* draft_logits, const float* q_rows,
                       int32_t dtype, const int32_t* draft_tokens, const int32_t* m, const int32_t* rule,
                       const sv_sampling* sampling, const sv_sdcp_session* sdcp, int32_t B,
                       int32_t M, int32_t V, uint64_t seed, uint32_t round,
                       int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                       size_t workspace_bytes, const sv_probe* probe, void* stream,
                       int32_t window0 = 0, const sv_commit_io* commit = nullptr) {
  if (!target_logits || !draft_tokens || !m || !rule || !sampling || !accepted_len ||
      !out_tokens || !workspace)
    return SV_ERR_ARG;
  if (commit && (!commit->contracts || !commit->states || !commit->emitted_len ||
                 !commit->action))
    return SV_ERR_ARG;
  if (!sizes_ok(B, M, V, dtype)) return SV_ERR_ARG;
  const WorkspaceLayout L = workspace_layout(B, M, V);
  if (workspace_bytes < L.total) return SV_ERR_WORKSPACE;

  LaunchArgs a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.qrows = q_rows;
  a.dtype = dtype;
  a.tokens = draft_tokens;
  a.m = m;
  a.rule = rule;
  a.sampling = sampling;
  a.B = B;
  a.M = M;
  a.V = V;
  a.seed = seed;
  a.round = round;
  a.accepted_len = accepted_len;
  a.out_tokens = out_tokens;
  a.p_tok = probe ? probe->p_tok : nullptr;
  a.q_tok = probe ? probe->q_tok : nullptr;
  char* ws = (char*)workspace;
  a.rows = (RowRec*)(ws + L.rows_off);
  a.sess_status = (int32_t*)(ws + L.status_off);
  a.sup_id = (int32_t*)(ws + L.supid_off);
  a.sup_p = (double*)(ws + L.supp_off);
  a.sdcp = sdcp;
  a.unif = sdcp ? (double*)(ws + L.unif_off) : nullptr;
  a.groups = (GroupRec*)(ws + L.chunk_off);
  a.draw_ctr = (uint32_t*)(ws + L.ctr_off);
  const DrawChunks dc = draw_chunks(B, V);
  a.draw_C = dc.C;
  a.draw_gw = dc.gw;
  a.draw_flag = (uint32_t*)(ws + L.flag_off);
  a.draw_token = next_draw_token();
  a.decided = window0 > 0 ? (int32_t*)(ws + L.decided_off) : nullptr;
  a.win_lo = 1;
  a.win_w = 0;
  a.win_index = 0;
  a.contracts = commit ? commit->contracts : nullptr;
  a.states = commit ? commit->states : nullptr;
  a.chain = commit ? (uint32_t*)(ws + L.chain_off) : nullptr;

  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();  // report only errors raised by the launches below
  if (g_row_ev[0]) (void)hipEventRecord(g_row_ev[0], st);
  if (window0 == 0) {
    launch_rows_stream(a, st);
    if (g_row_ev[1]) (void)hipEventRecord(g_row_ev[1], st);
    launch_rows_dense32(a, st);
  } else {
    // windows of positions [lo, lo + w), w growing, the last one ending at M+1
    int w = window0;
    for (int lo = 1; lo <= M + 1;) {
      a.win_lo = lo;
      a.win_w = w < M + 2 - lo ? w : M + 2 - lo;
      launch_rows_stream(a, st);
      launch_rows_dense32(a, st);
      const int hi = lo + a.win_w - 1;
      if (hi < M + 1) launch_advance(a, st, hi);  // after the last window: the finalize
      lo = hi + 1;
      w = w < 64 ? kWindowGrowth * w : w;
      ++a.win_index;
    }
    if (g_row_ev[1]) (void)hipEventRecord(g_row_ev[1], st);
  }
  if (g_row_ev[2]) (void)hipEventRecord(g_row_ev[2], st);
  launch_finalize(a, st);
  if (commit)
    launch_commit(commit->contracts, commit->states, m, accepted_len, out_tokens,
                  commit->self_decode_ok, B, M, commit->emitted_len, commit->action, a.chain, st);
  if (hipGetLastError() != hipSuccess) return SV_ERR_DEVICE;
  return SV_OK;
}

}  // namespace sv

extern "C" int sv_verify(const void* target_logits, const void* draft_logits, int32_t dtype,
                         const int32_t* draft_tokens, const int32_t* m, const int32_t* rule,
                         const sv_sampling* sampling, int32_t B, int32_t M, int32_t V,
                         uint64_t seed, uint32_t round, int32_t* accepted_len,
                         int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                         const sv_probe* probe, void* stream) {
  return sv::verify_impl(target_logits, draft_logits, nullptr, dtype, draft_tokens, m, rule,
                         sampling, nullptr, B, M, V, seed, round, accepted_len, out_tokens,
                         workspace, workspace_bytes, probe, stream);
}

extern "C" int sv_verify_sdcp(const void* target_logits, const void* draft_logits,
                              int32_t dtype, const int32_t* draft_tokens, const int32_t* m,
                              const int32_t* rule, const sv_sampling* sampling,
                              const sv_sdcp_session* sessions, int32_t B, int32_t M, int32_t V,
                              int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                              size_t workspace_bytes, const sv_probe* probe, void* stream) {
  if (!sessions) return SV_ERR_ARG;
  return sv::verify_impl(target_logits, draft_logits, nullptr, dtype, draft_tokens, m, rule,
                         sampling, sessions, B, M, V, 0, 0, accepted_len, out_tokens, workspace,
                         workspace_bytes, probe, stream);
}

extern "C" int sv_verify_qrows(const void* target_logits, int32_t dtype, const float* q_rows,
                               const int32_t* draft_tokens, const int32_t* m, const int32_t* rule,
                               const sv_sampling* sampling, const sv_sdcp_session* sessions,
                               int32_t B, int32_t M, int32_t V, uint64_t seed, uint32_t round,
                               int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                               size_t workspace_bytes, const sv_probe* probe, void* stream) {
  return sv::verify_impl(target_logits, nullptr, q_rows, dtype, draft_tokens, m, rule, sampling,
                         sessions, B, M, V, seed, round, accepted_len, out_tokens, workspace,
                         workspace_bytes, probe, stream);
}

extern "C" int sv_verify_early(const void* target_logits, const void* draft_logits,
                               const float* q_rows, int32_t dtype, const int32_t* draft_tokens,
                               const int32_t* m, const int32_t* rule, const sv_sampling* sampling,
                               const sv_sdcp_session* sessions, int32_t B, int32_t M, int32_t V,
                               uint64_t seed, uint32_t round, int32_t window0,
                               int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                               size_t workspace_bytes, const sv_probe* probe, void* stream) {
  if (window0 < 1 || window0 > SV_M_MAX + 1) return SV_ERR_ARG;
  if (draft_logits && q_rows) return SV_ERR_ARG;
  return sv::verify_impl(target_logits, draft_logits, q_rows, dtype, draft_tokens, m, rule,
                         sampling, sessions, B, M, V, seed, round, accepted_len, out_tokens,
                         workspace, workspace_bytes, probe, stream, window0);
}

extern "C" int sv_verify_commit(const void* target_logits, const void* draft_logits,
                                int32_t dtype, const int32_t* draft_tokens, const int32_t* m,
                                const int32_t* rule, const sv_sampling* sampling,
                                const sv_sdcp_session* sessions, int32_t B, int32_t M, int32_t V,
                                uint64_t seed, uint32_t round, int32_t* accepted_len,
                                int32_t* out_tokens, const sv_commit_io* commit, void* workspace,
                                size_t workspace_bytes, const sv_probe* probe, void* stream) {
  if (!commit) return SV_ERR_ARG;
  return sv::verify_impl(target_logits, draft_logits, nullptr, dtype, draft_tokens, m, rule,
                         sampling, sessions, B, M, V, seed, round, accepted_len, out_tokens,
                         workspace, workspace_bytes, probe, stream, 0, commit);
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing (sv_verify_noalloc): its workspace is
// a file-scope device array, one per GPU, held until the process ends.  Host
// code never uses the array's name as an address: on the first call on each
// device, with that device current, hipGetSymbolAddress gives this device's
// copy, kept per device and passed to the kernels like a caller's workspace.
namespace sv {
constexpr size_t kScratchBytes = (size_t)SV_NOALLOC_WORKSPACE_MAX;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices] = {};
static std::mutex g_scratch_mu;

// This device's copy of scratch, or null (with *rc set) if it cannot be had.
static void* device_scratch(int* rc) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = SV_ERR_DEVICE;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      *rc = SV_ERR_DEVICE;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace sv

extern "C" int sv_verify_noalloc(const void* target_logits, const void* draft_logits,
                                 int32_t dtype, const int32_t* draft_tokens, const int32_t* m,
                                 const int32_t* rule, const sv_sampling* sampling, int32_t B,
                                 int32_t M, int32_t V, uint64_t seed, uint32_t round,
                                 int32_t* accepted_len, int32_t* out_tokens, const sv_probe* probe,
                                 void* stream) {
  if (!target_logits || !draft_tokens || !m || !rule || !sampling || !accepted_len ||
      !out_tokens || !sv::sizes_ok(B, M, V, dtype))
    return SV_ERR_ARG;
  if (sv::workspace_layout(B, M, V).total > sv::kScratchBytes) return SV_ERR_WORKSPACE;
  int rc = SV_OK;
  void* ws = sv::device_scratch(&rc);
  if (!ws) return rc;
  return sv::verify_impl(target_logits, draft_logits, nullptr, dtype, draft_tokens, m, rule,
                         sampling, nullptr, B, M, V, seed, round, accepted_len, out_tokens, ws,
                         sv::kScratchBytes, probe, stream);
}

extern "C" int sv_bench_row_events(void* start, void* mid, void* stop) {
  sv::g_row_ev[0] = (hipEvent_t)start;
  sv::g_row_ev[1] = (hipEvent_t)mid;
  sv::g_row_ev[2] = (hipEvent_t)stop;
  return SV_OK;
}

extern "C" const char* sv_strerror(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_ERR_ARG: return "invalid argument (null pointer, size out of range or unknown dtype)";
    case SV_ERR_DEVICE: return "a kernel launch failed";
    case SV_ERR_WORKSPACE: return "workspace smaller than sv_workspace_bytes()";
    default: return "unknown error code";
  }
}

extern "C" const char* sv_status_str(int status) {
  if (status >= 0) return "accepted";
  switch (status) {
    case SV_S_BAD_PROPOSAL: return "sdcp-bad-proposal: token out of range or q_i(x_i) == 0";
    case SV_S_LIMIT: return "sdcp-limit: m outside [1, M]";
    case SV_S_Q_UNAVAILABLE: return "sdcp-q-unavailable: rule 2 without draft logits";
    case SV_S_BAD_PROFILE: return "bad profile: unknown rule, top_p_milli > 1000 or reserved != 0";
    case SV_S_BAD_LOGITS: return "bad logits: NaN or +inf, or no finite logit, in a row read";
    default: return "unknown status";
  }
}

extern "C" int sv_version(void) { return SV_VERSION; }
