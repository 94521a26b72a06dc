/*
 * specverify.h -- C ABI of libspecverify, the MI355X (gfx950) verifier
 * acceptance step for speculative decoding.
 *
 * The operation follows the SDCP Internet-Draft "Speculative Decoding
 * Coordination Protocol (SDCP) for Distributed Inference with Multi-Level
 * Caches" (draft-li-mlc-inference-acceleration-00):
 *   Sec. 4.1  sampling profile: temperature, then top-k, then top-p; a
 *             temperature of zero is the argmax with ties to the smallest id;
 *   Sec. 6.3  step 5: for a rule that needs draft probabilities, q_i(x_i) must
 *             be non-zero at every proposed position before any random draw;
 *             step 7: the acceptance rule yields a accepted tokens plus one;
 *   Sec. 6.4  Rule 1 (greedy) and Rule 2 (speculative sampling), positions
 *             evaluated in order; verifier uniforms are 53-bit values keyed by
 *             seed, session, round, position and purpose (0 = acceptance
 *             test, 1 = additional token);
 *   Sec. 5.2  verdict: accepted a with 0 <= a <= M, emitted tokens;
 *   Table 2   problem types (sdcp-bad-proposal, sdcp-limit, sdcp-q-unavailable);
 *   Sec. 10.2.2  rule registry: 1 = greedy, 2 = speculative sampling.
 * and the textbook chapter "Inference: KV Cache, Batching, Speculative
 * Decoding", section "The acceptance rule" (residual max(0, p - q), bonus
 * token from p at position M+1).
 *
 * Readings where the pages are silent (the library implements exactly these):
 *  - draft distribution q_i = the same profile applied to draft logits row i;
 *  - uniforms of sv_verify: Philox4x64-10 (Salmon et al., SC'11) with key
 *    (seed, session_key) and counter (round, i, 0, 0), i = 1-based position;
 *    word 0 >> 11 times 2^-53 is the acceptance uniform, word 1 the
 *    additional-token uniform.  sv_verify_sdcp takes the draft's own values
 *    instead (HMAC-SHA-256, Sec. 6.4; see sv_sdcp_session);
 *  - top-k keeps exactly k tokens in the order (logit desc, id asc); top_k = 0
 *    or >= the number of finite logits is "off";
 *  - top-p keeps the shortest non-empty prefix of that order whose mass C
 *    (after top-k) satisfies 1000*C >= top_p_milli * Z_k; top_p_milli = 1000
 *    is "off";
 *  - -inf logits have probability zero; -0 and +0 are equal logits;
 *  - the additional token is the inverse CDF over ascending token ids;
 *  - NaN or +inf logits, or a row with no finite logit, in a row the rule
 *    reads: the session fails with SV_S_BAD_LOGITS.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_VERSION 1
#define SV_M_MAX 64          /* SDCP Sec. 4.1: m_max <= 64 */
#define SV_V_MAX (1 << 24)   /* largest vocabulary accepted */
#define SV_B_MAX (1 << 21)   /* most sessions per call */
#define SV_SLOTS_MAX (1 << 25) /* most row slots B * (2M + 1) per call */

/* Per-session sampling profile (SDCP Sec. 4.1 "sampling"), 24 bytes,
 * 8-byte aligned; passed as a DEVICE array [B]. */
typedef struct sv_sampling {
  uint32_t temperature_milli; /* T * 1000; 0 => one-hot argmax */
  uint32_t top_k;             /* 0 (or >= finite count) => off */
  uint32_t top_p_milli;       /* 0..1000; 1000 => off; > 1000 => SV_S_BAD_PROFILE */
  uint32_t reserved;          /* must be 0, else SV_S_BAD_PROFILE */
  uint64_t session_key;       /* the session's identity in the generator key */
} sv_sampling;

/* Optional per-call probe (host struct; every member may be NULL):
 *  p_tok, q_tok: DEVICE arrays [B, M] of float64, written for
 *    speculative-sampling sessions with p_i(x_i) and q_i(x_i) for i <= m[b]
 *    (every position, also past the first rejection); -1 elsewhere and for
 *    greedy or failed sessions. */
typedef struct sv_probe {
  double *p_tok;
  double *q_tok;
} sv_probe;

/* Per-session inputs of the SDCP verifier values (Sec. 6.4), 32 bytes, 8-byte
 * aligned; passed to sv_verify_sdcp as a DEVICE array [B].  The value for
 * 1-based position i and purpose (0 = acceptance test, 1 = additional token)
 * is HMAC-SHA-256 keyed with seed as eight octets in network byte order, over
 * "SDCP-VERIFY-1" || 0x00 || session_id || uint32(round) || uint32(i) ||
 * uint8(purpose) (integers in network byte order); the first 53 bits of the
 * MAC, most significant first, divided by 2^53. */
typedef struct sv_sdcp_session {
  uint8_t session_id[16]; /* the session's 16-octet identifier */
  uint64_t seed;          /* the sampling profile's seed (Sec. 4.1) */
  uint32_t round;         /* the round being verified (numbered from 1) */
  uint32_t reserved;      /* ignored; set to 0 */
} sv_sdcp_session;

/* Acceptance rules: 1 and 2 are SDCP's (Sec. 6.4, registry Sec. 10.2.2).  192,
 * from the registry's private-use range (192-255), is the relaxed rule of the
 * textbook chapter (section "Speculative decoding": acceptance by membership
 * of the target's top-k, which gives up sampling exactly from p); read as:
 * x_i is accepted while p_i(x_i) > 0, i.e.
 * while the target's profile could sample it (with top-k alone, membership of
 * the target's top-k); the additional token is drawn from p_{a+1} with the
 * purpose-1 value of position a+1; no draft row or q is read; the probe's
 * p_tok holds p_i(x_i) at every position and q_tok is -1. */
enum { SV_RULE_GREEDY = 1, SV_RULE_SPECULATIVE = 2, SV_RULE_RELAXED = 192 };
enum { SV_BF16 = 0, SV_FP32 = 1 };                   /* logits element type */

/* Call-level return codes of sv_verify, sv_verify_sdcp and sv_verify_qrows. */
enum {
  SV_OK = 0,
  SV_ERR_ARG = -1,       /* null pointer, bad size or dtype, size overflow */
  SV_ERR_DEVICE = -2,    /* a kernel launch failed */
  SV_ERR_WORKSPACE = -3  /* workspace smaller than sv_workspace_bytes() */
};

/* Per-session statuses written to accepted_len[b] (< 0) when a session fails;
 * that session's out_tokens row is then all -1.  Other sessions are unaffected.
 * Checked in this order. */
enum {
  SV_S_LIMIT = -2,         /* m[b] outside [1, M]          (sdcp-limit) */
  SV_S_BAD_PROFILE = -4,   /* rule not 1, 2 or 192, top_p_milli > 1000, reserved != 0 */
  SV_S_Q_UNAVAILABLE = -3, /* rule 2 and draft_logits == NULL (sdcp-q-unavailable) */
  SV_S_BAD_PROPOSAL = -1,  /* a token outside [0, V); or, after the logits check,
                              q_i(x_i) == 0 for some i <= m[b] (sdcp-bad-proposal) */
  SV_S_BAD_LOGITS = -5     /* NaN / +inf, or no finite logit, in a row the rule reads */
};

/* Bytes of device workspace sv_verify needs for (B, M, V).  0 if the sizes
 * are out of range. */
size_t sv_workspace_bytes(int32_t B, int32_t M, int32_t V);

/*
 * The batched acceptance step.  All array pointers are caller-owned DEVICE
 * memory, row-major and contiguous:
 *   target_logits [B, M+1, V] of dtype: target row i (1-based) of session b is
 *                 target_logits[b, i-1, :]; row M+1 scores the bonus position.
 *   draft_logits  [B, M, V] of dtype: draft row i is draft_logits[b, i-1, :];
 *                 may be NULL when no session uses rule 2 (a rule-2 session
 *                 then fails with SV_S_Q_UNAVAILABLE).  Greedy sessions never
 *                 read it.
 *   draft_tokens  [B, M] int32: x_i = draft_tokens[b, i-1]; entries i > m[b]
 *                 are ignored.
 *   m [B], rule [B] int32; sampling [B] sv_sampling.
 *   1 <= B <= SV_B_MAX, 1 <= M <= 64, B * (2M + 1) <= SV_SLOTS_MAX,
 *   1 <= V <= SV_V_MAX; a session uses rows
 *   1..m[b]+1 of the target and, for rule 2, rows 1..m[b] of the draft.
 *   seed, round: the generator key and counter for this call (SDCP rounds are
 *   numbered from 1; any value is accepted).
 * Outputs:
 *   accepted_len [B] int32: a in [0, m[b]] or a negative SV_S_* status;
 *   out_tokens [B, M+1] int32: x_1..x_a, then the additional token, then -1.
 *   probe: host struct pointer or NULL.
 * workspace: DEVICE memory of at least sv_workspace_bytes(B, M, V) bytes, not
 *   aliased with any other argument; its contents need not be initialised.
 * stream: hipStream_t to launch on; NULL = the default stream.
 *
 * The call only enqueues work: it is asynchronous with respect to the host,
 * allocates nothing, and keeps no pointer after returning.  Outputs are valid
 * once the stream has completed.  Concurrent calls need distinct workspaces
 * and outputs.  A session's result depends only on its own rows, tokens, m,
 * rule, sampling record, seed and round (not on B, its batch position, the
 * stream or repetition).
 * Returns SV_OK or an SV_ERR_* code; on an error nothing has been enqueued
 * (except for SV_ERR_DEVICE, where some kernels may have been launched).
 */
int sv_verify(const void *target_logits, const void *draft_logits, int32_t dtype,
              const int32_t *draft_tokens, const int32_t *m, const int32_t *rule,
              const sv_sampling *sampling, int32_t B, int32_t M, int32_t V, uint64_t seed,
              uint32_t round, int32_t *accepted_len, int32_t *out_tokens, void *workspace,
              size_t workspace_bytes, const sv_probe *probe, void *stream);

/*
 * sv_verify with the verifier values of SDCP Sec. 6.4 itself: each session's
 * acceptance tests and additional-token draw take the HMAC-SHA-256 values of
 * sessions[b] (a DEVICE array [B] of sv_sdcp_session, caller-owned, not
 * aliased with any output) in place of the Philox values of (seed, round);
 * sampling[b].session_key is not used.  Every other argument, output, status
 * and return code is as for sv_verify; the workspace size is the same.
 * sessions == NULL returns SV_ERR_ARG.  A session's result depends only on
 * its own rows, tokens, m, rule, sampling and sessions records.
 */
int sv_verify_sdcp(const void *target_logits, const void *draft_logits, int32_t dtype,
                   const int32_t *draft_tokens, const int32_t *m, const int32_t *rule,
                   const sv_sampling *sampling, const sv_sdcp_session *sessions, int32_t B,
                   int32_t M, int32_t V, int32_t *accepted_len, int32_t *out_tokens,
                   void *workspace, size_t workspace_bytes, const sv_probe *probe, void *stream);

/*
 * sv_verify with the draft distributions given as SDCP q_rows (Sec. 5.2):
 * q_rows [B, M, V] binary32 DEVICE array (caller-owned), row i of session b at
 * q_rows[b, i-1, :], the distribution x_i was drawn from.  The rows are used as
 * published: no profile, no renormalisation, values widened exactly to
 * binary64.  No draft logits are read.  q_rows may be NULL when no session uses
 * rule 2 (a rule-2 session then fails with SV_S_Q_UNAVAILABLE).
 * Reads: q_i(x_i) at every position i <= m[b], checked before any draw (Sec.
 * 6.3 step 5): a value that is not a positive finite number fails the session
 * with SV_S_BAD_PROPOSAL.  At the first rejection, the residual max(0, p - q)
 * reads q(y) only where p(y) > 0 (its weight is zero elsewhere); an entry read
 * there that is negative, NaN or infinite fails the session with
 * SV_S_BAD_PROPOSAL (found only when that row is the residual's).  Other
 * entries are never read.  The probe's q_tok holds the widened q_i(x_i).
 * sessions: SDCP value records as for sv_verify_sdcp, or NULL for the Philox
 * values of (seed, round) as for sv_verify.  Every other argument, output,
 * status and return code is as for sv_verify; the workspace size is the same.
 */
int sv_verify_qrows(const void *target_logits, int32_t dtype, const float *q_rows,
                    const int32_t *draft_tokens, const int32_t *m, const int32_t *rule,
                    const sv_sampling *sampling, const sv_sdcp_session *sessions, int32_t B,
                    int32_t M, int32_t V, uint64_t seed, uint32_t round, int32_t *accepted_len,
                    int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                    const sv_probe *probe, void *stream);

/*
 * The acceptance step read in order (textbook "Inference: KV Cache, Batching,
 * Speculative Decoding", "The acceptance rule": the proposals are checked one
 * after another and the first rejection ends the round).  Position i reads
 * target row i and, for rule 2, draft row i (or q_rows' q_i(x_i)); a
 * session's rows after the position that ends its round are never read.  The
 * rows are read in windows of positions: window0 positions first
 * (1..window0), then 4 window0, 16 window0, ... positions, the last one
 * ending at M+1, each window only for the sessions still undecided; fewer
 * windows cost fewer launches, smaller ones read fewer rows.
 * Statuses follow the order: the first position (1-based i <= m[b] + 1)
 * with a bad target or draft row fails the session with SV_S_BAD_LOGITS, one
 * with an unusable q_i(x_i) with SV_S_BAD_PROPOSAL, and a rejection ends the
 * round; problems in rows after that position are not seen.  This departs
 * from sv_verify, which checks every row and every q_i(x_i) before any
 * decision (SDCP Sec. 6.3 step 5); where every row of a session is usable and
 * every q_i(x_i) positive, the two give the same result.  The probes hold
 * p_i(x_i), q_i(x_i) for the positions up to the one ending the round, -1
 * after it.
 * draft_logits or q_rows (at most one of them, both DEVICE arrays laid out
 * as for sv_verify and sv_verify_qrows) gives rule 2's draft distributions;
 * sessions: SDCP value records as for sv_verify_sdcp, or NULL for the Philox
 * values of (seed, round).  1 <= window0 <= 65.  Every other argument, output,
 * status and return code is as for sv_verify; the workspace size is the same.
 * Returns SV_ERR_ARG for window0 out of range or both draft sources given.
 */
int sv_verify_early(const void *target_logits, const void *draft_logits, const float *q_rows,
                    int32_t dtype, const int32_t *draft_tokens, const int32_t *m,
                    const int32_t *rule, const sv_sampling *sampling,
                    const sv_sdcp_session *sessions, int32_t B, int32_t M, int32_t V,
                    uint64_t seed, uint32_t round, int32_t window0, int32_t *accepted_len,
                    int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                    const sv_probe *probe, void *stream);

/* ---------------------------------------------------------------------------
 * The verifier's commit step (SDCP Sec. 4.2, Sec. 6.3 steps 6-8, Sec. 6.5).
 * ------------------------------------------------------------------------- */
#define SV_STOP_MAX 8     /* stop tokens per contract */
#define SV_FALLBACK_MAX 8 /* fallback list entries per contract */

/* Verdict actions, SDCP Sec. 6.5.2. */
enum {
  SV_ACT_CONTINUE = 0,
  SV_ACT_REDUCE = 1,
  SV_ACT_SWITCH = 2,
  SV_ACT_SELF_DECODE = 3,
  SV_ACT_FINISH = 4,
  SV_ACT_FAIL = 5
};

/* The contract members the commit step reads (SDCP Sec. 4.1), 64 bytes,
 * 4-byte aligned; a DEVICE array [B]. */
typedef struct sv_contract {
  uint32_t m_max;      /* largest M (1..64); m_cap is restored up to it */
  uint32_t max_new;    /* most output tokens of the session */
  uint32_t low_rounds; /* R >= 1 */
  uint32_t low_ratio;  /* percent, 0..100; 0 = absent */
  uint32_t n_stop;     /* stop tokens used: min(n_stop, SV_STOP_MAX) */
  int32_t stop[SV_STOP_MAX];
  uint32_t n_fallback; /* entries used: min(n_fallback, SV_FALLBACK_MAX) */
  uint8_t fallback[SV_FALLBACK_MAX]; /* SV_ACT_REDUCE, _SWITCH, _SELF_DECODE, _FAIL */
} sv_contract;

/* A session's verifier state, 64 bytes, 4-byte aligned; a DEVICE array [B]
 * that sv_commit reads and updates.  Initially: digest = d[0] (see
 * sv_prefix_digest), n = 0, m_cap = the first round's limit, c = g = j = 0. */
typedef struct sv_session_state {
  uint8_t digest[32];   /* d[n] (Sec. 4.2) */
  uint32_t n;           /* committed output tokens */
  uint32_t m_cap;       /* the verdict's speculation limit (Sec. 6.5.1) */
  uint32_t c, g, j;     /* low-round counters (Sec. 6.5.2) */
  uint32_t reserved[3]; /* not used */
} sv_session_state;

/*
 * One round's commit for B sessions, enqueued on stream after the acceptance
 * step of the same round.  DEVICE arrays: contracts [B], states [B] (updated),
 * m [B] (the proposal lengths), accepted_len [B] and out_tokens [B, M+1] as
 * written by sv_verify / sv_verify_sdcp / sv_verify_qrows, self_decode_ok [B]
 * (1 where self_decode is permitted this round: the contract has self_load and
 * the verifier's load does not exceed it) or NULL (never permitted).
 * Outputs: emitted_len [B], action [B] (SV_ACT_*); out_tokens truncated in
 * place (entries past the committed ones become -1).  Per session:
 *  - accepted_len outside [0, M] (a failed session): nothing is committed, the
 *    state is unchanged, emitted_len = 0, action = -1;
 *  - truncation (Sec. 6.3 step 6): the a+1 emitted tokens end after the first
 *    stop token, and at max_new committed tokens in all;
 *  - commit (Sec. 6.3 step 7, Sec. 4.2): n += e and
 *    d[n+k] = SHA-256(d[n+k-1] || uint32(o_k)) for each committed token;
 *  - control (Sec. 6.5.2): the round is low if 100*a < low_ratio*m, or a == 0
 *    when low_ratio is 0; low -> c += 1, g = 0; else c = 0, g += 1 and j = 0
 *    when g reaches R.  When c reaches R, fallback entry j is applied (a
 *    self_decode that is not permitted is skipped), j advances past every entry
 *    applied or skipped, c = 0; with no entry left the action is fail;
 *    otherwise continue.  reduce sets m_cap = max(1, m_cap / 2); after a round
 *    that is not low m_cap is restored by one up to m_max (the gradual restore
 *    of Sec. 6.5.1).  When a stop token was committed or max_new was reached,
 *    the action is finish.
 * Calls that overlap on the same states race.  Returns SV_OK, SV_ERR_ARG
 * (null pointer, B or M out of range) or SV_ERR_DEVICE.
 */
int sv_commit(const sv_contract *contracts, sv_session_state *states, const int32_t *m,
              const int32_t *accepted_len, int32_t *out_tokens, const uint8_t *self_decode_ok,
              int32_t B, int32_t M, int32_t *emitted_len, int32_t *action, void *stream);

/* The commit step's arrays for sv_verify_commit (a HOST struct of DEVICE
 * pointers): contracts [B], states [B] (read and updated), self_decode_ok [B]
 * or NULL (never permitted); outputs emitted_len [B] and action [B].  Their
 * meaning is sv_commit's. */
typedef struct sv_commit_io {
  const sv_contract *contracts;
  sv_session_state *states;
  const uint8_t *self_decode_ok;
  int32_t *emitted_len;
  int32_t *action;
} sv_commit_io;

/*
 * One round's acceptance step and commit step in one call (SDCP Sec. 6.3
 * steps 5-8): sv_verify (sessions == NULL: Philox values from seed and round)
 * or sv_verify_sdcp (sessions != NULL: the Sec. 6.4 values; seed and round are
 * ignored), then sv_commit on its verdict, with the same arguments, outputs,
 * statuses and results, bit for bit.  The difference is only where the work
 * runs: the commit's digest links over the drafted tokens (Sec. 4.2) do not
 * depend on the verdict, so the row kernel's first workgroups compute them,
 * one session per work-item, while the rows stream; after the verdict each
 * session links at most the additional token.  These links read the states
 * and contracts while the row kernel runs, so nothing else may write them
 * during the call.  The workspace (sv_workspace_bytes) holds the links.
 * Returns SV_OK, SV_ERR_ARG (as sv_verify, or a null commit pointer or
 * member other than self_decode_ok), SV_ERR_WORKSPACE or SV_ERR_DEVICE.
 */
int sv_verify_commit(const void *target_logits, const void *draft_logits, int32_t dtype,
                     const int32_t *draft_tokens, const int32_t *m, const int32_t *rule,
                     const sv_sampling *sampling, const sv_sdcp_session *sessions, int32_t B,
                     int32_t M, int32_t V, uint64_t seed, uint32_t round, int32_t *accepted_len,
                     int32_t *out_tokens, const sv_commit_io *commit, void *workspace,
                     size_t workspace_bytes, const sv_probe *probe, void *stream);

/* d[0] of SDCP Sec. 4.2: SHA-256("SDCP-PREFIX-1" || 0x00 || contract_digest ||
 * uint32(P) || uint32(prompt[0]) || ... ), integers in network byte order.
 * HOST memory: contract_digest[32], prompt[P], out[32].  Runs on the host.
 * Returns SV_OK or SV_ERR_ARG. */
int sv_prefix_digest(const uint8_t *contract_digest, const int32_t *prompt, uint32_t P,
                     uint8_t *out);

/* contract_digest of SDCP Sec. 4.1: SHA-256("SDCP-CONTRACT-1" || 0x00 || cbor),
 * over the contract's deterministic CBOR encoding supplied by the caller.
 * HOST memory; runs on the host.  Returns SV_OK or SV_ERR_ARG. */
int sv_contract_digest(const uint8_t *cbor, size_t len, uint8_t *out);

/*
 * sv_verify for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call without a workspace argument.  Its workspace is a device array
 * inside the library, SV_NOALLOC_WORKSPACE_MAX bytes per GPU, set up on the
 * first call on each device and held until the process ends; the call itself
 * allocates and frees nothing.  Every call on one GPU shares that GPU's array
 * (a later call overwrites it; the kernels need none of its contents at the
 * start of a call), so calls that overlap on one GPU (other streams or host
 * threads) race and must be serialised by the caller.  Arguments, outputs,
 * statuses and return codes are those of sv_verify, plus SV_ERR_WORKSPACE
 * when sv_workspace_bytes(B, M, V) > SV_NOALLOC_WORKSPACE_MAX, and
 * SV_ERR_DEVICE when the array's device address cannot be obtained.
 */
#define SV_NOALLOC_WORKSPACE_MAX (128u << 20) /* bytes: B=1024, M=64, V=129280 needs 108 MiB */
int sv_verify_noalloc(const void *target_logits, const void *draft_logits, int32_t dtype,
                      const int32_t *draft_tokens, const int32_t *m, const int32_t *rule,
                      const sv_sampling *sampling, int32_t B, int32_t M, int32_t V, uint64_t seed,
                      uint32_t round, int32_t *accepted_len, int32_t *out_tokens,
                      const sv_probe *probe, void *stream);

/* Benchmark hook, not part of the acceptance step: hipEvent_t handles that
 * the sv_verify* calls made afterwards from the calling host thread record on
 * their launch stream, immediately before the row-profile kernels (start),
 * between the single-pass kernel and the kernel for the other rows (mid; read
 * in order: after the last window's kernels), and after them (stop), once per
 * call.  A NULL handle leaves its slot unrecorded; three NULLs turn the hook
 * off.  The caller owns the events and keeps them alive while it is on.
 * Returns SV_OK. */
int sv_bench_row_events(void *start, void *mid, void *stop);

/* Text for an sv_verify return code; never NULL. */
const char *sv_strerror(int code);

/* Text for a per-session status (accepted_len < 0); never NULL. */
const char *sv_status_str(int status);

/* SV_VERSION of the built library. */
int sv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
