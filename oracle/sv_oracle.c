/*
 * sv_oracle.c -- plain, slow, single-threaded CPU oracle for the verifier's
 * batched speculative-decoding acceptance step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file.  Only the test suite, the smoke check of the package entry
 * module and the CPU-baseline leg of the benchmark use it.  It shares no code,
 * header, table or constant with the GPU library; the two are compared, never
 * combined.
 *
 * Sources (cited by page title and section):
 *  [SDCP]  "Speculative Decoding Coordination Protocol (SDCP) for Distributed
 *          Inference with Multi-Level Caches" (IETF Internet-Draft
 *          draft-li-mlc-inference-acceleration-00):
 *          Sec. 2 (rounds are numbered from 1), Sec. 4.1 (sampling profile:
 *          temperature, then top-k, then top-p; temperature 0 = argmax with
 *          ties to the smallest id), Sec. 5.2 (verdict: 0 <= accepted <= M),
 *          Sec. 6.3 steps 5-7 (q rows checked before any random draw),
 *          Sec. 6.4 (Rule 1 greedy, Rule 2 speculative sampling, 53-bit
 *          uniforms with purpose 0 = acceptance test, 1 = additional token),
 *          Table 2 (problem types), Appendix A (worked greedy round).
 *  [TXT]   "Inference: KV Cache, Batching, Speculative Decoding", section
 *          "Speculative decoding" / "The acceptance rule" (rejection sampling,
 *          residual distribution proportional to max(0, p - q), bonus token
 *          when every proposal is accepted).
 *  [PHX]   Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *          1, 2, 3", SC'11 -- the Philox4x64 counter-based generator.
 *  [SHS]   FIPS 180-4, Secure Hash Standard, Sec. 4.1.2, 4.2.2, 5, 6.2 --
 *          SHA-256 (the hash the SDCP text names, via RFC 6234).
 *  [HMAC]  RFC 2104 -- HMAC, with SHA-256 (64-octet blocks).
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *  - ov_verify: the verifier's uniforms come from Philox4x64-10 keyed by
 *    (seed, session_key) at counter (round, i, 0, 0); word 0 gives the
 *    acceptance uniform and word 1 the additional-token uniform, each as its
 *    top 53 bits times 2^-53;
 *  - ov_verify_sdcp: the uniforms of SDCP Sec. 6.4 itself: HMAC-SHA-256 keyed
 *    with the session's seed (8 octets, network order) over "SDCP-VERIFY-1" ||
 *    0x00 || session id (16 octets) || uint32(round) || uint32(i) ||
 *    uint8(purpose); the first 53 bits of the MAC (most significant first)
 *    times 2^-53;
 *  - ov_verify, ov_verify_sdcp: q_i is the same sampling profile applied to
 *    the draft logits row i;
 *  - ov_verify_qrows: q_i is the published q_rows row (SDCP Sec. 5.2), binary32
 *    values widened exactly and used as given (no profile, no
 *    renormalisation).  q_i(x_i) must be a positive finite number, checked at
 *    every position before any draw (else BAD_PROPOSAL); the residual reads
 *    q_i(y) only where p_i(y) > 0, and an entry read there that is negative,
 *    NaN or infinite makes the session fail with BAD_PROPOSAL;
 *  - top-k keeps exactly k tokens in the order (logit desc, id asc);
 *  - top-p keeps the shortest non-empty prefix of that order whose mass C
 *    satisfies 1000*C >= top_p_milli * Z_k (Z_k = mass after top-k);
 *    top_p_milli = 1000 and top_k = 0 (or >= number of finite logits) are "off";
 *  - a -inf logit has probability 0; a NaN or +inf logit, or a row with no
 *    finite logit, makes the session fail with status BAD_LOGITS;
 *  - the inverse CDF walks token ids in ascending order and returns the first
 *    y whose running sum exceeds u*S;
 *  - an all-zero residual (reachable only through rounding) falls back to p_i;
 *  - rule 192 (private use, the relaxed rule): accept x_i while p_i(x_i) > 0;
 *    the additional token is drawn from p_{a+1} with the purpose-1 value of
 *    position a+1; no draft row or q is read;
 *  - ov_commit (SDCP Sec. 6.3 steps 6-8, 6.5): a session whose acceptance step
 *    failed commits nothing and keeps its state; the proposal length M of the
 *    low-round test is the session's m; m_cap is restored by one after every
 *    round that is not low (the text's example of a gradual restore), up to
 *    m_max; finish takes precedence over the escalation's action when a stop
 *    token was committed or max_new was reached.
 *
 * All floating-point arithmetic is IEEE binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OV_BF16 = 0, OV_FP32 = 1 };
/* rules: SDCP Sec. 10.2.2 (1, 2); 192 is a private-use value (192-255) for the
 * relaxed rule the textbook describes (accept a token the target's profile
 * could sample), which does not preserve the target distribution */
enum { OV_RULE_GREEDY = 1, OV_RULE_SPECULATIVE = 2, OV_RULE_RELAXED = 192 };
enum {
  OV_OK = 0,
  OV_ERR_ARG = -1,
  OV_ERR_NOMEM = -2,
  /* per-session statuses, SDCP Table 2 */
  OV_S_BAD_PROPOSAL = -1,
  OV_S_LIMIT = -2,
  OV_S_Q_UNAVAILABLE = -3,
  OV_S_BAD_PROFILE = -4,
  OV_S_BAD_LOGITS = -5
};

/* SDCP Sec. 4.1 "sampling" map; the session identity enters the generator key. */
typedef struct {
  uint32_t temperature_milli;
  uint32_t top_k;
  uint32_t top_p_milli;
  uint32_t reserved;
  uint64_t session_key;
} ov_sampling;

/* ------------------------------------------------------------------------ */
/* Philox4x64-10 [PHX]: ten rounds of two 64x64->128 multiplies, with the    */
/* key bumped by two Weyl constants between rounds.                          */
/* ------------------------------------------------------------------------ */
static const uint64_t PHX_MUL0 = 0xD2E7470EE14C6C93ULL;
static const uint64_t PHX_MUL1 = 0xCA5A826395121157ULL;
static const uint64_t PHX_WEYL0 = 0x9E3779B97F4A7C15ULL; /* golden ratio */
static const uint64_t PHX_WEYL1 = 0xBB67AE8584CAA73BULL; /* sqrt(3) - 1  */

void ov_philox4x64_10(const uint64_t counter[4], const uint64_t key[2], uint64_t out[4]) {
  uint64_t x0 = counter[0], x1 = counter[1], x2 = counter[2], x3 = counter[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    unsigned __int128 p0 = (unsigned __int128)PHX_MUL0 * x0;
    unsigned __int128 p1 = (unsigned __int128)PHX_MUL1 * x2;
    uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    uint64_t y0 = hi1 ^ x1 ^ k0;
    uint64_t y1 = lo1;
    uint64_t y2 = hi0 ^ x3 ^ k1;
    uint64_t y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    k0 += PHX_WEYL0;
    k1 += PHX_WEYL1;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* SDCP Sec. 6.4: a uniform in [0,1) is the first 53 bits of a random word
 * divided by 2^53.  purpose 0 = acceptance test, 1 = additional token. */
double ov_uniform(uint64_t seed, uint64_t session_key, uint32_t round, uint32_t i, int purpose) {
  uint64_t ctr[4] = {round, i, 0, 0};
  uint64_t key[2] = {seed, session_key};
  uint64_t o[4];
  ov_philox4x64_10(ctr, key, o);
  uint64_t word = purpose == 0 ? o[0] : o[1];
  return ldexp((double)(word >> 11), -53);
}

/* ------------------------------------------------------------------------ */
/* SHA-256 [SHS].  The round constants are the first 32 bits of the          */
/* fractional parts of the cube roots of the first 64 primes, the initial    */
/* hash value those of the square roots of the first 8 primes [SHS Sec.      */
/* 4.2.2, 5.3.3]; both are derived here from that definition.                */
/* ------------------------------------------------------------------------ */
static uint32_t SHA_K[64], SHA_H0[8];
static int sha_ready = 0;

static uint32_t frac32(double x) { return (uint32_t)ldexp(x - floor(x), 32); }

static void sha_init_constants(void) {
  if (sha_ready) return;
  int primes[64], n = 0;
  for (int c = 2; n < 64; ++c) {
    int prime = 1;
    for (int d = 2; d * d <= c; ++d)
      if (c % d == 0) { prime = 0; break; }
    if (prime) primes[n++] = c;
  }
  for (int i = 0; i < 64; ++i) SHA_K[i] = frac32(cbrt((double)primes[i]));
  for (int i = 0; i < 8; ++i) SHA_H0[i] = frac32(sqrt((double)primes[i]));
  sha_ready = 1;
}

static uint32_t rotr(uint32_t x, int r) { return (x >> r) | (x << (32 - r)); }

/* one 64-octet block into the hash state [SHS Sec. 6.2.2] */
static void sha256_block(uint32_t h[8], const uint8_t blk[64]) {
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t)blk[4 * t] << 24 | (uint32_t)blk[4 * t + 1] << 16 |
           (uint32_t)blk[4 * t + 2] << 8 | (uint32_t)blk[4 * t + 3];
  for (int t = 16; t < 64; ++t) {
    const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = s1 + w[t - 7] + s0 + w[t - 16];
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], k = h[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t T1 = k + S1 + ch + SHA_K[t] + w[t];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t T2 = S0 + maj;
    k = g; g = f; f = e; e = d + T1; d = c; c = b; b = a; a = T1 + T2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += k;
}

/* SHA-256 of msg[0..len): padding with 0x80, zeros and the 64-bit bit length
 * [SHS Sec. 5.1.1], then the blocks in order; the digest is the state words
 * big-endian [SHS Sec. 6.2.2]. */
void ov_sha256(const uint8_t *msg, size_t len, uint8_t out[32]) {
  sha_init_constants();
  uint32_t h[8];
  memcpy(h, SHA_H0, sizeof h);
  size_t done = 0;
  while (len - done >= 64) {
    sha256_block(h, msg + done);
    done += 64;
  }
  uint8_t tail[128];
  memset(tail, 0, sizeof tail);
  const size_t r = len - done;
  memcpy(tail, msg + done, r);
  tail[r] = 0x80;
  const size_t tl = r + 1 + 8 <= 64 ? 64 : 128;
  const uint64_t bits = (uint64_t)len * 8u;
  for (int i = 0; i < 8; ++i) tail[tl - 1 - i] = (uint8_t)(bits >> (8 * i));
  sha256_block(h, tail);
  if (tl == 128) sha256_block(h, tail + 64);
  for (int i = 0; i < 8; ++i) {
    out[4 * i] = (uint8_t)(h[i] >> 24);
    out[4 * i + 1] = (uint8_t)(h[i] >> 16);
    out[4 * i + 2] = (uint8_t)(h[i] >> 8);
    out[4 * i + 3] = (uint8_t)h[i];
  }
}

/* HMAC-SHA-256 [HMAC]: H((K ^ opad) || H((K ^ ipad) || text)), the key padded
 * with zeros to the 64-octet block (keys longer than a block are hashed
 * first). */
void ov_hmac_sha256(const uint8_t *key, size_t klen, const uint8_t *msg, size_t len,
                    uint8_t out[32]) {
  uint8_t k0[64];
  memset(k0, 0, sizeof k0);
  if (klen > 64)
    ov_sha256(key, klen, k0);
  else
    memcpy(k0, key, klen);
  uint8_t *inner = (uint8_t *)malloc(64 + len);
  for (int i = 0; i < 64; ++i) inner[i] = k0[i] ^ 0x36;
  memcpy(inner + 64, msg, len);
  uint8_t ih[32];
  ov_sha256(inner, 64 + len, ih);
  free(inner);
  uint8_t outer[64 + 32];
  for (int i = 0; i < 64; ++i) outer[i] = k0[i] ^ 0x5c;
  memcpy(outer + 64, ih, 32);
  ov_sha256(outer, sizeof outer, out);
}

/* SDCP Sec. 6.4: the verifier's value for position i and purpose (0 =
 * acceptance test, 1 = additional token): HMAC-SHA-256 keyed with the seed
 * as eight octets in network byte order, over "SDCP-VERIFY-1" || 0x00 ||
 * session || uint32(round) || uint32(i) || uint8(purpose); the first 53 bits
 * of the result divided by 2^53. */
double ov_sdcp_uniform(uint64_t seed, const uint8_t session[16], uint32_t round, uint32_t i,
                       int purpose) {
  uint8_t key[8], msg[13 + 1 + 16 + 4 + 4 + 1];
  for (int j = 0; j < 8; ++j) key[j] = (uint8_t)(seed >> (56 - 8 * j));
  size_t n = 0;
  memcpy(msg + n, "SDCP-VERIFY-1", 13);
  n += 13;
  msg[n++] = 0x00;
  memcpy(msg + n, session, 16);
  n += 16;
  for (int j = 0; j < 4; ++j) msg[n++] = (uint8_t)(round >> (24 - 8 * j));
  for (int j = 0; j < 4; ++j) msg[n++] = (uint8_t)(i >> (24 - 8 * j));
  msg[n++] = (uint8_t)purpose;
  uint8_t mac[32];
  ov_hmac_sha256(key, sizeof key, msg, n, mac);
  uint64_t w = 0;
  for (int j = 0; j < 8; ++j) w = w << 8 | mac[j];
  return ldexp((double)(w >> 11), -53);
}

/* SDCP per-session inputs of the uniforms (the same 32-octet layout as the
 * library's record): session id, seed, round. */
typedef struct {
  uint8_t id[16];
  uint64_t seed;
  uint32_t round;
  uint32_t reserved;
} ov_sdcp_session;

/* Where a session's uniforms come from. */
typedef struct {
  uint64_t seed, session_key;  /* Philox */
  uint32_t round;
  const ov_sdcp_session *sdcp; /* non-NULL: SDCP Sec. 6.4 */
} ov_rng;

static double rng_uniform(const ov_rng *g, uint32_t i, int purpose) {
  if (g->sdcp) return ov_sdcp_uniform(g->sdcp->seed, g->sdcp->id, g->sdcp->round, i, purpose);
  return ov_uniform(g->seed, g->session_key, g->round, i, purpose);
}

/* ------------------------------------------------------------------------ */
/* Rows                                                                      */
/* ------------------------------------------------------------------------ */
static double widen_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static void load_row(const void *base, int dtype, int64_t row, int V, double *out) {
  if (dtype == OV_BF16) {
    const uint16_t *p = (const uint16_t *)base + row * (int64_t)V;
    for (int y = 0; y < V; ++y) out[y] = widen_bf16(p[y]);
  } else {
    const float *p = (const float *)base + row * (int64_t)V;
    for (int y = 0; y < V; ++y) out[y] = (double)p[y];
  }
}

/* 1 if the row holds a NaN or +inf, or no finite logit (the BAD_LOGITS reading). */
static int row_is_bad(const double *l, int V) {
  int finite = 0;
  for (int y = 0; y < V; ++y) {
    if (isnan(l[y]) || (isinf(l[y]) && l[y] > 0)) return 1;
    if (!isinf(l[y])) finite = 1;
  }
  return !finite;
}

/* Smallest token id attaining the largest logit (SDCP Sec. 4.1 / Sec. 6.4 Rule 1). */
static int row_argmax(const double *l, int V) {
  int g = 0;
  for (int y = 1; y < V; ++y)
    if (l[y] > l[g]) g = y;
  return g;
}

typedef struct {
  double logit;
  int id;
} ov_entry;

/* total order of the profile: logit descending, token id ascending */
static int entry_cmp(const void *a, const void *b) {
  const ov_entry *x = (const ov_entry *)a, *y = (const ov_entry *)b;
  if (x->logit > y->logit) return -1;
  if (x->logit < y->logit) return 1;
  return (x->id > y->id) - (x->id < y->id);
}

/*
 * SDCP Sec. 4.1: the distribution after temperature, top-k and top-p, in that
 * order.  Writes prob[0..V-1]; returns OV_OK or OV_S_BAD_LOGITS.
 * *delta_topp receives |1000*C - P*Z_k| / (1000*Z_k), the smallest over the
 * cutoff step and the step before it (INFINITY when top-p is off or T = 0).
 * ent: caller scratch of V entries.
 */
static int profile_row(const double *l, int V, const ov_sampling *s, double *prob,
                       double *delta_topp, ov_entry *ent) {
  *delta_topp = INFINITY;
  if (row_is_bad(l, V)) return OV_S_BAD_LOGITS;
  for (int y = 0; y < V; ++y) prob[y] = 0.0;

  if (s->temperature_milli == 0) { /* one-hot argmax */
    prob[row_argmax(l, V)] = 1.0;
    return OV_OK;
  }
  const double T = (double)s->temperature_milli / 1000.0;

  int n = 0; /* finite tokens only: a -inf logit has probability zero */
  for (int y = 0; y < V; ++y)
    if (!isinf(l[y])) { ent[n].logit = l[y]; ent[n].id = y; ++n; }
  qsort(ent, (size_t)n, sizeof *ent, entry_cmp);

  int kept = n; /* top-k: the first k tokens of the order */
  if (s->top_k > 0 && (int64_t)s->top_k < (int64_t)n) kept = (int)s->top_k;

  const double lmax = ent[0].logit;
  double Zk = 0.0;
  for (int j = 0; j < kept; ++j) Zk += exp((ent[j].logit - lmax) / T);

  int cut = kept; /* top-p: shortest prefix with 1000*C >= P*Z_k */
  double Zp = Zk;
  if (s->top_p_milli < 1000) {
    const double P = (double)s->top_p_milli;
    double C = 0.0, Cprev = 0.0;
    cut = 0;
    for (int j = 0; j < kept; ++j) {
      Cprev = C;
      C += exp((ent[j].logit - lmax) / T);
      if (1000.0 * C >= P * Zk) { cut = j + 1; break; }
    }
    if (cut == 0) { cut = kept; C = Zk; } /* unreachable: C reaches Z_k at the end */
    double d = fabs(1000.0 * C - P * Zk);
    if (cut > 1) {
      double d2 = fabs(1000.0 * Cprev - P * Zk);
      if (d2 < d) d = d2;
    }
    *delta_topp = d / (1000.0 * Zk);
    Zp = C;
  }
  for (int j = 0; j < cut; ++j) prob[ent[j].id] = exp((ent[j].logit - lmax) / T) / Zp;
  return OV_OK;
}

/*
 * Inverse CDF in ascending token-id order: the smallest y with
 * sum_{t<=y} w(t) > u * S, S = sum of all w.  If rounding leaves no such y,
 * the largest y with w(y) > 0.  *delta = distance of u*S to the nearest CDF
 * boundary around the pick, divided by S.
 */
static int inverse_cdf(const double *w, int V, double u, double *delta) {
  double S = 0.0;
  for (int y = 0; y < V; ++y) S += w[y];
  const double target = u * S;
  double C = 0.0;
  for (int y = 0; y < V; ++y) {
    double Cprev = C;
    C += w[y];
    if (C > target) {
      double d1 = target - Cprev, d2 = C - target;
      *delta = (d1 < d2 ? d1 : d2) / S;
      return y;
    }
  }
  *delta = 0.0;
  for (int y = V - 1; y >= 0; --y)
    if (w[y] > 0.0) return y;
  return -1;
}

/*
 * SDCP Sec. 6.4 Rule 2 / textbook "The acceptance rule": at the first
 * rejection the additional token is drawn from norm(max(0, p - q)) with the
 * purpose-1 uniform.  If rounding leaves that residual with no mass, draw
 * from p instead.  w: caller scratch of V doubles.
 */
static int residual_pick(const double *p, const double *q, int V, double u, double *w,
                         double *delta) {
  double S = 0.0;
  for (int y = 0; y < V; ++y) {
    double r = p[y] - q[y];
    w[y] = r > 0.0 ? r : 0.0;
    S += w[y];
  }
  if (S == 0.0) memcpy(w, p, sizeof(double) * (size_t)V);
  return inverse_cdf(w, V, u, delta);
}

/* ------------------------------------------------------------------------ */
/* Exported single-row helpers (for the oracle's own pins)                   */
/* ------------------------------------------------------------------------ */
int ov_profile_row(const void *row, int dtype, int V, const ov_sampling *s, double *prob,
                   double *delta_topp) {
  if (!row || !s || !prob || !delta_topp || V < 1 || (dtype != OV_BF16 && dtype != OV_FP32))
    return OV_ERR_ARG;
  double *l = (double *)malloc(sizeof(double) * (size_t)V);
  ov_entry *ent = (ov_entry *)malloc(sizeof(ov_entry) * (size_t)V);
  if (!l || !ent) { free(l); free(ent); return OV_ERR_NOMEM; }
  load_row(row, dtype, 0, V, l);
  int st = profile_row(l, V, s, prob, delta_topp, ent);
  free(l);
  free(ent);
  return st;
}

int ov_inverse_cdf(const double *w, int V, double u, double *delta) {
  if (!w || V < 1 || !delta) return OV_ERR_ARG;
  return inverse_cdf(w, V, u, delta);
}

int ov_residual_pick(const double *p, const double *q, int V, double u, double *delta) {
  if (!p || !q || V < 1 || !delta) return OV_ERR_ARG;
  double *w = (double *)malloc(sizeof(double) * (size_t)V);
  if (!w) return OV_ERR_NOMEM;
  int y = residual_pick(p, q, V, u, w, delta);
  free(w);
  return y;
}

/* ------------------------------------------------------------------------ */
/* The batched step                                                          */
/* ------------------------------------------------------------------------ */
typedef struct {
  double *l, *p, *q, *w;
  ov_entry *ent;
} ov_scratch;

static void set_if(double *arr, int64_t idx, double v) {
  if (arr) arr[idx] = v;
}

/*
 * One session.  Returns a = accepted count (>= 0) or a negative status; on
 * success writes out[0..a] (a accepted tokens, then the additional token).
 */
static int verify_session(int64_t b, const void *target, const void *draft, const float *qrows,
                          int dtype, const int32_t *x, int m, int rule, const ov_sampling *s,
                          int M, int V,
                          const ov_rng *g, int32_t *out, double *p_tok,
                          double *q_tok, double *d_acc, double *d_topp_t, double *d_topp_d,
                          double *d_cdf, ov_scratch *sc) {
  /* SDCP Sec. 6.2 / Table 2 "sdcp-limit": 1 <= M <= m_max (<= 64) */
  if (m < 1 || m > M) return OV_S_LIMIT;
  if ((rule != OV_RULE_GREEDY && rule != OV_RULE_SPECULATIVE && rule != OV_RULE_RELAXED) ||
      s->reserved != 0 ||
      s->top_p_milli > 1000)
    return OV_S_BAD_PROFILE;
  /* SDCP Sec. 6.3 step 5: no q rows for a rule that needs them */
  if (rule == OV_RULE_SPECULATIVE && draft == NULL && qrows == NULL) return OV_S_Q_UNAVAILABLE;
  for (int i = 0; i < m; ++i)
    if (x[i] < 0 || x[i] >= V) return OV_S_BAD_PROPOSAL;

  const int64_t trow0 = b * (int64_t)(M + 1); /* target row i (1-based) = trow0 + i - 1 */
  const int64_t drow0 = b * (int64_t)M;       /* draft row i (1-based)  = drow0 + i - 1 */

  /* every row the rule reads must be usable before any decision */
  for (int i = 1; i <= m + 1; ++i) {
    load_row(target, dtype, trow0 + i - 1, V, sc->l);
    if (row_is_bad(sc->l, V)) return OV_S_BAD_LOGITS;
  }
  if (rule == OV_RULE_SPECULATIVE && qrows == NULL)
    for (int i = 1; i <= m; ++i) {
      load_row(draft, dtype, drow0 + i - 1, V, sc->l);
      if (row_is_bad(sc->l, V)) return OV_S_BAD_LOGITS;
    }

  if (rule == OV_RULE_RELAXED) {
    /* Relaxed rule (textbook, "Speculative decoding": accept a token that is
     * in the target's top-k): x_i is accepted while p_i(x_i) > 0, i.e. while
     * the target's profile (temperature, top-k, top-p) could sample it; the
     * additional token is drawn from p_{a+1} with the purpose-1 value of
     * position a+1.  The probe holds p_i(x_i) at every position. */
    int a = -1;
    for (int i = 1; i <= m; ++i) {
      double dt;
      load_row(target, dtype, trow0 + i - 1, V, sc->l);
      profile_row(sc->l, V, s, sc->p, &dt, sc->ent);
      set_if(d_topp_t, b * (int64_t)(M + 1) + i - 1, dt);
      const double px = sc->p[x[i - 1]];
      set_if(p_tok, b * (int64_t)M + i - 1, px);
      if (a < 0 && !(px > 0.0)) a = i - 1;
      if (a < 0) out[i - 1] = x[i - 1];
      if (a >= 0 && !p_tok) break;
    }
    if (a < 0) a = m;
    double dt, dc;
    load_row(target, dtype, trow0 + a, V, sc->l);
    profile_row(sc->l, V, s, sc->p, &dt, sc->ent);
    set_if(d_topp_t, b * (int64_t)(M + 1) + a, dt);
    out[a] = inverse_cdf(sc->p, V, rng_uniform(g, (uint32_t)(a + 1), 1), &dc);
    set_if(d_cdf, b, dc);
    return a;
  }

  if (rule == OV_RULE_GREEDY) {
    /* SDCP Sec. 6.4 Rule 1: accept x_i while it equals argmax p_i (the argmax
     * of p_i is the argmax of the raw logits; ties to the smallest id); the
     * additional token is argmax p_{a+1}. */
    int a = 0;
    while (a < m) {
      load_row(target, dtype, trow0 + a, V, sc->l);
      if (x[a] != row_argmax(sc->l, V)) break;
      out[a] = x[a];
      ++a;
    }
    load_row(target, dtype, trow0 + a, V, sc->l);
    out[a] = row_argmax(sc->l, V);
    return a;
  }

  /* SDCP Sec. 6.3 step 5 and Sec. 6.4 Rule 2: q_i(x_i) != 0 for every i,
   * checked before any random value is drawn. */
  double qx[64];
  for (int i = 1; i <= m; ++i) {
    if (qrows) {
      /* SDCP Sec. 5.2: q_i is the published row itself (binary32) */
      qx[i - 1] = (double)qrows[(drow0 + i - 1) * (int64_t)V + x[i - 1]];
    } else {
      double dt;
      load_row(draft, dtype, drow0 + i - 1, V, sc->l);
      profile_row(sc->l, V, s, sc->q, &dt, sc->ent);
      set_if(d_topp_d, b * (int64_t)M + i - 1, dt);
      qx[i - 1] = sc->q[x[i - 1]];
    }
    set_if(q_tok, b * (int64_t)M + i - 1, qx[i - 1]);
  }
  /* a published q_i(x_i) must be a positive number: zero, negative, NaN or
   * infinite values are all unusable proposals */
  for (int i = 0; i < m; ++i)
    if (!(qx[i] > 0.0) || isinf(qx[i])) return OV_S_BAD_PROPOSAL;

  /* Rule 2, positions in order: accept x_i if u < min(1, p_i(x_i)/q_i(x_i)). */
  int a = m, decided = 0;
  for (int i = 1; i <= m; ++i) {
    if (decided && !p_tok) break; /* the rest only feeds the probe */
    double dt;
    load_row(target, dtype, trow0 + i - 1, V, sc->l);
    profile_row(sc->l, V, s, sc->p, &dt, sc->ent);
    set_if(d_topp_t, b * (int64_t)(M + 1) + i - 1, dt);
    const double px = sc->p[x[i - 1]];
    set_if(p_tok, b * (int64_t)M + i - 1, px);
    if (decided) continue;

    const double ratio = px / qx[i - 1];
    const double acc = ratio < 1.0 ? ratio : 1.0;
    const double u = rng_uniform(g, (uint32_t)i, 0);
    set_if(d_acc, b * (int64_t)M + i - 1, fabs(u - acc));
    if (u < acc) {
      out[i - 1] = x[i - 1];
      continue;
    }
    /* first rejection: additional token from norm(max(0, p_i - q_i)) */
    if (qrows) {
      /* the residual reads q_i(y) only where p_i(y) > 0 (elsewhere its weight
       * is zero for any probability q_i(y)); an entry read there must be a
       * finite non-negative number */
      const float *qr = qrows + (drow0 + i - 1) * (int64_t)V;
      for (int y = 0; y < V; ++y) {
        if (sc->p[y] > 0.0) {
          const double qy = (double)qr[y];
          if (!(qy >= 0.0) || isinf(qy)) return OV_S_BAD_PROPOSAL;
          sc->q[y] = qy;
        } else {
          sc->q[y] = 0.0;
        }
      }
    } else {
      load_row(draft, dtype, drow0 + i - 1, V, sc->l);
      profile_row(sc->l, V, s, sc->q, &dt, sc->ent);
    }
    double dc;
    out[i - 1] = residual_pick(sc->p, sc->q, V,
                               rng_uniform(g, (uint32_t)i, 1), sc->w, &dc);
    set_if(d_cdf, b, dc);
    a = i - 1;
    decided = 1;
  }
  if (!decided) {
    /* every proposal accepted: bonus token from p_{m+1} */
    double dt, dc;
    load_row(target, dtype, trow0 + m, V, sc->l);
    profile_row(sc->l, V, s, sc->p, &dt, sc->ent);
    set_if(d_topp_t, b * (int64_t)(M + 1) + m, dt);
    out[m] = inverse_cdf(sc->p, V, rng_uniform(g, (uint32_t)(m + 1), 1), &dc);
    set_if(d_cdf, b, dc);
  }
  return a;
}

/*
 * The same session with positions examined in order, each row read only when
 * its position is reached (textbook "The acceptance rule": the proposals are
 * checked one after another and the first rejection ends the round).  This
 * departs from verify_session, which follows SDCP Sec. 6.3 step 5 and checks
 * every row and every q_i(x_i) before any decision.
 * Position i reads target row i, and for rule 2 draft row i (or the published
 * q_i(x_i)); a bad row there fails the session with BAD_LOGITS, then an
 * unusable q_i(x_i) with BAD_PROPOSAL; then the position's test.  Rows after
 * the deciding position are never read, so a problem there changes nothing.
 * With every proposal accepted, row m+1 is read for the additional token.
 * The session checks that read no logits (limit, profile, q availability,
 * drafted tokens in range) come first, as in verify_session.  Where every
 * row is usable and every q_i(x_i) positive, the verdict is verify_session's.
 */
static int verify_session_early(int64_t b, const void *target, const void *draft,
                                const float *qrows, int dtype, const int32_t *x, int m, int rule,
                                const ov_sampling *s, int M, int V, const ov_rng *g, int32_t *out,
                                double *p_tok, double *q_tok, double *d_acc, double *d_topp_t,
                                double *d_topp_d, double *d_cdf, ov_scratch *sc) {
  if (m < 1 || m > M) return OV_S_LIMIT;
  if ((rule != OV_RULE_GREEDY && rule != OV_RULE_SPECULATIVE && rule != OV_RULE_RELAXED) ||
      s->reserved != 0 || s->top_p_milli > 1000)
    return OV_S_BAD_PROFILE;
  if (rule == OV_RULE_SPECULATIVE && draft == NULL && qrows == NULL) return OV_S_Q_UNAVAILABLE;
  for (int i = 0; i < m; ++i)
    if (x[i] < 0 || x[i] >= V) return OV_S_BAD_PROPOSAL;

  const int64_t trow0 = b * (int64_t)(M + 1);
  const int64_t drow0 = b * (int64_t)M;
  for (int i = 1; i <= m; ++i) {
    double dt;
    load_row(target, dtype, trow0 + i - 1, V, sc->l);
    if (row_is_bad(sc->l, V)) return OV_S_BAD_LOGITS;
    if (rule == OV_RULE_GREEDY) {
      /* Rule 1 at position i: the additional token at a mismatch is argmax p_i */
      const int y = row_argmax(sc->l, V);
      out[i - 1] = y;
      if (x[i - 1] != y) return i - 1;
      continue;
    }
    profile_row(sc->l, V, s, sc->p, &dt, sc->ent);
    set_if(d_topp_t, b * (int64_t)(M + 1) + i - 1, dt);
    const double px = sc->p[x[i - 1]];
    if (rule == OV_RULE_RELAXED) {
      set_if(p_tok, b * (int64_t)M + i - 1, px);
      if (px > 0.0) {
        out[i - 1] = x[i - 1];
        continue;
      }
      double dc;
      out[i - 1] = inverse_cdf(sc->p, V, rng_uniform(g, (uint32_t)i, 1), &dc);
      set_if(d_cdf, b, dc);
      return i - 1;
    }
    /* Rule 2 at position i: q_i(x_i), checked before the position's test */
    double qx;
    if (qrows) {
      qx = (double)qrows[(drow0 + i - 1) * (int64_t)V + x[i - 1]];
    } else {
      load_row(draft, dtype, drow0 + i - 1, V, sc->l);
      if (row_is_bad(sc->l, V)) return OV_S_BAD_LOGITS;
      profile_row(sc->l, V, s, sc->q, &dt, sc->ent);
      set_if(d_topp_d, b * (int64_t)M + i - 1, dt);
      qx = sc->q[x[i - 1]];
    }
    set_if(q_tok, b * (int64_t)M + i - 1, qx);
    set_if(p_tok, b * (int64_t)M + i - 1, px);
    if (!(qx > 0.0) || isinf(qx)) return OV_S_BAD_PROPOSAL;
    const double ratio = px / qx;
    const double acc = ratio < 1.0 ? ratio : 1.0;
    const double u = rng_uniform(g, (uint32_t)i, 0);
    set_if(d_acc, b * (int64_t)M + i - 1, fabs(u - acc));
    if (u < acc) {
      out[i - 1] = x[i - 1];
      continue;
    }
    if (qrows) {
      /* the published residual row, read where p_i > 0 (as in verify_session) */
      const float *qr = qrows + (drow0 + i - 1) * (int64_t)V;
      for (int y = 0; y < V; ++y) {
        if (sc->p[y] > 0.0) {
          const double qy = (double)qr[y];
          if (!(qy >= 0.0) || isinf(qy)) return OV_S_BAD_PROPOSAL;
          sc->q[y] = qy;
        } else {
          sc->q[y] = 0.0;
        }
      }
    }
    double dc;
    out[i - 1] = residual_pick(sc->p, sc->q, V, rng_uniform(g, (uint32_t)i, 1), sc->w, &dc);
    set_if(d_cdf, b, dc);
    return i - 1;
  }
  /* every proposal accepted: row m+1 gives the additional token */
  double dt, dc;
  load_row(target, dtype, trow0 + m, V, sc->l);
  if (row_is_bad(sc->l, V)) return OV_S_BAD_LOGITS;
  if (rule == OV_RULE_GREEDY) {
    out[m] = row_argmax(sc->l, V);
    return m;
  }
  profile_row(sc->l, V, s, sc->p, &dt, sc->ent);
  set_if(d_topp_t, b * (int64_t)(M + 1) + m, dt);
  out[m] = inverse_cdf(sc->p, V, rng_uniform(g, (uint32_t)(m + 1), 1), &dc);
  set_if(d_cdf, b, dc);
  return m;
}

/*
 * The batched step over B sessions (same layout as the GPU entry point):
 *   target   [B, M+1, V]  dtype (bf16 bits as uint16, or float32)
 *   draft    [B, M,   V]  dtype, or NULL
 *   tokens   [B, M]; m [B]; rule [B]; sampling [B]
 * Outputs: accepted_len[B] (a, or a negative status), out_tokens[B, M+1]
 * (a+1 tokens, then -1).  Optional (NULL to skip), all [B, M] unless noted,
 * -1 / +inf where not computed: p_tok, q_tok (rule 2 only), d_acc,
 * d_topp_t [B, M+1], d_topp_d, d_cdf [B].
 * Returns OV_OK or OV_ERR_*.
 */
static int verify_batch(const void *target, const void *draft, const float *qrows, int dtype,
              const int32_t *tokens,
              const int32_t *m, const int32_t *rule, const ov_sampling *sampling, int64_t B,
              int M, int V, uint64_t seed, uint32_t round, const ov_sdcp_session *sdcp,
              int early, int32_t *accepted_len,
              int32_t *out_tokens, double *p_tok, double *q_tok, double *d_acc,
              double *d_topp_t, double *d_topp_d, double *d_cdf) {
  if (!target || !tokens || !m || !rule || !sampling || !accepted_len || !out_tokens)
    return OV_ERR_ARG;
  if (B < 1 || M < 1 || M > 64 || V < 1 || (dtype != OV_BF16 && dtype != OV_FP32))
    return OV_ERR_ARG;

  ov_scratch sc;
  sc.l = (double *)malloc(sizeof(double) * (size_t)V);
  sc.p = (double *)malloc(sizeof(double) * (size_t)V);
  sc.q = (double *)malloc(sizeof(double) * (size_t)V);
  sc.w = (double *)malloc(sizeof(double) * (size_t)V);
  sc.ent = (ov_entry *)malloc(sizeof(ov_entry) * (size_t)V);
  if (!sc.l || !sc.p || !sc.q || !sc.w || !sc.ent) {
    free(sc.l); free(sc.p); free(sc.q); free(sc.w); free(sc.ent);
    return OV_ERR_NOMEM;
  }

  for (int64_t b = 0; b < B; ++b) {
    int32_t *out = out_tokens + b * (int64_t)(M + 1);
    for (int j = 0; j <= M; ++j) out[j] = -1;
    for (int j = 0; j < M; ++j) {
      set_if(p_tok, b * (int64_t)M + j, -1.0);
      set_if(q_tok, b * (int64_t)M + j, -1.0);
      set_if(d_acc, b * (int64_t)M + j, INFINITY);
      set_if(d_topp_d, b * (int64_t)M + j, INFINITY);
    }
    for (int j = 0; j <= M; ++j) set_if(d_topp_t, b * (int64_t)(M + 1) + j, INFINITY);
    set_if(d_cdf, b, INFINITY);

    const ov_rng g = {seed, sampling[b].session_key, round, sdcp ? &sdcp[b] : NULL};
    int a = (early ? verify_session_early : verify_session)(
        b, target, draft, qrows, dtype, tokens + b * (int64_t)M, m[b], rule[b], &sampling[b], M,
        V, &g, out, p_tok, q_tok, d_acc, d_topp_t, d_topp_d, d_cdf, &sc);
    accepted_len[b] = a;
    if (a < 0) { /* a failed session emits nothing; its diagnostics are kept */
      for (int j = 0; j <= M; ++j) out[j] = -1;
      for (int j = 0; j < M; ++j) {
        set_if(p_tok, b * (int64_t)M + j, -1.0);
        set_if(q_tok, b * (int64_t)M + j, -1.0);
      }
    }
  }
  free(sc.l); free(sc.p); free(sc.q); free(sc.w); free(sc.ent);
  return OV_OK;
}

int ov_verify(const void *target, const void *draft, int dtype, const int32_t *tokens,
              const int32_t *m, const int32_t *rule, const ov_sampling *sampling, int64_t B,
              int M, int V, uint64_t seed, uint32_t round, int32_t *accepted_len,
              int32_t *out_tokens, double *p_tok, double *q_tok, double *d_acc,
              double *d_topp_t, double *d_topp_d, double *d_cdf) {
  return verify_batch(target, draft, NULL, dtype, tokens, m, rule, sampling, B, M, V, seed, round,
                      NULL, 0, accepted_len, out_tokens, p_tok, q_tok, d_acc, d_topp_t, d_topp_d,
                      d_cdf);
}

/* The same batched step with the uniforms of SDCP Sec. 6.4 (HMAC-SHA-256);
 * sessions[B] give each session's id, seed and round. */
int ov_verify_sdcp(const void *target, const void *draft, int dtype, const int32_t *tokens,
                   const int32_t *m, const int32_t *rule, const ov_sampling *sampling,
                   const ov_sdcp_session *sessions, int64_t B, int M, int V,
                   int32_t *accepted_len, int32_t *out_tokens, double *p_tok, double *q_tok,
                   double *d_acc, double *d_topp_t, double *d_topp_d, double *d_cdf) {
  if (!sessions) return OV_ERR_ARG;
  return verify_batch(target, draft, NULL, dtype, tokens, m, rule, sampling, B, M, V, 0, 0,
                      sessions, 0, accepted_len, out_tokens, p_tok, q_tok, d_acc, d_topp_t, d_topp_d,
                      d_cdf);
}

/* The batched step with the draft distributions given as SDCP q_rows (Sec.
 * 5.2): qrows [B, M, V] binary32 probabilities, row i of session b at
 * qrows[b, i-1, :], used as published (no profile, no renormalisation).
 * sessions: SDCP values per session, or NULL for Philox from (seed, round). */
int ov_verify_qrows(const void *target, int dtype, const float *qrows, const int32_t *tokens,
                    const int32_t *m, const int32_t *rule, const ov_sampling *sampling,
                    const ov_sdcp_session *sessions, int64_t B, int M, int V, uint64_t seed,
                    uint32_t round, int32_t *accepted_len, int32_t *out_tokens, double *p_tok,
                    double *q_tok, double *d_acc, double *d_topp_t, double *d_cdf) {
  return verify_batch(target, NULL, qrows, dtype, tokens, m, rule, sampling, B, M, V, seed, round,
                      sessions, 0, accepted_len, out_tokens, p_tok, q_tok, d_acc, d_topp_t, NULL,
                      d_cdf);
}

/* The batched step with positions examined in order and each row read only
 * when its position is reached (verify_session_early).  Draft distributions
 * from draft logits (draft) or published q_rows (qrows), at most one of them;
 * uniforms from SDCP Sec. 6.4 records (sessions) or Philox (seed, round). */
int ov_verify_early(const void *target, const void *draft, const float *qrows, int dtype,
                    const int32_t *tokens, const int32_t *m, const int32_t *rule,
                    const ov_sampling *sampling, const ov_sdcp_session *sessions, int64_t B,
                    int M, int V, uint64_t seed, uint32_t round, int32_t *accepted_len,
                    int32_t *out_tokens, double *p_tok, double *q_tok, double *d_acc,
                    double *d_topp_t, double *d_topp_d, double *d_cdf) {
  if (draft && qrows) return OV_ERR_ARG;
  return verify_batch(target, draft, qrows, dtype, tokens, m, rule, sampling, B, M, V, seed,
                      round, sessions, 1, accepted_len, out_tokens, p_tok, q_tok, d_acc, d_topp_t,
                      d_topp_d, d_cdf);
}

/* ------------------------------------------------------------------------ */
/* The verifier's commit step around the acceptance step [SDCP Sec. 4.2,    */
/* 6.3 steps 6-8, 6.5]: truncation, the committed-prefix digest chain, the  */
/* low-round counters with the fallback ladder, and m_cap.                   */
/* ------------------------------------------------------------------------ */
enum { OV_ACT_CONTINUE = 0, OV_ACT_REDUCE = 1, OV_ACT_SWITCH = 2, OV_ACT_SELF_DECODE = 3,
       OV_ACT_FINISH = 4, OV_ACT_FAIL = 5 };

/* The contract members the commit step reads [SDCP Sec. 4.1] (the same
 * 64-octet layout as the library's record). */
typedef struct {
  uint32_t m_max, max_new, low_rounds, low_ratio; /* low_ratio 0 = absent */
  uint32_t n_stop;
  int32_t stop[8];
  uint32_t n_fallback;
  uint8_t fallback[8];
} ov_contract;

/* Per-session verifier state (the same 64-octet layout as the library's). */
typedef struct {
  uint8_t digest[32]; /* d[n] */
  uint32_t n;         /* committed output tokens */
  uint32_t m_cap;
  uint32_t c, g, j;   /* Sec. 6.5.2 counters */
  uint32_t reserved[3];
} ov_state;

/* [SDCP Sec. 4.2] d[0] over the domain separator, the contract digest, the
 * prompt length and the prompt tokens (each uint32, network byte order). */
void ov_prefix_digest(const uint8_t contract_digest[32], const int32_t *prompt, uint32_t P,
                      uint8_t out[32]) {
  const size_t len = 14 + 32 + 4 + 4 * (size_t)P;
  uint8_t *msg = (uint8_t *)malloc(len);
  memcpy(msg, "SDCP-PREFIX-1", 13);
  msg[13] = 0x00;
  memcpy(msg + 14, contract_digest, 32);
  size_t n = 46;
  for (int k = 0; k < 4; ++k) msg[n++] = (uint8_t)(P >> (24 - 8 * k));
  for (uint32_t t = 0; t < P; ++t)
    for (int k = 0; k < 4; ++k) msg[n++] = (uint8_t)((uint32_t)prompt[t] >> (24 - 8 * k));
  ov_sha256(msg, len, out);
  free(msg);
}

/* [SDCP Sec. 4.1] contract_digest over the domain separator and the contract's
 * deterministic CBOR encoding (given). */
void ov_contract_digest(const uint8_t *cbor, size_t len, uint8_t out[32]) {
  uint8_t *msg = (uint8_t *)malloc(16 + len);
  memcpy(msg, "SDCP-CONTRACT-1", 15);
  msg[15] = 0x00;
  memcpy(msg + 16, cbor, len);
  ov_sha256(msg, 16 + len, out);
  free(msg);
}

/*
 * One round's commit for B sessions, after the acceptance step:
 *   accepted_len [B]  a in [0, M], else (a negative status, or out of range)
 *                     the session commits nothing, its state is left as it is
 *                     and its action is -1;
 *   out_tokens [B, M+1]  the a+1 emitted tokens, then -1; truncated in place
 *                     after the first stop token and at max_new [Sec. 6.3
 *                     step 6]: entries past the committed ones become -1;
 *   m [B]             the proposal lengths;
 *   self_decode_ok [B] 1 where self_decode is permitted this round (the
 *                     contract has self_load and the load does not exceed it),
 *                     or NULL (never permitted).
 * Outputs: emitted_len [B] tokens committed; action [B]; state updated.
 * Per session, in the order of the text:
 *   commit [Sec. 6.3 step 7]: n += e; d[n+k] = SHA-256(d[n+k-1] || uint32(o_k));
 *   low round [Sec. 6.5.2]: 100*a < low_ratio*m, or a == 0 when low_ratio is 0;
 *   counters: low -> c += 1, g = 0; else c = 0, g += 1 and, when g reaches R,
 *     j = 0; when c reaches R the entry j of the fallback list is applied,
 *     self_decode skipped where not permitted, j advanced past every entry
 *     applied or skipped, then c = 0; no entry left -> fail; otherwise
 *     continue;
 *   m_cap [Sec. 6.5.1, 6.5.2]: reduce halves it (at least 1); after a round
 *     that is not low it is restored by one, up to m_max (the text's example
 *     of a gradual restore);
 *   finish [Sec. 6.5.2]: when a stop token was committed or n reached
 *     max_new, the action is finish.
 */
int ov_commit(const ov_contract *contract, ov_state *state, const int32_t *m,
              const int32_t *accepted_len, int32_t *out_tokens, const uint8_t *self_decode_ok,
              int64_t B, int M, int32_t *emitted_len, int32_t *action) {
  if (!contract || !state || !m || !accepted_len || !out_tokens || !emitted_len || !action ||
      B < 1 || M < 1 || M > 64)
    return OV_ERR_ARG;
  for (int64_t b = 0; b < B; ++b) {
    const ov_contract *k = &contract[b];
    ov_state *s = &state[b];
    int32_t *out = out_tokens + b * (int64_t)(M + 1);
    const int32_t a = accepted_len[b];
    if (a < 0 || a > M) {
      emitted_len[b] = 0;
      action[b] = -1;
      continue;
    }
    /* truncation: after the first stop token, and at max_new */
    int e = a + 1, finished = 0;
    for (int t = 0; t < e; ++t) {
      int is_stop = 0;
      for (uint32_t q = 0; q < k->n_stop && q < 8; ++q)
        if (out[t] == k->stop[q]) is_stop = 1;
      if (is_stop) {
        e = t + 1;
        finished = 1;
        break;
      }
    }
    const uint32_t room = s->n >= k->max_new ? 0u : k->max_new - s->n;
    if ((uint32_t)e >= room) {
      e = (int)room;
      finished = 1;
    }
    for (int t = e; t <= M; ++t) out[t] = -1;
    /* commit: extend the digest chain by every committed token */
    for (int t = 0; t < e; ++t) {
      uint8_t msg[36];
      memcpy(msg, s->digest, 32);
      for (int q = 0; q < 4; ++q) msg[32 + q] = (uint8_t)((uint32_t)out[t] >> (24 - 8 * q));
      ov_sha256(msg, 36, s->digest);
    }
    s->n += (uint32_t)e;
    /* control */
    const int low = k->low_ratio > 0 ? (100LL * a < (long long)k->low_ratio * m[b]) : (a == 0);
    int act = OV_ACT_CONTINUE;
    if (low) {
      s->c += 1;
      s->g = 0;
    } else {
      s->c = 0;
      s->g += 1;
      if (s->g == k->low_rounds) s->j = 0;
    }
    if (s->c == k->low_rounds) {
      int applied = 0;
      while (s->j < k->n_fallback && s->j < 8) {
        const int entry = k->fallback[s->j];
        s->j += 1;
        if (entry == OV_ACT_SELF_DECODE && !(self_decode_ok && self_decode_ok[b])) continue;
        act = entry;
        applied = 1;
        break;
      }
      if (!applied) act = OV_ACT_FAIL;
      s->c = 0;
    }
    if (act == OV_ACT_REDUCE) s->m_cap = s->m_cap / 2 > 1 ? s->m_cap / 2 : 1;
    if (!low && s->m_cap < k->m_max) s->m_cap += 1;
    if (finished) act = OV_ACT_FINISH;
    emitted_len[b] = e;
    action[b] = act;
  }
  return OV_OK;
}
