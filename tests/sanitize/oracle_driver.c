/*
 * A driver for the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_sanitizers.py with gcc -fsanitize=address,undefined):
 * every exported entry point on small seeded inputs, bf16 and binary32,
 * every rule and status, masks, NaN and infinities, in-order reading, q rows,
 * SDCP values, the commit step and the digests.  Exits 0 when every call
 * returns; a sanitizer report makes it exit non-zero.
 */
#include <stdio.h>

#include "../../oracle/sv_oracle.c"

static uint64_t rng_state = 0x9E3779B97F4A7C15ULL;
static uint64_t next_u64(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}
static double next_unit(void) { return (double)(next_u64() >> 11) * 0x1p-53; }
static float next_normal(void) {
  double u1 = next_unit(), u2 = next_unit();
  if (u1 < 1e-300) u1 = 1e-300;
  return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static int run_case(int B, int M, int V, int dtype, int with_draft) {
  const size_t tn = (size_t)B * (M + 1) * V, dn = (size_t)B * M * V;
  float *t32 = malloc(tn * sizeof(float)), *d32 = malloc(dn * sizeof(float));
  uint16_t *t16 = malloc(tn * sizeof(uint16_t)), *d16 = malloc(dn * sizeof(uint16_t));
  float *qrows = malloc(dn * sizeof(float));
  int32_t *tok = malloc((size_t)B * M * sizeof(int32_t)), *m = malloc(B * sizeof(int32_t));
  int32_t *rule = malloc(B * sizeof(int32_t)), *acc = malloc(B * sizeof(int32_t));
  int32_t *out = malloc((size_t)B * (M + 1) * sizeof(int32_t));
  double *pt = malloc((size_t)B * M * sizeof(double)), *qt = malloc((size_t)B * M * sizeof(double));
  double *da = malloc((size_t)B * M * sizeof(double)), *dt = malloc((size_t)B * (M + 1) * sizeof(double));
  double *dd = malloc((size_t)B * M * sizeof(double)), *dc = malloc(B * sizeof(double));
  ov_sampling *s = calloc((size_t)B, sizeof(ov_sampling));
  ov_sdcp_session *sess = calloc((size_t)B, sizeof(ov_sdcp_session));
  for (size_t j = 0; j < tn; ++j) t32[j] = 2.0f * next_normal();
  for (size_t j = 0; j < dn; ++j) d32[j] = t32[j] + next_normal();
  for (size_t j = 0; j < dn; ++j) qrows[j] = (float)next_unit();
  static const uint32_t prof[8][3] = {{1000, 0, 1000}, {700, 50, 900}, {800, 0, 950}, {0, 0, 1000},
                                      {1300, 7, 1000}, {500, 0, 0}, {1000, 1, 1000}, {2000, 3, 300}};
  for (int b = 0; b < B; ++b) {
    s[b].temperature_milli = prof[b % 8][0];
    s[b].top_k = prof[b % 8][1];
    s[b].top_p_milli = prof[b % 8][2];
    s[b].session_key = (uint64_t)b;
    sess[b].seed = next_u64();
    sess[b].round = (uint32_t)next_u64();
    for (int j = 0; j < 16; ++j) sess[b].id[j] = (uint8_t)next_u64();
    m[b] = 1 + (int)(next_u64() % (uint64_t)M);
    rule[b] = (b % 5 == 0) ? 1 : (b % 7 == 3 ? 192 : 2);
    for (int i = 0; i < M; ++i) tok[(size_t)b * M + i] = (int32_t)(next_u64() % (uint64_t)V);
  }
  /* edge cases: -inf masks, NaN, +inf, out-of-range token, bad m, bad profile */
  if (B > 6) {
    for (int y = 0; y < V; y += 2) t32[((size_t)1 * (M + 1)) * V + y] = -INFINITY;
    t32[((size_t)2 * (M + 1)) * V + 1] = NAN;
    d32[((size_t)3 * M) * V + 2] = INFINITY;
    tok[(size_t)4 * M] = V;
    m[5] = 0;
    s[6].top_p_milli = 1001;
  }
  for (size_t j = 0; j < tn; ++j) t16[j] = to_bf16(t32[j]);
  for (size_t j = 0; j < dn; ++j) d16[j] = to_bf16(d32[j]);
  const void *T = dtype == OV_BF16 ? (const void *)t16 : (const void *)t32;
  const void *D = !with_draft ? NULL : (dtype == OV_BF16 ? (const void *)d16 : (const void *)d32);
  int rc = 0;
  rc |= ov_verify(T, D, dtype, tok, m, rule, s, B, M, V, 7, 3, acc, out, pt, qt, da, dt, dd, dc);
  rc |= ov_verify(T, D, dtype, tok, m, rule, s, B, M, V, 7, 3, acc, out, NULL, NULL, NULL, NULL,
                  NULL, NULL);
  rc |= ov_verify_sdcp(T, D, dtype, tok, m, rule, s, sess, B, M, V, acc, out, pt, qt, da, dt, dd,
                       dc);
  rc |= ov_verify_qrows(T, dtype, qrows, tok, m, rule, s, NULL, B, M, V, 7, 3, acc, out, pt, qt,
                        da, dt, dc);
  rc |= ov_verify_early(T, D, NULL, dtype, tok, m, rule, s, NULL, B, M, V, 7, 3, acc, out, pt, qt,
                        da, dt, dd, dc);
  rc |= ov_verify_early(T, NULL, qrows, dtype, tok, m, rule, s, sess, B, M, V, 7, 3, acc, out, pt,
                        qt, da, dt, dd, dc);
  /* the commit step on the last verdicts */
  ov_contract *c = calloc((size_t)B, sizeof(ov_contract));
  ov_state *st = calloc((size_t)B, sizeof(ov_state));
  int32_t *em = malloc(B * sizeof(int32_t)), *act = malloc(B * sizeof(int32_t));
  uint8_t *ok = malloc((size_t)B);
  for (int b = 0; b < B; ++b) {
    c[b].m_max = (uint32_t)M;
    c[b].max_new = 5;
    c[b].low_rounds = 2;
    c[b].low_ratio = (uint32_t)(b % 3) * 30;
    c[b].n_stop = (uint32_t)(b % 10);
    for (int j = 0; j < 8; ++j) c[b].stop[j] = j;
    c[b].n_fallback = (uint32_t)(b % 9);
    for (int j = 0; j < 8; ++j) c[b].fallback[j] = (uint8_t)(1 + j % 4);
    st[b].m_cap = (uint32_t)M;
    ok[b] = (uint8_t)(b & 1);
  }
  for (int r = 0; r < 4; ++r)
    rc |= ov_commit(c, st, m, acc, out, ok, B, M, em, act);
  free(c); free(st); free(em); free(act); free(ok);
  free(t32); free(d32); free(t16); free(d16); free(qrows); free(tok); free(m); free(rule);
  free(acc); free(out); free(pt); free(qt); free(da); free(dt); free(dd); free(dc); free(s);
  free(sess);
  return rc;
}

int main(void) {
  int rc = 0;
  rc |= run_case(12, 4, 300, OV_BF16, 1);
  rc |= run_case(12, 4, 300, OV_FP32, 1);
  rc |= run_case(9, 64, 17, OV_BF16, 1);
  rc |= run_case(8, 3, 1, OV_FP32, 1);
  rc |= run_case(10, 2, 50, OV_BF16, 0);
  /* digests and single-row helpers */
  uint8_t h[32], cd[32];
  const uint8_t msg[] = "abc";
  ov_sha256(msg, 3, h);
  ov_hmac_sha256(msg, 3, msg, 3, h);
  ov_contract_digest(msg, 3, cd);
  int32_t prompt[5] = {1, 2, 3, 4, 5};
  ov_prefix_digest(cd, prompt, 5, h);
  double w[6] = {0.1, 0.0, 0.5, 0.2, 0.0, 0.2}, p[6] = {0.2, 0.2, 0.2, 0.2, 0.1, 0.1}, d;
  (void)ov_inverse_cdf(w, 6, 0.7, &d);
  (void)ov_residual_pick(p, w, 6, 0.3, &d);
  (void)ov_sdcp_uniform(5, h, 1, 2, 1);
  (void)ov_uniform(1, 2, 3, 4, 0);
  printf("oracle driver done rc=%d\n", rc);
  return rc != 0;
}
