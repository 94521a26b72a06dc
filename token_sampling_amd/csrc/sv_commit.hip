// sv_commit.hip -- the verifier's commit step after the acceptance step, per
// the SDCP Internet-Draft ("Speculative Decoding Coordination Protocol (SDCP)
// for Distributed Inference with Multi-Level Caches"):
//   Sec. 6.3 step 6  truncate the emitted tokens after the first stop token
//                    and at max_new;
//   Sec. 6.3 step 7  commit: n and the prefix digest d[n] (Sec. 4.2), one
//                    SHA-256 link per committed token;
//   Sec. 6.5         control: low rounds, the counters c, g, j, the fallback
//                    ladder, m_cap.
// One lane per session; each lane's digest chain is one compression per
// committed token, or, after sv_verify_commit, at most one: the links over
// the drafted tokens were computed beside the row stream (sv_commit.hpp).
// Host functions give d[0] and the contract digest.
#include <string.h>

#include "sv_commit.hpp"
#include "sv_kernels.hpp"

namespace sv {

namespace {

__global__ __launch_bounds__(kWave) void k_commit(const sv_contract* __restrict__ contracts,
                                                  sv_session_state* __restrict__ states,
                                                  const int32_t* __restrict__ m,
                                                  const int32_t* __restrict__ accepted_len,
                                                  int32_t* __restrict__ out_tokens,
                                                  const uint8_t* __restrict__ self_decode_ok, int B,
                                                  int M, int32_t* __restrict__ emitted_len,
                                                  int32_t* __restrict__ action,
                                                  const uint32_t* __restrict__ chain) {
  const int b = (int)(blockIdx.x * kWave + threadIdx.x);
  if (b >= B) return;
  const int32_t a = accepted_len[b];
  if (a < 0 || a > M) {  // no verdict: nothing is committed
    emitted_len[b] = 0;
    action[b] = -1;
    return;
  }
  // the contract's members are read where they are used (a local copy of the
  // record with its two small arrays would be placed in LDS)
  const sv_contract& k = contracts[b];
  sv_session_state* st = states + b;
  uint32_t n = st->n, m_cap = st->m_cap, c = st->c, g = st->g, j = st->j;
  // the digest as eight big-endian words (the record is 4-byte aligned)
  uint32_t* dg = (uint32_t*)st->digest;
  int32_t* out = out_tokens + (size_t)b * (M + 1);

  // truncation: after the first stop token, and at max_new
  int e = a + 1;
  bool finished = false;
  const uint32_t nstop = k.n_stop < SV_STOP_MAX ? k.n_stop : SV_STOP_MAX;
  for (int t = 0; t < e; ++t) {
    if (commit::is_stop(k, nstop, out[t])) {
      e = t + 1;
      finished = true;
      break;
    }
  }
  const uint32_t room = n >= k.max_new ? 0u : k.max_new - n;
  if ((uint32_t)e >= room) {
    e = (int)room;
    finished = true;
  }

  // commit: d[n+t+1] = SHA-256(d[n+t] || uint32(o_t)), one 36-octet block each.
  // With the drafted tokens' links given, d[n+t0] for t0 = min(e, a) is
  // chain[b][t0-1] (the first a committed tokens are the accepted drafts, and
  // t0 never exceeds the links chained: e <= a stops at max_new and at the
  // first stop token, and e = a+1 means no stop among x_1..x_a and a < room);
  // only the additional token, if committed, is linked here.
  uint32_t h[8];
  int t0 = 0;
  if (chain != nullptr) t0 = e < a ? e : a;
  if (t0 > 0) {
    const uint4* c = (const uint4*)(chain + ((size_t)b * M + (t0 - 1)) * 8);
    const uint4 lo = c[0], hi = c[1];
    h[0] = lo.x, h[1] = lo.y, h[2] = lo.z, h[3] = lo.w;
    h[4] = hi.x, h[5] = hi.y, h[6] = hi.z, h[7] = hi.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = __builtin_bswap32(dg[i]);
  }
  for (int t = t0; t < e; ++t) commit::link(h, out[t]);
#pragma unroll
  for (int i = 0; i < 8; ++i) dg[i] = __builtin_bswap32(h[i]);
  for (int t = e; t <= M; ++t) out[t] = -1;
  n += (uint32_t)e;

  // control (Sec. 6.5.2): low round, counters, the fallback ladder
  const bool low = k.low_ratio > 0 ? (100ll * a < (long long)k.low_ratio * m[b]) : (a == 0);
  int32_t act = SV_ACT_CONTINUE;
  if (low) {
    c += 1;
    g = 0;
  } else {
    c = 0;
    g += 1;
    if (g == k.low_rounds) j = 0;
  }
  if (c == k.low_rounds) {
    // the permission is read before the walk: with that load inside the loop
    // (under the self_decode test) this compiler returned the previous action
    // instead of the applied self_decode entry
    const bool self_ok = self_decode_ok != nullptr && self_decode_ok[b] != 0;
    const uint32_t nfb = k.n_fallback < SV_FALLBACK_MAX ? k.n_fallback : SV_FALLBACK_MAX;
    int32_t applied = SV_ACT_FAIL;  // no entry left
    while (j < nfb) {
      const int32_t entry = k.fallback[j];
      j += 1;
      if (entry != SV_ACT_SELF_DECODE || self_ok) {
        applied = entry;
        break;
      }
    }
    act = applied;
    c = 0;
  }
  // m_cap (Sec. 6.5.1): halved by reduce, restored by one after a round that
  // is not low, up to m_max
  if (act == SV_ACT_REDUCE) m_cap = m_cap / 2 > 1 ? m_cap / 2 : 1;
  if (!low && m_cap < k.m_max) m_cap += 1;
  if (finished) act = SV_ACT_FINISH;

  st->n = n;
  st->m_cap = m_cap;
  st->c = c;
  st->g = g;
  st->j = j;
  emitted_len[b] = e;
  action[b] = act;
}

}  // namespace

void launch_commit(const sv_contract* contracts, sv_session_state* states, const int32_t* m,
                   const int32_t* accepted_len, int32_t* out_tokens, const uint8_t* self_decode_ok,
                   int B, int M, int32_t* emitted_len, int32_t* action, const uint32_t* chain,
                   hipStream_t st) {
  const unsigned grid = (unsigned)((B + kWave - 1) / kWave);
  hipLaunchKernelGGL(k_commit, dim3(grid), dim3(kWave), 0, st, contracts, states, m, accepted_len,
                     out_tokens, self_decode_ok, B, M, emitted_len, action, chain);
}

}  // namespace sv

extern "C" int sv_commit(const sv_contract* contracts, sv_session_state* states, const int32_t* m,
                         const int32_t* accepted_len, int32_t* out_tokens,
                         const uint8_t* self_decode_ok, int32_t B, int32_t M,
                         int32_t* emitted_len, int32_t* action, void* stream) {
  if (!contracts || !states || !m || !accepted_len || !out_tokens || !emitted_len || !action)
    return SV_ERR_ARG;
  if (B < 1 || B > SV_B_MAX || M < 1 || M > SV_M_MAX) return SV_ERR_ARG;
  (void)hipGetLastError();
  sv::launch_commit(contracts, states, m, accepted_len, out_tokens, self_decode_ok, B, M,
                    emitted_len, action, nullptr, (hipStream_t)stream);
  if (hipGetLastError() != hipSuccess) return SV_ERR_DEVICE;
  return SV_OK;
}

extern "C" int sv_prefix_digest(const uint8_t* contract_digest, const int32_t* prompt,
                                uint32_t P, uint8_t* out) {
  if (!contract_digest || !out || (P > 0 && !prompt)) return SV_ERR_ARG;
  if (P > (1u << 28)) return SV_ERR_ARG;
  const size_t len = 14 + 32 + 4 + 4 * (size_t)P;
  uint8_t* msg = (uint8_t*)malloc(len);
  if (!msg) return SV_ERR_ARG;
  memcpy(msg, "SDCP-PREFIX-1", 13);
  msg[13] = 0x00;
  memcpy(msg + 14, contract_digest, 32);
  size_t n = 46;
  for (int i = 0; i < 4; ++i) msg[n++] = (uint8_t)(P >> (24 - 8 * i));
  for (uint32_t t = 0; t < P; ++t)
    for (int i = 0; i < 4; ++i) msg[n++] = (uint8_t)((uint32_t)prompt[t] >> (24 - 8 * i));
  sv::sdcp::sha256_host(msg, len, out);
  free(msg);
  return SV_OK;
}

extern "C" int sv_contract_digest(const uint8_t* cbor, size_t len, uint8_t* out) {
  if ((!cbor && len > 0) || !out) return SV_ERR_ARG;
  if (len > ((size_t)1 << 30)) return SV_ERR_ARG;
  uint8_t* msg = (uint8_t*)malloc(16 + len);
  if (!msg) return SV_ERR_ARG;
  memcpy(msg, "SDCP-CONTRACT-1", 15);
  msg[15] = 0x00;
  if (len) memcpy(msg + 16, cbor, len);
  sv::sdcp::sha256_host(msg, 16 + len, out);
  free(msg);
  return SV_OK;
}
