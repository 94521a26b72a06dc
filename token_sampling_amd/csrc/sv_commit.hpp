// sv_commit.hpp -- the committed-prefix digest chain of the SDCP Internet-Draft
// ("Speculative Decoding Coordination Protocol (SDCP) for Distributed Inference
// with Multi-Level Caches"), Sec. 4.2: d[n+1] = SHA-256(d[n] || uint32(o)),
// the token in network byte order.  The 36-octet message and its padding are
// one block, so a link is one compression from the initial state.
//
// The links over a session's drafted tokens depend on nothing the acceptance
// step decides: the tokens it commits are a prefix of x_1..x_m, plus possibly
// the additional token.  chain_drafted computes them beside the row stream
// (one lane per session), so that the commit after the verdict needs at most
// one compression.
#pragma once

#include "sv_common.hpp"
#include "sv_sdcp.hpp"

namespace sv {
namespace commit {

// h = the state words of d (d as big-endian words); h becomes those of the
// next digest d' = SHA-256(d || uint32(o)).
__device__ inline void link(uint32_t h[8], int32_t o) {
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = h[i];
  w[8] = (uint32_t)o;
  w[9] = 0x80000000u;
#pragma unroll
  for (int i = 10; i < 15; ++i) w[i] = 0;
  w[15] = 36 * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = sdcp::kH0[i];
  sdcp::compress(h, w);
}

__device__ inline bool is_stop(const sv_contract& k, uint32_t nstop, int32_t o) {
  bool stop = false;
  for (uint32_t q = 0; q < nstop; ++q) stop |= o == k.stop[q];
  return stop;
}

// Links a session can commit from its drafted tokens: at most m, at most the
// room left before max_new, and none past the first drafted stop token.
__device__ inline int drafted_links(const sv_contract& k, uint32_t n, int mb,
                                   const int32_t* __restrict__ x) {
  const uint32_t room = n >= k.max_new ? 0u : k.max_new - n;
  int L = (uint32_t)mb < room ? mb : (int)room;
  const uint32_t nstop = k.n_stop < SV_STOP_MAX ? k.n_stop : SV_STOP_MAX;
  for (int t = 0; t < L; ++t)
    if (is_stop(k, nstop, x[t])) {
      L = t + 1;
      break;
    }
  return L;
}

// Session b's digests after its first 1..L drafted tokens, L = drafted_links,
// into chain[b][0..L-1] (eight state words each); nothing for a session whose
// m is out of range (it fails with a limit status and commits nothing).
__device__ inline void chain_drafted(int64_t b, const sv_contract* __restrict__ contracts,
                                     const sv_session_state* __restrict__ states,
                                     const int32_t* __restrict__ tokens,
                                     const int32_t* __restrict__ m, int B, int M,
                                     uint32_t* __restrict__ chain) {
  if (b >= B) return;
  const int mb = m[b];
  if (mb < 1 || mb > M) return;
  const sv_contract& k = contracts[b];
  const sv_session_state* st = states + b;
  const int32_t* x = tokens + (size_t)b * M;
  const int L = drafted_links(k, st->n, mb, x);
  const uint32_t* dg = (const uint32_t*)st->digest;
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = __builtin_bswap32(dg[i]);
  uint4* out = (uint4*)(chain + (size_t)b * M * 8);
  for (int t = 0; t < L; ++t) {
    link(h, x[t]);
    out[2 * t] = make_uint4(h[0], h[1], h[2], h[3]);
    out[2 * t + 1] = make_uint4(h[4], h[5], h[6], h[7]);
  }
}

}  // namespace commit
}  // namespace sv
