// sv_sdcp.hpp -- the verifier values of the SDCP Internet-Draft ("Speculative
// Decoding Coordination Protocol (SDCP) for Distributed Inference with
// Multi-Level Caches"), Sec. 6.4, on the GPU: one value per lane.
//
// The value for position i and purpose (0 = acceptance test, 1 = additional
// token) is HMAC-SHA-256 (RFC 2104) keyed with the session's seed as eight
// octets in network byte order, over the message
//   "SDCP-VERIFY-1" || 0x00 || session id (16 octets) || uint32(round) ||
//   uint32(i) || uint8(purpose)                         (39 octets)
// and the verifier uses the first 53 bits of the MAC, most significant first,
// divided by 2^53.
//
// SHA-256 is FIPS 180-4 Sec. 6.2.  The key (8 octets) fits one block, and so
// do the 39-octet message and the 32-octet inner digest with their padding,
// so one value costs four compression calls: key xor ipad, message, key xor
// opad, inner digest.  The message words are assembled directly in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {
namespace sdcp {

// FIPS 180-4 Sec. 4.2.2: the first 32 bits of the fractional parts of the cube
// roots of the first 64 primes (one literal table for the device copy in
// constant memory and the host copy).
#define SV_SHA256_K                                                                           \
  0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu, 0x59f111f1u, 0x923f82a4u,   \
      0xab1c5ed5u, 0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u, 0x72be5d74u,           \
      0x80deb1feu, 0x9bdc06a7u, 0xc19bf174u, 0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u,           \
      0x240ca1ccu, 0x2de92c6fu, 0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau, 0x983e5152u,           \
      0xa831c66du, 0xb00327c8u, 0xbf597fc7u, 0xc6e00bf3u, 0xd5a79147u, 0x06ca6351u,           \
      0x14292967u, 0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu, 0x53380d13u, 0x650a7354u,           \
      0x766a0abbu, 0x81c2c92eu, 0x92722c85u, 0xa2bfe8a1u, 0xa81a664bu, 0xc24b8b70u,           \
      0xc76c51a3u, 0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u, 0x19a4c116u,           \
      0x1e376c08u, 0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu,           \
      0x682e6ff3u, 0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u, 0x90befffau,           \
      0xa4506cebu, 0xbef9a3f7u, 0xc67178f2u
__constant__ const uint32_t kK[64] = {SV_SHA256_K};
static const uint32_t kKHost[64] = {SV_SHA256_K};

// FIPS 180-4 Sec. 5.3.3: the first 32 bits of the fractional parts of the
// square roots of the first 8 primes.
#define SV_SHA256_H0 \
  0x6a09e667u, 0xbb67ae85u, 0x3c6ef372u, 0xa54ff53au, 0x510e527fu, 0x9b05688cu, 0x1f83d9abu, 0x5be0cd19u
constexpr uint32_t kH0[8] = {SV_SHA256_H0};

__host__ __device__ inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

// One compression of a 16-word block into the state h (FIPS 180-4 Sec. 6.2.2),
// with the round constants K (kK on the device, kKHost on the host).  The
// schedule is kept as a 16-word window that rolls every 16 rounds; the rounds
// run in four groups of sixteen so every window index is static.
__host__ __device__ inline void compress_k(uint32_t h[8], uint32_t w[16], const uint32_t* K) {
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], k = h[7];
#pragma unroll 1
  for (int grp = 0; grp < 4; ++grp) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (grp > 0) {
        const uint32_t w15 = w[(t + 1) & 15], w2 = w[(t + 14) & 15];
        const uint32_t s0 = rotr(w15, 7) ^ rotr(w15, 18) ^ (w15 >> 3);
        const uint32_t s1 = rotr(w2, 17) ^ rotr(w2, 19) ^ (w2 >> 10);
        w[t] += s0 + w[(t + 9) & 15] + s1;
      }
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = k + S1 + ch + K[grp * 16 + t] + w[t];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
      k = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + S0 + mj;
    }
  }
  h[0] += a;
  h[1] += b;
  h[2] += c;
  h[3] += d;
  h[4] += e;
  h[5] += f;
  h[6] += g;
  h[7] += k;
}

__device__ inline void compress(uint32_t h[8], uint32_t w[16]) { compress_k(h, w, kK); }

// SHA-256 of a message in host memory (FIPS 180-4 Sec. 5.1.1 padding).
inline void sha256_host(const uint8_t* msg, size_t len, uint8_t out[32]) {
  uint32_t h[8] = {SV_SHA256_H0};
  const size_t total = (len + 9 + 63) / 64 * 64;  // message, 0x80, 64-bit length
  for (size_t off = 0; off < total; off += 64) {
    uint8_t blk[64];
    for (int i = 0; i < 64; ++i) {
      const size_t p = off + (size_t)i;
      blk[i] = p < len ? msg[p] : (p == len ? 0x80 : 0);
    }
    if (off + 64 == total)
      for (int i = 0; i < 8; ++i) blk[56 + i] = (uint8_t)(((uint64_t)len * 8) >> (56 - 8 * i));
    uint32_t w[16];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t)blk[4 * t] << 24 | (uint32_t)blk[4 * t + 1] << 16 |
             (uint32_t)blk[4 * t + 2] << 8 | blk[4 * t + 3];
    compress_k(h, w, kKHost);
  }
  for (int i = 0; i < 8; ++i)
    for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
}

// The state after hashing one block of the key xor pad (pad = 0x36 or 0x5c
// repeated): the 8-octet key fills words 0 and 1, the rest of the block is pad.
__device__ inline void keyed_state(uint32_t h[8], uint64_t seed, uint32_t pad) {
  uint32_t w[16];
  w[0] = (uint32_t)(seed >> 32) ^ pad;
  w[1] = (uint32_t)seed ^ pad;
#pragma unroll
  for (int j = 2; j < 16; ++j) w[j] = pad;
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = kH0[j];
  compress(h, w);
}

// The 53-bit verifier value, as an integer in [0, 2^53).  id[0..3] are the
// session id's 16 octets read as four big-endian words.
__device__ inline uint64_t verifier_bits(uint64_t seed, const uint32_t id[4], uint32_t round,
                                         uint32_t i, uint32_t purpose) {
  // inner hash: (key xor ipad) || message; the message block holds octets
  // 64..102 of the inner input, then 0x80, zeros and the bit length 103 * 8.
  uint32_t hi[8];
  keyed_state(hi, seed, 0x36363636u);
  uint32_t w[16];
  w[0] = 0x53444350u;  // "SDCP"
  w[1] = 0x2D564552u;  // "-VER"
  w[2] = 0x4946592Du;  // "IFY-"
  w[3] = 0x31000000u | (id[0] >> 16);  // "1", 0x00, id octets 0-1
  w[4] = (id[0] << 16) | (id[1] >> 16);
  w[5] = (id[1] << 16) | (id[2] >> 16);
  w[6] = (id[2] << 16) | (id[3] >> 16);
  w[7] = (id[3] << 16) | (round >> 16);  // id octets 14-15, round octets 0-1
  w[8] = (round << 16) | (i >> 16);
  w[9] = (i << 16) | ((purpose & 0xFFu) << 8) | 0x80u;
#pragma unroll
  for (int j = 10; j < 15; ++j) w[j] = 0;
  w[15] = (64 + 39) * 8;
  compress(hi, w);
  // outer hash: (key xor opad) || inner digest (32 octets, then padding)
  uint32_t ho[8];
  keyed_state(ho, seed, 0x5C5C5C5Cu);
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = hi[j];
  w[8] = 0x80000000u;
#pragma unroll
  for (int j = 9; j < 15; ++j) w[j] = 0;
  w[15] = (64 + 32) * 8;
  compress(ho, w);
  return (((uint64_t)ho[0] << 32) | ho[1]) >> 11;
}

}  // namespace sdcp
}  // namespace sv
