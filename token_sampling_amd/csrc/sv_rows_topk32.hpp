// sv_rows_topk32.hpp -- one wave64 streams one binary32 logits row in a single
// pass and keeps an exact candidate set for its k <= 64 best tokens (greedy
// rows, temperature-0 rows, 1 <= top_k <= 64); the profile of those candidates
// (temperature, top-p, SDCP Sec. 4.1) is topk::row_finish on 32-bit keys.
//
// The design is the bf16 path's (sv_rows_topk.hpp) on one logit per dword:
//  - keys: a binary32 logit x maps to the signed 32-bit key +mag(x) if x >= 0,
//    -mag(x) if x < 0 (-0 and +0 tie); the profile order (logit desc, id asc)
//    is the order of the composite (key + 2^31) << 32 | ~id;
//  - raw mode: once the first bound is positive every token of the support is
//    positive, and positive logits' raw bits read as signed integers are their
//    keys (negative logits read as negative integers);
//  - the first bound is the k-th largest of the lane maxima of the first four
//    tiles, all in the load ring; a tile that could overflow the wave's
//    256-entry LDS region first cuts it to its k best, after which later tiles
//    must beat the k-th key strictly; a tile that would still overflow hands
//    the row back to the exact profile.
// One lane inserts one entry (8 bytes) per logit at or above the threshold,
// one ballot per dword position of the tile.
#pragma once

#include "sv_rows_topk.hpp"

namespace sv {
namespace topk32 {

using namespace stream;
using topk::Key32;

constexpr int kVec = 2;                  // 16-byte loads per lane per tile
constexpr int kNBuf = 6;                 // tiles in the load ring (kNBuf - 1 in flight)
constexpr int kTile = kWave * kVec * 4;  // binary32 logits per tile
constexpr int kCap = topk::kCap;         // candidate entries per wave
constexpr int kMinKey = -0x7F7FFFFF;     // smallest finite key (-inf is -0x7F800000)
constexpr int kBoundTiles = 4;
static_assert(kBoundTiles <= kNBuf - 1, "the first bound's tiles are all in the ring");

__device__ inline int key32(uint32_t x) {
  const int mag = (int)(x & 0x7FFFFFFFu);
  return (x >> 31) ? -mag : mag;
}
__device__ inline uint64_t composite(int key, uint32_t id) {
  return ((uint64_t)Key32::bias(key) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

// keys of one loaded tile, in place; the lane's largest key
__device__ inline int tile_keys(u32x4 (&v)[kVec], uint32_t& magmax) {
  int m = INT32_MIN;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = elem(v[j], d);
      const int k = key32(x);
      v[j][d] = (uint32_t)k;
      m = max(m, k);
      magmax = max(magmax, x & 0x7FFFFFFFu);
    }
  }
  return m;
}

// raw mode: the lane's largest raw bits as a signed integer, and its largest
// raw bit pattern as unsigned (above 0xFF800000 only for a negative NaN)
__device__ inline int tile_raw(const u32x4 (&v)[kVec], uint32_t& umax) {
  int m = INT32_MIN;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = elem(v[j], d);
      m = max(m, (int)x);
      umax = max(umax, x);
    }
  }
  return m;
}

__device__ inline int lane_max_raw(const u32x4 (&v)[kVec]) {
  int m = INT32_MIN;
#pragma unroll
  for (int j = 0; j < kVec; ++j)
#pragma unroll
    for (int d = 0; d < 4; ++d) m = max(m, (int)elem(v[j], d));
  return m;
}
__device__ inline int lane_max_key(const u32x4 (&v)[kVec]) {
  int m = INT32_MIN;
#pragma unroll
  for (int j = 0; j < kVec; ++j)
#pragma unroll
    for (int d = 0; d < 4; ++d) m = max(m, key32(elem(v[j], d)));
  return m;
}

// region slots this lane's tile needs at threshold te
__device__ inline int slots_ge(const u32x4 (&v)[kVec], int te) {
  int n = 0;
#pragma unroll
  for (int q = 0; q < kVec * 4; ++q) n += (int)elem(v[q >> 2], q & 3) >= te ? 1 : 0;
  return n;
}

struct WaveState {
  int n;            // region slots in use (empty entries are 0)
  int thr;          // candidates need key >= thr (or > thr when strict)
  bool strict;      // the threshold is the exact k-th best key of a cut
  bool overflow;    // the row is handed back to the exact profile
  bool raw;         // raw mode
  uint32_t magmax;  // largest |x| bit pattern seen in key mode
  uint32_t umax;    // largest raw bit pattern seen in raw mode
};

// One tile: keys in place (key mode), then candidate insertion one dword
// position at a time (one ballot each).
__device__ inline void tile_process(WaveState& s, uint64_t* reg, int k, u32x4 (&v)[kVec], int tile,
                                    int head, int lo, int hi) {
  if (s.overflow) return;
  const int lane = __lane_id();
  if (tile * kTile < lo || (tile + 1) * kTile > hi) mask_tile_f32<kVec>(v, tile, lo, hi);
  const int lm = s.raw ? tile_raw(v, s.umax) : tile_keys(v, s.magmax);
  int te = max(s.strict ? s.thr + 1 : s.thr, kMinKey);
  const uint64_t lanes = __ballot(lm >= te);
  if (!lanes) return;
  if (s.n + popc64(lanes) * (kVec * 4) > kCap) {
    int c = lm >= te ? slots_ge(v, te) : 0;
    c = wave_reduce(c, OpAdd());
    if (s.n + c > kCap && s.n >= k) {
      topk::Cut ct = topk::region_cut<Key32, false>(reg, s.n, k);
      te = max(ct.kth + 1, kMinKey);
      c = lm >= te ? slots_ge(v, te) : 0;
      c = wave_reduce(c, OpAdd());
      // ties at the k-th key left too little room: cut to exactly k
      if (ct.n + c > kCap) ct = topk::region_cut<Key32, true>(reg, ct.n, k);
      s.n = __builtin_amdgcn_readfirstlane(ct.n);
      s.thr = ct.kth;
      s.strict = true;
    }
    if (s.n + c > kCap) {
      s.overflow = true;
      return;
    }
  }
  const int base_pos = tile * kTile + lane * 4 - head;
#pragma unroll
  for (int q = 0; q < kVec * 4; ++q) {
    const int kq = (int)elem(v[q >> 2], q & 3);
    const bool hit = kq >= te;
    const uint64_t mk = __ballot(hit);
    if (mk) {
      if (hit) {
        const uint32_t p = (uint32_t)(base_pos + (q >> 2) * (kWave * 4) + (q & 3));
        reg[s.n + lanes_below(mk)] = composite(kq, p);
      }
      s.n += popc64(mk);
    }
  }
}

// The profile of one binary32 row of the top-k class, by one wave.  reg is
// the wave's LDS region of kCap entries.  Returns true if the row is handed
// back (the caller profiles it exactly).
__device__ __attribute__((always_inline)) inline bool row_profile(
    const uint32_t* row, int V, int k, bool one_hot, const sv_sampling& smp, int32_t x, RowRec* rec,
    int32_t* sup_id, double* sup_p, uint64_t* reg) {
  const int head = (int)(((uintptr_t)row & 15u) >> 2);
  const u32x4* vbase = (const u32x4*)(row - head);
  const int npos = head + V;
  const int nvec = (npos + 3) / 4;
  const int ntiles = (npos + kTile - 1) / kTile;
  const int gmax = nvec - 1;
  WaveState s{0, INT32_MIN, false, false, false, 0u, 0u};

  u32x4 ring[kNBuf][kVec];
#pragma unroll
  for (int u = 0; u < kNBuf - 1; ++u) {
    load_tile<kVec>(ring[u], vbase, u, gmax);
    __builtin_amdgcn_sched_barrier(0);
  }
  {  // the first bound, from the first kBoundTiles tiles
#pragma unroll
    for (int u = 0; u < kBoundTiles; ++u)
      if (u * kTile < head || (u + 1) * kTile > npos) mask_tile_f32<kVec>(ring[u], u, head, npos);
    int lmv[kBoundTiles];
#pragma unroll
    for (int u = 0; u < kBoundTiles; ++u) lmv[u] = lane_max_raw(ring[u]);
    const int t_raw = topk::wave_kth_largest_n<kBoundTiles, Key32>(lmv, k);
    s.raw = t_raw > 0;
    if (s.raw) {
      s.thr = t_raw;
    } else {
#pragma unroll
      for (int u = 0; u < kBoundTiles; ++u) lmv[u] = lane_max_key(ring[u]);
      s.thr = topk::wave_kth_largest_n<kBoundTiles, Key32>(lmv, k);
    }
  }
  const int nround = (ntiles + kNBuf - 1) / kNBuf;
  for (int r = 0; r < nround && !s.overflow; ++r) {
    set_priority(nround - r, nround);
#pragma unroll
    for (int u = 0; u < kNBuf; ++u) {
      const int tt = r * kNBuf + u;
      load_tile<kVec>(ring[(u + kNBuf - 1) % kNBuf], vbase, tt + kNBuf - 1, gmax);
      tile_process(s, reg, k, ring[u], tt, head, head, npos);
    }
  }
  if (s.overflow) return true;
  const uint32_t mm = wave_reduce(s.magmax, OpMax()), um = wave_reduce(s.umax, OpMax());
  const bool nan = mm > 0x7F800000u || um > 0xFF800000u;
  topk::row_finish<Key32>(reg, s.n, k, nan, 0x7F800000, one_hot, smp.temperature_milli,
                          smp.top_p_milli, x, rec, sup_id, sup_p);
  return false;
}

}  // namespace topk32
}  // namespace sv
