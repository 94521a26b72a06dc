// sv_stream.hpp -- pieces shared by the row kernels that stream bf16 logits
// rows with one wave64 per row: 16-byte nontemporal loads into a ring of
// tiles, masks for the row's ends, packed 16-bit helpers, issue priority.
#pragma once

#include "sv_common.hpp"

namespace sv {
namespace stream {

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Element reads from ext-vector values go through a scalar first: this
// compiler reads element 0 when __builtin_bit_cast is applied to an element.
__device__ inline uint32_t elem(const u32x4& v, int d) {
  const uint32_t w = v[d];
  return w;
}

__device__ inline uint32_t key_pair(uint32_t x) {
  const s16x2 v = __builtin_bit_cast(s16x2, x);
  const s16x2 mag = v & (s16x2)(0x7FFF);
  const s16x2 s = v >> 15;  // 0 or -1 per half
  return __builtin_bit_cast(uint32_t, (s16x2)((mag ^ s) - s));
}
__device__ inline uint32_t max_i16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, a),
                                                                __builtin_bit_cast(s16x2, b)));
}
__device__ inline uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ inline int lo16(uint32_t k) { return (int)(short)(k & 0xFFFFu); }
__device__ inline int hi16(uint32_t k) { return (int)(short)(k >> 16); }

__device__ inline int popc64(uint64_t m) { return __builtin_popcountll(m); }
__device__ inline int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Issue the loads of one tile (VEC 16-byte vectors per lane, 64 * VEC * 8
// bf16 logits).  Every call issues the same loads on every path, so the
// compiler's wait counts stay exact across a ring of tiles.  They are
// nontemporal buffer loads over vectors [0, gmax] of vbase (vbase and gmax
// wave-uniform): the tile's offset goes into the lane's byte offset, which
// the buffer's range check covers (its scalar offset would not be), so a
// vector past gmax reads as zeros without touching memory; the caller masks
// the positions past the row when it consumes the tile.  One add per tile
// instead of a clamp and a 64-bit address per load.
constexpr int kBufferDword3 = 0x00020000;  // raw buffer, this chip's default format
constexpr int kNonTemporal = 2;            // cache policy: nt
template <int VEC>
__device__ inline void load_tile(u32x4 (&v)[VEC], const u32x4* vbase, int tile, int gmax) {
  const int lane = __lane_id();
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, (gmax + 1) * 16, kBufferDword3);
  const int off = (tile * (kWave * VEC) + lane) * 16;
#pragma unroll
  for (int j = 0; j < VEC; ++j)
    v[j] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + j * kWave * 16, 0, kNonTemporal));
}

// Positions outside [lo, hi) read as -inf; only tiles that touch the window's
// ends call this.
template <int VEC>
__device__ inline void mask_tile(u32x4 (&v)[VEC], int tile, int lo, int hi) {
  const int lane = __lane_id();
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int p0 = 8 * (tile * (kWave * VEC) + j * kWave + lane);  // first logit of the vector
    if (p0 < lo || p0 + 8 > hi) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int p = p0 + 2 * d;
        uint32_t x = elem(v[j], d);
        if (p < lo || p >= hi) x = (x & 0xFFFF0000u) | 0xFF80u;
        if (p + 1 < lo || p + 1 >= hi) x = (x & 0x0000FFFFu) | 0xFF800000u;
        v[j][d] = x;
      }
    }
  }
}

// The same for a tile of binary32 logits (4 per 16-byte vector).
template <int VEC>
__device__ inline void mask_tile_f32(u32x4 (&v)[VEC], int tile, int lo, int hi) {
  const int lane = __lane_id();
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int p0 = 4 * (tile * (kWave * VEC) + j * kWave + lane);  // first logit of the vector
#pragma unroll
    for (int d = 0; d < 4; ++d)
      if (p0 + d < lo || p0 + d >= hi) v[j][d] = 0xFF800000u;
  }
}

// Issue priority from the work a wave has left: a SIMD's arbiter serves the
// highest priority first and the oldest wave among equals, so with equal
// priorities the oldest wave streams its row well ahead of the others, the
// others finish late and the memory system runs short of requests at the
// end.  Waves with more of their row left ask for a higher priority.
#ifndef SV_TOPK_PRIO
#define SV_TOPK_PRIO 1
#endif
__device__ inline void set_priority(int left, int total) {
#if SV_TOPK_PRIO == 1
  if (2 * left > total) __builtin_amdgcn_s_setprio(3);
  else if (4 * left > total) __builtin_amdgcn_s_setprio(2);
  else if (8 * left > total) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
#elif SV_TOPK_PRIO == 2
  if (4 * left > 3 * total) __builtin_amdgcn_s_setprio(3);
  else if (2 * left > total) __builtin_amdgcn_s_setprio(2);
  else if (4 * left > total) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
#else
  (void)left;
  (void)total;
#endif
}

}  // namespace stream
}  // namespace sv
