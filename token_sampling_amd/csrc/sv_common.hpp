// sv_common.hpp -- device-side building blocks of libspecverify (gfx950).
//
// Ordered keys: every logit is mapped to an unsigned key whose integer order
// is the float order, with -0 and +0 mapped to the same key (equal logits tie
// by token id).  The profile's total order (logit desc, id asc) is then
// (key desc, id asc) on exact integers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr int kWave = 64;

// ---------------------------------------------------------------- row record
// Everything the per-session kernels need about one logits row, written by
// the row kernel.  The profile's support is {y : key(y) > kcut} plus the
// tokens with key(y) == kcut and y <= idcut; every member has the weight
// 2^((l_y - lmax) * scale), and the normaliser of the support is zsum.
// When nsup > 0 the support is also listed (ids ascending, with p(y)) in the
// workspace's support arrays, and the additional token is drawn from that
// list instead of the logits row.
constexpr int kSupMax = 64;
struct RowRec {
  int32_t status;  // 0, or SV_S_BAD_LOGITS
  int32_t argmax;  // smallest id attaining the largest logit
  uint32_t kcut;   // key of the last token of the support (in profile order)
  int32_t idcut;   // its token id (< 0: not resolved, see ntie)
  float lmax;      // largest logit
  int32_t nsup;    // entries of the listed support (0: not listed)
  double scale;    // log2(e) * 1000 / temperature_milli; 0 when T = 0
  double zsum;     // mass of the support
  double ptok;     // probability of the drafted token; -1 for the bonus row
  int32_t ntie;    // idcut < 0: the support keeps the ntie smallest ids at key kcut
  int32_t pad;
};
static_assert(sizeof(RowRec) == 56, "RowRec layout");

// Per-session draw left for the whole workgroup after the acceptance wave.
enum JobKind : int32_t { kJobNone = 0, kJobResidual = 1, kJobBonus = 2 };
struct Job {
  int32_t kind;
  int32_t pos;   // 0-based output position of the additional token (= a)
  int32_t trow;  // 0-based target row index inside the session
  int32_t drow;  // 0-based draft row index (residual only)
  double u;      // purpose-1 uniform
};
static_assert(sizeof(Job) == 24, "Job layout");

// ---------------------------------------------------------------- element traits
struct Bf16 {
  using elem_t = uint16_t;
  static constexpr int32_t kDtype = SV_BF16;
  static constexpr uint32_t kSign = 0x8000u;
  static constexpr uint32_t kInfKey = 0x8000u + 0x7F80u;  // key(+inf)
  static constexpr uint32_t kNegInfKey = 0x8000u - 0x7F80u;  // key(-inf)
  static constexpr int kKeyBits = 16;
  static constexpr uint32_t kNegInfBits = 0xFF80u;
  __device__ static inline uint32_t bits(elem_t e) { return e; }
  __device__ static inline float value(uint32_t u) { return __uint_as_float(u << 16); }
  __device__ static inline uint32_t key(uint32_t u) {
    uint32_t mag = u & 0x7FFFu;
    return (u & kSign) ? kSign - mag : kSign + mag;
  }
  __device__ static inline uint32_t unkey(uint32_t k) {
    return k >= kSign ? k - kSign : (kSign | (kSign - k));
  }
};

struct F32 {
  using elem_t = uint32_t;
  static constexpr int32_t kDtype = SV_FP32;
  static constexpr uint32_t kSign = 0x80000000u;
  static constexpr uint32_t kInfKey = 0x80000000u + 0x7F800000u;
  static constexpr uint32_t kNegInfKey = 0x80000000u - 0x7F800000u;
  static constexpr int kKeyBits = 32;
  static constexpr uint32_t kNegInfBits = 0xFF800000u;
  __device__ static inline uint32_t bits(elem_t e) { return e; }
  __device__ static inline float value(uint32_t u) { return __uint_as_float(u); }
  __device__ static inline uint32_t key(uint32_t u) {
    uint32_t mag = u & 0x7FFFFFFFu;
    return (u & kSign) ? kSign - mag : kSign + mag;
  }
  __device__ static inline uint32_t unkey(uint32_t k) {
    return k >= kSign ? k - kSign : (kSign | (kSign - k));
  }
};

// Weight of a support member: exp((l - lmax) / T) = 2^((l - lmax) * scale),
// evaluated in binary64.  The difference of two binary32 values is exact in
// binary64.
__device__ inline double weight64(float l, float lmax, double scale) {
  return exp2(((double)l - (double)lmax) * scale);
}

// ---------------------------------------------------------------- Philox4x64-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): ten rounds of two 64x64->128-bit products; the key is bumped by two
// Weyl constants after each round.
__device__ inline void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t m0 = 0xD2E7470EE14C6C93ull, m1 = 0xCA5A826395121157ull;
  const uint64_t w0 = 0x9E3779B97F4A7C15ull, w1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = m0 * c[0], hi0 = __umul64hi(m0, c[0]);
    const uint64_t lo1 = m1 * c[2], hi1 = __umul64hi(m1, c[2]);
    const uint64_t n0 = hi1 ^ c[1] ^ k0;
    const uint64_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += w0;
    k1 += w1;
  }
}

// Verifier uniforms (SDCP Sec. 6.4 structure): word 0 -> acceptance test,
// word 1 -> additional token; the top 53 bits times 2^-53.
__device__ inline void verifier_uniforms(uint64_t seed, uint64_t session_key, uint32_t round,
                                         uint32_t pos1, double* u_acc, double* u_add) {
  uint64_t c[4] = {round, pos1, 0, 0};
  philox4x64_10(c, seed, session_key);
  *u_acc = (double)(c[0] >> 11) * 0x1p-53;
  *u_add = (double)(c[1] >> 11) * 0x1p-53;
}

// ------------------------------------------------------- lane exchanges
// The value of lane (this lane xor S), without the LDS crossbar that a
// general shuffle (ds_bpermute) goes through: DPP within rows of 16 lanes
// (quad permutes for 1 and 2; a rotate by 8 for 8; for 4, the rotates by 4
// and by 12, one of which brings the partner), the permlane swaps between
// rows for 16 and 32 (called with the value as both operands, the swap
// leaves the partner's value in the first result in the upper rows and in
// the second result in the lower rows).  Each takes a few cycles where a
// shuffle waits on the LDS.  Every lane of the wave must be active.
template <int kCtrl>
__device__ inline uint32_t dpp_u32(uint32_t x) {  // every source lane lies in the row
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kCtrl, 0xF, 0xF, true);
}
template <int S>
__device__ inline uint32_t lane_xor_u32(uint32_t x) {
  static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "xor distance");
  const int lane = __lane_id();
  if constexpr (S == 1) {
    return dpp_u32<0xB1>(x);  // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return dpp_u32<0x4E>(x);  // quad_perm [2,3,0,1]
  } else if constexpr (S == 4) {
    const uint32_t up = dpp_u32<0x120 + 12>(x), dn = dpp_u32<0x120 + 4>(x);  // row_ror
    return (lane & 4) ? dn : up;
  } else if constexpr (S == 8) {
    return dpp_u32<0x120 + 8>(x);  // row_ror:8
  } else if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}
template <int S, typename T>
__device__ inline T lane_xor(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, lane_xor_u32<S>(__builtin_bit_cast(uint32_t, v)));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = lane_xor_u32<S>((uint32_t)u), hi = lane_xor_u32<S>((uint32_t)(u >> 32));
    return __builtin_bit_cast(T, lo | (hi << 32));
  }
}
// The value of lane l of a 32- or 64-bit value, l the same in every lane.
template <typename T>
__device__ inline T lane_read(T v, int l) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  l = __builtin_amdgcn_readfirstlane(l);
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(T, lo | (hi << 32));
  }
}

// ---------------------------------------------------------------- reductions
// Deterministic block-wide reductions: a fixed xor-butterfly inside each
// wave64 (distances 32, 16, ..., 1), then the wave totals combined in wave
// order by every thread.
template <typename T, typename Op>
__device__ inline T wave_reduce(T v, Op op) {
  v = op(v, lane_xor<32>(v));
  v = op(v, lane_xor<16>(v));
  v = op(v, lane_xor<8>(v));
  v = op(v, lane_xor<4>(v));
  v = op(v, lane_xor<2>(v));
  v = op(v, lane_xor<1>(v));
  return v;
}

// Inclusive prefix sum over the wave's lanes, in lane order: within rows of
// 16 lanes (DPP shifts by 1, 2, 4, 8; a lane whose source would lie before
// its row's first lane adds 0), then the rows' totals carried on (lane 15
// broadcast into rows 1 and 3, then lane 31 into rows 2 and 3).  Every lane
// of the wave must be active.
template <int kCtrl, int kRowMask, typename T>
__device__ inline T dpp_move(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(
        T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF, false));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, kCtrl, kRowMask, 0xF, false);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), kCtrl,
                                                              kRowMask, 0xF, false);
    return __builtin_bit_cast(T, lo | (hi << 32));
  }
}
template <typename T>
__device__ inline T wave_incl_scan(T v) {
  v += dpp_move<0x111, 0xF>(v);  // row_shr:1
  v += dpp_move<0x112, 0xF>(v);  // row_shr:2
  v += dpp_move<0x114, 0xF>(v);  // row_shr:4
  v += dpp_move<0x118, 0xF>(v);  // row_shr:8
  v += dpp_move<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

template <int NT, typename T, typename Op>
__device__ inline T block_reduce(T v, Op op, T* smem) {
  static_assert(NT % kWave == 0, "block of whole waves");
  v = wave_reduce(v, op);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[threadIdx.x / kWave] = v;
  __syncthreads();
  T r = smem[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) r = op(r, smem[w]);
  return r;
}

struct OpAdd {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a > b ? a : b; }
};
struct OpMin {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a < b ? a : b; }
};
struct OpOr {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a | b; }
};

}  // namespace sv
