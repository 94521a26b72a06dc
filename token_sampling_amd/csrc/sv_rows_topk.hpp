// sv_rows_topk.hip -- one wave64 streams one bf16 logits row in a single pass
// and keeps an exact candidate set for the top-k tokens; then it applies
// temperature and top-p on those candidates (SDCP Sec. 4.1) and writes the
// row's support, sorted by token id, for the acceptance and sampling steps.
//
// Handles rows whose support lies inside the k best tokens with k <= 64: greedy
// rows and temperature-0 rows (k = 1) and rows with 1 <= top_k <= 64.
//
// Keys: a bf16 logit x maps to the signed 16-bit key  +mag(x) if x >= 0,
// -mag(x) if x < 0  (so -0 and +0 tie), computed two logits at a time with
// packed 16-bit instructions.  The profile order (logit desc, id asc) is the
// order of the 48-bit composite  (key + 0x8000) << 32 | ~id  (larger first).
// Positions outside the row (alignment head, tail of the last tile) are read
// as -inf, and -inf never enters the candidates (it has probability zero).
// Raw mode: when the first tiles already show k (lane, tile) maxima holding a
// positive logit, every token of the support is positive, and for positive
// values the raw bf16 bits read as a signed 16-bit integer equal the key
// (negative values read as negative integers and never pass a positive
// threshold).  Such rows skip the key transform.
//
// Candidate filter: a wave keeps, in its own LDS region, a superset of the k
// best (key, id) pairs seen so far.  Before the first tile is processed, the
// k-th largest of the lane maxima of the first four tiles (all in the load
// ring) bounds the k-th best key from below, so keys below it never enter.
// Before a tile that could overflow the region, the region is cut to exactly
// its k best and the threshold rises to the k-th best key; from then on a
// token must beat that key strictly (later tiles hold larger ids, which lose
// ties).  A tile that would overflow the region even after a cut (at most 256
// entries; adversarial rows such as ascending logits or tiny vocabularies) is
// handed back: the caller profiles the row exactly (sv_rows_exact.hpp).
#pragma once

#include "sv_kernels.hpp"
#include "sv_stream.hpp"

namespace sv {
namespace topk {

using namespace stream;

#ifndef SV_TOPK_VEC
#define SV_TOPK_VEC 2
#endif
#ifndef SV_TOPK_NBUF
#define SV_TOPK_NBUF 6
#endif
constexpr int kVec = SV_TOPK_VEC;          // 16-byte loads per lane per tile
constexpr int kNBuf = SV_TOPK_NBUF;        // tiles in the load ring (kNBuf - 1 in flight)
constexpr int kTile = kWave * kVec * 8;    // bf16 logits per tile
#ifndef SV_TOPK_CAP
#define SV_TOPK_CAP 256
#endif
constexpr int kCap = SV_TOPK_CAP;          // candidate entries per wave
constexpr int kMinKey = -0x7F7F;           // smallest finite key (-inf is -0x7F80)
#ifndef SV_TOPK_LOOSE_CUT
#define SV_TOPK_LOOSE_CUT 1  // cuts during the stream keep every tie at the k-th key
#endif
#ifndef SV_TOPK_BOUND_TILES
#define SV_TOPK_BOUND_TILES 4
#endif
constexpr int kBoundTiles = SV_TOPK_BOUND_TILES;  // tiles behind the first bound
static_assert(kBoundTiles <= kNBuf - 1, "the first bound's tiles are all in the ring");

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

// Key widths of the candidate composites (key + bias) << 32 | ~id: the signed
// 16-bit keys of bf16 rows, the signed 32-bit keys of binary32 rows.
struct Key16 {
  static constexpr int kBits = 16;
  __device__ static int unbias(uint32_t t) { return (int)t - 0x8000; }
  __device__ static uint32_t bias(int k) { return (uint32_t)(k + 0x8000); }
};
struct Key32 {
  static constexpr int kBits = 32;
  __device__ static int unbias(uint32_t t) { return (int)(t - 0x80000000u); }
  __device__ static uint32_t bias(int k) { return (uint32_t)k + 0x80000000u; }
};

__device__ inline uint64_t composite(int key, uint32_t id) {
  return ((uint64_t)(uint32_t)(key + 0x8000) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ inline int comp_key(uint64_t c) { return (int)(uint32_t)(c >> 32) - 0x8000; }
__device__ inline uint32_t comp_id(uint64_t c) { return 0xFFFFFFFFu - (uint32_t)c; }
__device__ inline float key_value(int key) {  // signed key -> bf16 value
  const uint32_t bits = key >= 0 ? (uint32_t)key : (0x8000u | (uint32_t)(-key));
  return __uint_as_float(bits << 16);
}
struct Cut {
  int n;    // entries left (all non-empty)
  int kth;  // k-th best key (valid when n == k)
};

// Cut the region reg[0..n) to its k best entries (k <= 64, n <= kCap) and
// compact them to the front; empty entries (0) are dropped.  An odd count is
// followed by one empty entry so that pair stores stay 16-byte aligned.
// kExact = false (the cuts during the stream) keeps every tie at the k-th key
// instead of the smallest ids among them, which skips the search over ids:
// later tokens must beat that key strictly, and a later token tied with it has
// a larger id than k kept entries, so the k best of the row are still there.
template <class K = Key16, bool kExact = true>
__device__ __attribute__((always_inline)) Cut region_cut(uint64_t* reg, int n, int k) {
  const int lane = __lane_id();
  uint64_t e[kCap / kWave];
  int live = 0;
#pragma unroll
  for (int i = 0; i < kCap / kWave; ++i) {
    const int j = i * kWave + lane;
    e[i] = j < n ? reg[j] : 0ull;
    live += popc64(__ballot(e[i] != 0));
  }
  // keep entries with biased key (key + 0x8000) > t, or == t with low word >= lowcut;
  // every non-empty entry has a biased key above 0, so t = 0 keeps them all
  uint32_t t = 0, lowcut = 0;
  int kth = K::unbias(0);
  if (live > k) {
    // the k-th largest biased key lies between the smallest and the largest
    // present, so it has their common leading bits: search the bits below
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kCap / kWave; ++i) {
      const uint32_t h = (uint32_t)(e[i] >> 32);
      if (e[i]) {
        lo = min(lo, h);
        hi = max(hi, h);
      }
    }
    lo = wave_reduce(lo, OpMin());
    hi = wave_reduce(hi, OpMax());
    const uint32_t diff = __builtin_amdgcn_readfirstlane(lo ^ hi);
    const int top = diff ? 31 - __builtin_clz(diff) : -1;
    t = (uint32_t)(((uint64_t)__builtin_amdgcn_readfirstlane(hi) >> (top + 1)) << (top + 1));
    for (int bit = top; bit >= 0; --bit) {  // k-th largest biased key, bit by bit
      const uint32_t cand = t | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < kCap / kWave; ++i) cnt += popc64(__ballot((uint32_t)(e[i] >> 32) >= cand));
      if (cnt >= k) t = cand;
    }
  int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kCap / kWave; ++i) {
      gt += popc64(__ballot((uint32_t)(e[i] >> 32) > t));
      eq += popc64(__ballot((uint32_t)(e[i] >> 32) == t));
    }
    const int need = k - gt;  // ties kept at key t, smallest ids first
    if (kExact && eq > need) {
      // the need-th largest low word among the ties lies between their
      // smallest and largest: search only the bits below their common ones
      uint32_t wlo = 0xFFFFFFFFu, whi = 0u;
#pragma unroll
      for (int i = 0; i < kCap / kWave; ++i) {
        if ((uint32_t)(e[i] >> 32) == t) {
          wlo = min(wlo, (uint32_t)e[i]);
          whi = max(whi, (uint32_t)e[i]);
        }
      }
      wlo = wave_reduce(wlo, OpMin());
      whi = wave_reduce(whi, OpMax());
      const uint32_t wdiff = __builtin_amdgcn_readfirstlane(wlo ^ whi);
      const int wtop = wdiff ? 31 - __builtin_clz(wdiff) : -1;
      uint32_t u =
          (uint32_t)(((uint64_t)__builtin_amdgcn_readfirstlane(whi) >> (wtop + 1)) << (wtop + 1));
      for (int bit = wtop; bit >= 0; --bit) {
        const uint32_t cand = u | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < kCap / kWave; ++i)
          cnt += popc64(__ballot((uint32_t)(e[i] >> 32) == t && (uint32_t)e[i] >= cand));
        if (cnt >= need) u = cand;
      }
      lowcut = u;
    }
    kth = K::unbias(t);
  } else if (live == k) {
    int mn = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kCap / kWave; ++i)
      if (e[i]) mn = min(mn, K::unbias((uint32_t)(e[i] >> 32)));
    mn = wave_reduce(mn, OpMin());
    kth = mn;
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < kCap / kWave; ++i) {
    const uint32_t hk = (uint32_t)(e[i] >> 32);
    const bool keep = e[i] != 0 && (hk > t || (hk == t && (uint32_t)e[i] >= lowcut));
    const uint64_t mask = __ballot(keep);
    if (keep) reg[base + lanes_below(mask)] = e[i];
    base += popc64(mask);
  }
  if ((base & 1) && lane == 0) reg[base] = 0ull;
  return Cut{base, kth};
}

// keys of one loaded tile, in place; returns the lane's largest key
__device__ inline int tile_keys(u32x4 (&v)[kVec], uint32_t& magmax) {
  uint32_t m = 0x80008000u;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = elem(v[j], d);
      const uint32_t k = key_pair(x);
      v[j][d] = k;
      m = max_i16x2(m, k);
      magmax = max_u16x2(magmax, x & 0x7FFF7FFFu);
    }
  }
  return max(lo16(m), hi16(m));
}

// raw mode: lane maximum of the raw bits as signed 16-bit integers, and the
// largest raw bit pattern as unsigned (above 0xFF80 only for a negative NaN)
__device__ inline int tile_raw(const u32x4 (&v)[kVec], uint32_t& umax) {
  uint32_t m = 0x80008000u;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = elem(v[j], d);
      m = max_i16x2(m, x);
      umax = max_u16x2(umax, x);
    }
  }
  return max(lo16(m), hi16(m));
}

// region slots this lane's tile needs at threshold te: two per dword
// holding a key >= te (the pair insertion below)
__device__ inline int slots_ge(const u32x4 (&v)[kVec], int te) {
  int n = 0;
#pragma unroll
  for (int q = 0; q < kVec * 4; ++q) {
    const uint32_t kq = elem(v[q >> 2], q & 3);
    n += max(lo16(kq), hi16(kq)) >= te ? 2 : 0;
  }
  return n;
}

// k-th largest of the N * 64 values held N per lane (k <= 64), as a signed
// 16-bit key
template <int N, class K = Key16>
__device__ inline int wave_kth_largest_n(const int (&v)[N], int k) {
  uint32_t t = 0;
  for (int bit = K::kBits - 1; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) cnt += popc64(__ballot(K::bias(v[i]) >= cand));
    if (cnt >= k) t = cand;
  }
  return K::unbias(t);
}

// lane maxima of one tile without changing it: raw bits as signed 16-bit
// integers, and keys
__device__ inline int lane_max_raw(const u32x4 (&v)[kVec]) {
  uint32_t m = 0x80008000u;
#pragma unroll
  for (int j = 0; j < kVec; ++j)
#pragma unroll
    for (int d = 0; d < 4; ++d) m = max_i16x2(m, elem(v[j], d));
  return max(lo16(m), hi16(m));
}
__device__ inline int lane_max_key(const u32x4 (&v)[kVec]) {
  uint32_t m = 0x80008000u;
#pragma unroll
  for (int j = 0; j < kVec; ++j)
#pragma unroll
    for (int d = 0; d < 4; ++d) m = max_i16x2(m, key_pair(elem(v[j], d)));
  return max(lo16(m), hi16(m));
}

struct WaveState {
  int n;            // region slots in use (even; empty entries are 0)
  int thr;          // candidates need key >= thr (or > thr when strict)
  bool strict;      // the threshold is the exact k-th best key of a cut
  bool overflow;    // the row is handed back to the exact profile
  bool raw;         // raw mode (see the file comment)
  uint32_t magmax;  // largest |x| bit pattern seen in key mode, packed pair
  uint32_t umax;    // largest raw bit pattern seen in raw mode, packed pair
};

// One tile: keys in place, the first-tile bound, then candidate insertion one
// dword (two logits per lane) at a time.  A lane whose dword holds a key at or
// above the threshold stores both halves as a pair of region entries, the
// half below the threshold as an empty entry: one ballot per dword.
// Positions outside the window [lo, hi) (the row, or a chunk of it) read as
// -inf; ids are positions minus head.
__device__ inline void tile_process(WaveState& s, uint64_t* reg, int k, u32x4 (&v)[kVec], int tile,
                                    int head, int lo, int hi) {
  if (s.overflow) return;
  const int lane = __lane_id();
  if (tile * kTile < lo || (tile + 1) * kTile > hi) mask_tile<kVec>(v, tile, lo, hi);
  int lm;
  if (s.raw) {
    lm = tile_raw(v, s.umax);
  } else {
    lm = tile_keys(v, s.magmax);
  }
  int te = max(s.strict ? s.thr + 1 : s.thr, kMinKey);
  const uint64_t lanes = __ballot(lm >= te);
  if (!lanes) return;
  if (s.n + popc64(lanes) * (kVec * 8) > kCap) {
    int c = lm >= te ? slots_ge(v, te) : 0;
    c = wave_reduce(c, OpAdd());
    if (s.n + c > kCap && s.n >= k) {
      Cut ct = region_cut<Key16, !SV_TOPK_LOOSE_CUT>(reg, s.n, k);
      te = max(ct.kth + 1, kMinKey);
      c = lm >= te ? slots_ge(v, te) : 0;
      c = wave_reduce(c, OpAdd());
      // ties at the k-th key left too little room: cut to exactly k
      if (((ct.n + 1) & ~1) + c > kCap) ct = region_cut<Key16, true>(reg, ct.n, k);
      s.n = __builtin_amdgcn_readfirstlane((ct.n + 1) & ~1);
      s.thr = ct.kth;
      s.strict = true;
    }
    if (s.n + c > kCap) {
      s.overflow = true;
      return;
    }
  }
  const int base_pos = tile * kTile + lane * 8 - head;
#pragma unroll
  for (int q = 0; q < kVec * 4; ++q) {
    const uint32_t kq = elem(v[q >> 2], q & 3);
    const int klo = lo16(kq), khi = hi16(kq);
    const bool hit = max(klo, khi) >= te;
    const uint64_t mk = __ballot(hit);
    if (mk) {
      if (hit) {
        const uint32_t p = (uint32_t)(base_pos + (q >> 2) * (kWave * 8) + 2 * (q & 3));
        u64x2 pr;
        pr[0] = klo >= te ? composite(klo, p) : 0ull;
        pr[1] = khi >= te ? composite(khi, p + 1) : 0ull;
        *(u64x2*)(reg + s.n + 2 * lanes_below(mk)) = pr;
      }
      s.n += 2 * popc64(mk);
    }
  }
}

// One compare-exchange stage of a bitonic sort over the wave's lanes (block
// size `size`, distance S): the partner's value by a lane exchange; desc
// sorts each block's first half largest first.
template <int S>
__device__ inline uint64_t bitonic_stage_desc(uint64_t x, int size) {
  const int lane = __lane_id();
  const uint64_t y = lane_xor<S>(x);
  const bool up = (lane & size) == 0;   // this block sorts descending
  const bool lower = (lane & S) == 0;   // I hold the first slot
  return (lower == up) ? (x > y ? x : y) : (x < y ? x : y);
}
template <int S>
__device__ inline void bitonic_stage_asc(uint32_t& key, double& val, int size) {
  const int lane = __lane_id();
  const uint32_t ok = lane_xor<S>(key);
  const double ov = lane_xor<S>(val);
  const bool up = (lane & size) == 0;  // this block sorts ascending
  const bool lower = (lane & S) == 0;
  // selects, not branches: the partner's pair replaces this lane's when it
  // belongs here (the smaller key in the block's first slot when ascending)
  const bool swap = (ok != key) & ((ok < key) == (lower == up));
  key = swap ? ok : key;
  val = swap ? ov : val;
}
template <int S>
__device__ inline uint64_t bitonic_merge_desc(uint64_t x, int size) {
  x = bitonic_stage_desc<S>(x, size);
  if constexpr (S > 1) x = bitonic_merge_desc<S / 2>(x, size);
  return x;
}
template <int S>
__device__ inline void bitonic_merge_asc(uint32_t& key, double& val, int size) {
  bitonic_stage_asc<S>(key, val, size);
  if constexpr (S > 1) bitonic_merge_asc<S / 2>(key, val, size);
}

// bitonic sort of one u64 per lane, largest first
__device__ inline uint64_t wave_sort_desc(uint64_t x) {
  x = bitonic_merge_desc<1>(x, 2);
  x = bitonic_merge_desc<2>(x, 4);
  x = bitonic_merge_desc<4>(x, 8);
  x = bitonic_merge_desc<8>(x, 16);
  x = bitonic_merge_desc<16>(x, 32);
  x = bitonic_merge_desc<32>(x, 64);
  return x;
}

// bitonic sort by ascending 32-bit key, carrying a binary64 payload
__device__ inline void wave_sort_asc(uint32_t& key, double& val) {
  bitonic_merge_asc<1>(key, val, 2);
  bitonic_merge_asc<2>(key, val, 4);
  bitonic_merge_asc<4>(key, val, 8);
  bitonic_merge_asc<8>(key, val, 16);
  bitonic_merge_asc<16>(key, val, 32);
  bitonic_merge_asc<32>(key, val, 64);
}

__device__ inline double wave_incl_scan_f64(double v) { return wave_incl_scan(v); }

// Wave maxima of packed 16-bit pairs, as one value.
__device__ inline int wave_pair_max(uint32_t pair) {
  pair = max_u16x2(pair, lane_xor<32>(pair));
  pair = max_u16x2(pair, lane_xor<16>(pair));
  pair = max_u16x2(pair, lane_xor<8>(pair));
  pair = max_u16x2(pair, lane_xor<4>(pair));
  pair = max_u16x2(pair, lane_xor<2>(pair));
  pair = max_u16x2(pair, lane_xor<1>(pair));
  return max((int)(pair & 0xFFFFu), (int)(pair >> 16));
}

// Key decoding of a composite, for the key width K: the signed key and its
// logit value.
template <class K>
__device__ inline int ckey(uint64_t c) { return K::unbias((uint32_t)(c >> 32)); }
template <class K>
__device__ inline float ckey_value(int key) {
  if constexpr (K::kBits == 16) return key_value(key);
  else return __uint_as_float(key >= 0 ? (uint32_t)key : (0x80000000u | (uint32_t)(-key)));
}

// The row's profile from its candidates: exactly the k best, sorted (one per
// lane), then the BAD_LOGITS checks, temperature and top-p (SDCP Sec. 4.1);
// the support is written sorted by id with its probabilities.  bad_seen: a
// NaN was seen in the row (the caller's wave maxima of magnitudes and of raw
// bits); kInfKey: the key of +inf.
template <class K>
__device__ __noinline__ void row_finish(uint64_t* reg, int n_reg, int k, bool bad_seen, int kInfKey,
                                        bool one_hot, uint32_t t_milli, uint32_t p_milli,
                                        int32_t x, RowRec* rec, int32_t* sup_id, double* sup_p) {
  const int lane = __lane_id();
  // the k best: a cut that keeps the ties at the k-th key, then the sort
  // below orders them by id; only when the ties leave more than a wave's
  // worth of entries the exact cut (a search over the ties' ids) first
  Cut ct = region_cut<K, false>(reg, n_reg, k);
  if (ct.n > kWave) ct = region_cut<K, true>(reg, ct.n, k);
  const int n = ct.n < k ? ct.n : k;  // entries of the k best (all of them when fewer)
  uint64_t e = lane < ct.n ? reg[lane] : 0ull;
  e = wave_sort_desc(e);

  const uint64_t top = lane_read(e, 0);
  const int kmax = ckey<K>(top);
  // NaN anywhere, +inf at the top, or no finite logit at all
  const bool bad = bad_seen || n == 0 || kmax >= kInfKey;

  RowRec r;
  r.ntie = 0;
  r.pad = 0;
  r.status = bad ? SV_S_BAD_LOGITS : 0;
  r.argmax = (int32_t)comp_id(top);
  r.nsup = 0;
  r.lmax = ckey_value<K>(kmax);
  r.ptok = -1.0;
  if (bad) {
    r.kcut = 0;
    r.idcut = 0;
    r.scale = 0.0;
    r.zsum = 1.0;
    if (lane == 0) *rec = r;
    return;
  }
  // weights exp((l - lmax) / T) of the top-k (one-hot: the argmax, weight 1)
  const double scale = one_hot ? 0.0 : 1.4426950408889634074 * 1000.0 / (double)t_milli;
  const bool live = lane < (one_hot ? 1 : n);
  const int kept = popc64(__ballot(live));
  const double w = live ? exp2(((double)ckey_value<K>(ckey<K>(e)) - (double)r.lmax) * scale) : 0.0;
  const double C = wave_incl_scan_f64(w);
  const double Zk = lane_read(C, kept - 1);
  int cut = kept;
  if (!one_hot && p_milli < 1000) {  // shortest prefix with 1000 * C >= P * Z_k
    const double tgt = (double)p_milli * Zk;
    const uint64_t hit = __ballot(live && 1000.0 * C >= tgt);
    cut = hit ? __builtin_ctzll(hit) + 1 : kept;
  }
  const double zsum = lane_read(C, cut - 1);
  const uint64_t last = lane_read(e, cut - 1);
  r.kcut = K::bias(ckey<K>(last));
  r.idcut = (int32_t)comp_id(last);
  r.scale = scale;
  r.zsum = zsum;
  r.nsup = cut;
  if (x >= 0) {
    const uint64_t hitx = __ballot(lane < cut && comp_id(e) == (uint32_t)x);
    const int jx = hitx ? __builtin_ctzll(hitx) : 0;
    const double wx = lane_read(w, jx);
    r.ptok = hitx ? wx / zsum : 0.0;
  }
  // the support in ascending id order, with p(y) = w(y) / Z'
  uint32_t sid = lane < cut ? comp_id(e) : 0xFFFFFFFFu;
  double sp = lane < cut ? w / zsum : 0.0;
  wave_sort_asc(sid, sp);
  if (lane < cut) {
    sup_id[lane] = (int32_t)sid;
    sup_p[lane] = sp;
  }
  if (lane == 0) *rec = r;
}

// Tiles of a row in the 16-byte aligned window over it: positions
// [head, head + V) are the row.
__device__ inline int row_head(const uint16_t* row) { return (int)(((uintptr_t)row & 15u) >> 1); }
__device__ inline int row_tiles(const uint16_t* row, int V) {
  return (row_head(row) + V + kTile - 1) / kTile;
}

// Stream tiles [t0, t1) of one row into the wave's candidate region reg (a
// superset of that chunk's k best is left there, s.n entries, unless
// s.overflow).  Loads past the chunk re-read its last vector; an empty chunk
// (t1 <= t0) loads nothing.
__device__ __attribute__((always_inline)) inline void chunk_scan(const uint16_t* row, int V, int k,
                                                                 int t0, int t1, WaveState& s,
                                                                 uint64_t* reg) {
  const int head = row_head(row);
  const u32x4* vbase = (const u32x4*)(row - head);
  const int npos = head + V;
  const int nvec = (npos + 7) / 8;
  const int lo = max(head, t0 * kTile), hi = min(npos, t1 * kTile);
  const int gmax = min(nvec, (t1 * kTile) / 8) - 1;  // last vector of the chunk
  const int ntiles = t1 - t0;

  s.n = 0;
  s.thr = -0x8000;
  s.strict = false;
  s.overflow = false;
  s.raw = false;
  s.magmax = 0;
  s.umax = 0;
  if (ntiles <= 0) return;  // gmax would be below the row

  // ring of kNBuf tiles: while one is processed the next kNBuf - 1 are in
  // flight.  The loop runs whole rounds of kNBuf tiles with no exit inside a
  // round, so each ring slot keeps its registers; tiles past the row's end
  // read as -inf (their loads re-read the row's last vector).
  u32x4 ring[kNBuf][kVec];
  // the first kNBuf - 1 tiles are issued in ring order (kept by the
  // scheduling barriers), as the steady state issues them
#pragma unroll
  for (int u = 0; u < kNBuf - 1; ++u) {
    load_tile<kVec>(ring[u], vbase, t0 + u, gmax);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the first bound: among the first kBoundTiles tiles, the k-th largest of
  // their lane maxima (k distinct tokens reach it, so the row's k-th best key
  // is at least that); raw mode when it is positive in raw bits
  {
#pragma unroll
    for (int u = 0; u < kBoundTiles; ++u)
      if ((t0 + u) * kTile < lo || (t0 + u + 1) * kTile > hi) mask_tile<kVec>(ring[u], t0 + u, lo, hi);
    int lmv[kBoundTiles];
#pragma unroll
    for (int u = 0; u < kBoundTiles; ++u) lmv[u] = lane_max_raw(ring[u]);
    const int t_raw = wave_kth_largest_n<kBoundTiles>(lmv, k);
    s.raw = t_raw > 0;
    if (s.raw) {
      s.thr = t_raw;
    } else {
#pragma unroll
      for (int u = 0; u < kBoundTiles; ++u) lmv[u] = lane_max_key(ring[u]);
      s.thr = wave_kth_largest_n<kBoundTiles>(lmv, k);
    }
  }
  const int nround = (ntiles + kNBuf - 1) / kNBuf;
  for (int r = 0; r < nround && !s.overflow; ++r) {
    set_priority(nround - r, nround);
#pragma unroll
    for (int u = 0; u < kNBuf; ++u) {
      const int tt = t0 + r * kNBuf + u;
      load_tile<kVec>(ring[(u + kNBuf - 1) % kNBuf], vbase, tt + kNBuf - 1, gmax);
      tile_process(s, reg, k, ring[u], tt, head, lo, hi);
    }
  }
}

// The profile of one row of the top-k class, by one wave: rows whose support
// lies among the k <= 64 best tokens (k = 1 for one-hot profiles).  reg is
// the wave's LDS region of kCap entries; sup_id, sup_p its listed support.
__device__ __attribute__((always_inline)) inline bool row_profile(
    const uint16_t* row, int V, int k, bool one_hot, const sv_sampling& smp, int32_t x, RowRec* rec,
    int32_t* sup_id, double* sup_p, uint64_t* reg) {
  WaveState s;
  chunk_scan(row, V, k, 0, row_tiles(row, V), s, reg);
  if (s.overflow) return true;  // handed back: the caller profiles it exactly
  const bool nan = wave_pair_max(s.magmax) > 0x7F80 || wave_pair_max(s.umax) > 0xFF80;
  row_finish<Key16>(reg, s.n, k, nan, 0x7F80, one_hot, smp.temperature_milli, smp.top_p_milli, x,
                    rec, sup_id, sup_p);
  return false;
}

}  // namespace topk
}  // namespace sv
