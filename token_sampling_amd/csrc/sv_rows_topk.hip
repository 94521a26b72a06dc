// sv_rows_topk.hip -- one wave64 streams one bf16 logits row in a single pass
// and keeps an exact candidate set for the top-k tokens; then it applies
// temperature and top-p on those candidates (SDCP Sec. 4.1).
//
// Handles rows whose support lies inside the k best tokens with k <= 64: greedy
// rows and temperature-0 rows (k = 1) and rows with 1 <= top_k <= 64.
//
// Keys: a bf16 logit x maps to the signed 16-bit key  +mag(x) if x >= 0,
// -mag(x) if x < 0  (so -0 and +0 tie), computed two logits at a time with
// packed 16-bit instructions.  The profile order (logit desc, id asc) is the
// order of the 48-bit composite  (key + 0x8000) << 32 | ~id  (larger first).
//
// Candidate filter: a wave keeps, in its own LDS region, a superset of the k
// best (key, id) pairs seen so far.  On the first tile the k-th largest lane
// maximum bounds the k-th best key from below, so keys below it never enter.
// Before a tile that could overflow the region, the region is cut to exactly
// its k best and the threshold rises to the k-th best key; from then on a
// token must beat that key strictly (later tiles hold larger ids, which lose
// ties).  A tile that would overflow the region even after a cut (at most 256
// entries; adversarial rows such as ascending logits or tiny vocabularies) is
// left to the generic kernel (status kRowFallback).
#include "sv_kernels.hpp"

namespace sv {

namespace {

constexpr int kVec = 4;                    // 16-byte loads per lane per tile
constexpr int kTile = kWave * kVec * 8;    // bf16 logits per tile (4096)
constexpr int kCap = 256;                  // candidate entries per wave
constexpr int kWavesPerBlock = 4;          // independent rows per workgroup

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

__device__ inline uint64_t composite(int key, uint32_t id) {
  return ((uint64_t)(uint32_t)(key + 0x8000) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ inline int comp_key(uint64_t c) { return (int)(uint32_t)(c >> 32) - 0x8000; }
__device__ inline uint32_t comp_id(uint64_t c) { return 0xFFFFFFFFu - (uint32_t)c; }
__device__ inline float key_value(int key) {  // signed key -> bf16 value
  const uint32_t bits = key >= 0 ? (uint32_t)key : (0x8000u | (uint32_t)(-key));
  return __uint_as_float(bits << 16);
}

__device__ inline int wave_excl_scan(int v, int* total) {
  const int lane = __lane_id();
  int inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += t;
  }
  *total = __shfl(inc, kWave - 1, kWave);
  return inc - v;
}

__device__ inline int popc64(uint64_t m) { return __builtin_popcountll(m); }

// Cut the region reg[0..n) to its k best entries (k <= 64, n <= kCap).
// Returns the new count (min(n, k)); *kth receives the k-th best key if n >= k.
__device__ __noinline__ int region_cut(uint64_t* reg, int n, int k, int* kth) {
  const int lane = __lane_id();
  uint64_t e[kCap / kWave];
#pragma unroll
  for (int i = 0; i < kCap / kWave; ++i) {
    const int j = i * kWave + lane;
    e[i] = j < n ? reg[j] : 0ull;
  }
  if (n <= k) {
    if (n == k) {
      int mn = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < kCap / kWave; ++i)
        if (e[i]) mn = min(mn, comp_key(e[i]));
      for (int off = kWave / 2; off > 0; off >>= 1) mn = min(mn, __shfl_xor(mn, off, kWave));
      *kth = mn;
    }
    return n;
  }
  // k-th largest biased key (key + 0x8000), bit by bit
  uint32_t t = 0;
  for (int bit = 15; bit >= 0; --bit) {
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
    eq += popc64(__ballot(e[i] != 0 && (uint32_t)(e[i] >> 32) == t));
  }
  const int need = k - gt;  // ties kept at key t, smallest ids first
  uint32_t lowcut = 0;      // keep ties whose low word (~id) >= lowcut
  if (eq > need) {
    uint32_t u = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = u | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < kCap / kWave; ++i)
        cnt += popc64(__ballot(e[i] != 0 && (uint32_t)(e[i] >> 32) == t && (uint32_t)e[i] >= cand));
      if (cnt >= need) u = cand;
    }
    lowcut = u;
  }
  int base = 0;
#pragma unroll
  for (int i = 0; i < kCap / kWave; ++i) {
    const uint32_t hk = (uint32_t)(e[i] >> 32);
    const bool keep = e[i] != 0 && (hk > t || (hk == t && (uint32_t)e[i] >= lowcut));
    const uint64_t mask = __ballot(keep);
    if (keep) reg[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0))] = e[i];
    base += popc64(mask);
  }
  *kth = (int)t - 0x8000;
  return base;  // == k
}

struct WaveState {
  uint64_t* reg;    // this wave's LDS region
  int n;            // entries in the region
  int k;            // tokens the support may hold
  int thr;          // candidates need key >= thr (or > thr when strict)
  bool strict;      // the threshold is the exact k-th best key of a cut
  bool overflow;    // the row is left to the generic kernel
  uint32_t magmax;  // largest |x| bit pattern seen (NaN detection), packed pair
};

template <bool kFull>
__device__ inline void load_tile(u32x4 (&v)[kVec], const u32x4* vbase, int tile, int nvec) {
  const int lane = __lane_id();
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int g = tile * (kTile / 8) + j * kWave + lane;
    if (kFull) {
      v[j] = __builtin_nontemporal_load(vbase + g);
    } else {
      v[j] = (u32x4)(0u);
      if (g < nvec) v[j] = __builtin_nontemporal_load(vbase + g);
    }
  }
}

__device__ inline void load_tile_any(u32x4 (&v)[kVec], const u32x4* vbase, int tile, int nvec) {
  if ((tile + 1) * (kTile / 8) <= nvec) load_tile<true>(v, vbase, tile, nvec);
  else load_tile<false>(v, vbase, tile, nvec);
}

// keys of one loaded tile, in place; positions outside the row (boundary
// tiles only) get key -32768.  Returns the lane's largest key.
template <bool kInterior>
__device__ inline int tile_keys(u32x4 (&v)[kVec], int tile, int head, int V, uint32_t& magmax) {
  const int lane = __lane_id();
  const int tile_pos = tile * kTile;
  uint32_t m = 0x80008000u;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = v[j][d];
      uint32_t k = key_pair(x);
      uint32_t mg = x & 0x7FFF7FFFu;
      if (!kInterior) {
        const int p = tile_pos + (j * kWave + lane) * 8 + 2 * d;
        const bool vlo = p >= head && p < head + V;
        const bool vhi = p + 1 >= head && p + 1 < head + V;
        k = (vlo ? (k & 0xFFFFu) : 0x8000u) | (vhi ? (k & 0xFFFF0000u) : 0x80000000u);
        mg = (vlo ? (mg & 0xFFFFu) : 0u) | (vhi ? (mg & 0xFFFF0000u) : 0u);
      }
      v[j][d] = k;
      m = max_i16x2(m, k);
      magmax = max_u16x2(magmax, mg);
    }
  }
  return max(lo16(m), hi16(m));
}

// k-th largest of the 64 lane values (k <= 64), as a signed 16-bit key
__device__ inline int wave_kth_largest(int v, int k) {
  uint32_t t = 0;
  const uint32_t b = (uint32_t)(v + 0x8000);
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    if (popc64(__ballot(b >= cand)) >= k) t = cand;
  }
  return (int)t - 0x8000;
}

__device__ inline int count_ge(const u32x4 (&v)[kVec], int te) {
  // tokens of this lane with key >= te, counted on packed pairs
  const s16x2 t2 = (s16x2)((short)te);
  s16x2 acc = (s16x2)((short)0);
#pragma unroll
  for (int q = 0; q < kVec * 4; ++q) {
    // copy the element to a scalar first: __builtin_bit_cast applied directly
    // to an ext-vector element reads element 0 with this compiler
    const uint32_t w = v[q >> 2][q & 3];
    const s16x2 kq = __builtin_bit_cast(s16x2, w);
    acc += __builtin_elementwise_sub_sat(kq, t2) >> 15;  // -1 where key < te
  }
  return 2 * kVec * 4 + acc.x + acc.y;
}

// One tile: keys in place, the first-tile bound, then candidate insertion one
// dword (two logits per lane) at a time.
template <bool kInterior>
__device__ inline void tile_process(WaveState& s, u32x4 (&v)[kVec], int tile, int head, int V) {
  const int lane = __lane_id();
  const int tile_pos = tile * kTile;
  const int lm = tile_keys<kInterior>(v, tile, head, V, s.magmax);
  if (tile == 0) s.thr = wave_kth_largest(lm, s.k);
  // valid keys are >= -0x7FFF; positions outside the row hold -0x8000
  int te = max(s.strict ? s.thr + 1 : s.thr, -0x7FFF);
  const uint64_t lanes = __ballot(lm >= te);
  if (!lanes) return;
  if (s.n + popc64(lanes) * (kVec * 8) > kCap) {
    int c = lm >= te ? count_ge(v, te) : 0;
    for (int off = kWave / 2; off > 0; off >>= 1) c += __shfl_xor(c, off, kWave);
    if (s.n + c > kCap) {
      if (s.n >= s.k) {
        int kth;
        s.n = region_cut(s.reg, s.n, s.k, &kth);
        s.thr = kth;
        s.strict = true;
        te = max(kth + 1, -0x7FFF);
        c = lm >= te ? count_ge(v, te) : 0;
        for (int off = kWave / 2; off > 0; off >>= 1) c += __shfl_xor(c, off, kWave);
      }
      if (s.n + c > kCap) {
        s.overflow = true;
        return;
      }
    }
  }
  // sign bits of the saturated difference key - te mark the tokens below te
  const s16x2 te2 = (s16x2)((short)te);
#pragma unroll
  for (int q = 0; q < kVec * 4; ++q) {
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t kq = v[q >> 2][q & 3];
    const uint32_t below =
        __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(s16x2, kq), te2)) &
        0x80008000u;
    const bool plo = (below & 0x8000u) == 0, phi = (below >> 31) == 0;
    const uint64_t mlo = __ballot(plo), mhi = __ballot(phi);
    if (mlo | mhi) {
      const int p = tile_pos + ((q >> 2) * kWave + lane) * 8 + 2 * (q & 3) - head;
      const int nlo = popc64(mlo);
      const int rlo = __builtin_amdgcn_mbcnt_hi((uint32_t)(mlo >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mlo, 0));
      const int rhi = __builtin_amdgcn_mbcnt_hi((uint32_t)(mhi >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mhi, 0));
      if (plo) s.reg[s.n + rlo] = composite(lo16(kq), (uint32_t)p);
      if (phi) s.reg[s.n + nlo + rhi] = composite(hi16(kq), (uint32_t)(p + 1));
      s.n += nlo + popc64(mhi);
    }
  }
}

// bitonic sort of one u64 per lane, largest first
__device__ inline uint64_t wave_sort_desc(uint64_t x) {
  const int lane = __lane_id();
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t y = __shfl_xor(x, stride, kWave);
      const bool up = (lane & size) == 0;         // this block sorts descending
      const bool lower = (lane & stride) == 0;    // I hold the first slot
      const bool take_max = (lower == up);
      x = take_max ? (x > y ? x : y) : (x < y ? x : y);
    }
  }
  return x;
}

__device__ inline double wave_incl_scan_f64(double v) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// The row's profile from its candidates: exactly the k best, sorted (one per
// lane), then the BAD_LOGITS checks, temperature and top-p (SDCP Sec. 4.1).
__device__ __noinline__ void row_finish(WaveState& s, int k, bool one_hot, const sv_sampling& smp,
                                        int32_t x, RowRec* rec) {
  const int lane = __lane_id();
  int kth;
  const int n = region_cut(s.reg, s.n, k, &kth);
  uint64_t e = lane < n ? s.reg[lane] : 0ull;
  e = wave_sort_desc(e);

  uint32_t mm = s.magmax;
  for (int off = kWave / 2; off > 0; off >>= 1) mm = max_u16x2(mm, __shfl_xor(mm, off, kWave));
  const int magmax = max((int)(mm & 0xFFFFu), (int)(mm >> 16));
  const uint64_t top = __shfl(e, 0, kWave);
  const int kmax = comp_key(top);
  // NaN anywhere, +inf at the top, or no finite logit at all
  const bool bad = magmax > 0x7F80 || kmax >= 0x7F80 || kmax <= -0x7F80;

  RowRec r;
  r.status = bad ? SV_S_BAD_LOGITS : 0;
  r.argmax = (int32_t)comp_id(top);
  r.pad = 0;
  r.lmax = key_value(kmax);
  r.ptok = -1.0;
  if (bad || one_hot) {
    r.kcut = (uint32_t)(kmax + 0x8000);
    r.idcut = r.argmax;
    r.scale = 0.0;
    r.zsum = 1.0;
    if (x >= 0 && !bad) r.ptok = (x == r.argmax) ? 1.0 : 0.0;
  } else {
    // top-k: the candidates that are finite (at most k of them); weights
    // exp((l - lmax) / T); top-p on the renormalised top-k distribution
    const double scale = 1.4426950408889634074 * 1000.0 / (double)smp.temperature_milli;
    const bool live = lane < n && comp_key(e) > -0x7F80;
    const int kept = popc64(__ballot(live));
    const double w = live ? exp2(((double)key_value(comp_key(e)) - (double)r.lmax) * scale) : 0.0;
    const double C = wave_incl_scan_f64(w);
    const double Zk = __shfl(C, kept - 1, kWave);
    int cut = kept;
    if (smp.top_p_milli < 1000) {
      const double tgt = (double)smp.top_p_milli * Zk;
      const uint64_t hit = __ballot(live && 1000.0 * C >= tgt);
      cut = hit ? __builtin_ctzll(hit) + 1 : kept;
    }
    const double zsum = __shfl(C, cut - 1, kWave);
    const uint64_t last = __shfl(e, cut - 1, kWave);
    r.kcut = (uint32_t)(comp_key(last) + 0x8000);
    r.idcut = (int32_t)comp_id(last);
    r.scale = scale;
    r.zsum = zsum;
    if (x >= 0) {
      const uint64_t hitx = __ballot(lane < cut && comp_id(e) == (uint32_t)x);
      const int jx = hitx ? __builtin_ctzll(hitx) : 0;
      const double wx = __shfl(w, jx, kWave);
      r.ptok = hitx ? wx / zsum : 0.0;
    }
  }
  if (lane == 0) *rec = r;
}

__global__ __launch_bounds__(kWave * kWavesPerBlock) void k_rows_topk(
    const uint16_t* __restrict__ target, const uint16_t* __restrict__ draft,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling,
    const int32_t* __restrict__ sess_status, int B, int M, int V, RowRec* __restrict__ rows) {
  __shared__ uint64_t region[kWavesPerBlock][kCap];
  const int wave = threadIdx.x / kWave;
  const int lane = __lane_id();
  const int R = 2 * M + 1;
  const long slot_g = (long)blockIdx.x * kWavesPerBlock + wave;
  const int b = (int)(slot_g / R);
  const int slot = (int)(slot_g - (long)b * R);
  if (b >= B || sess_status[b] != 0) return;
  const int mb = m[b];
  const int rl = rule[b];
  const bool is_target = slot <= M;
  const int i = is_target ? slot + 1 : slot - M;
  if (is_target ? (i > mb + 1) : (rl != SV_RULE_SPECULATIVE || i > mb)) return;
  const sv_sampling smp = sampling[b];
  if (!row_uses_topk_kernel(SV_BF16, rl, smp)) return;
  const bool one_hot = rl == SV_RULE_GREEDY || smp.temperature_milli == 0;
  const int k = one_hot ? 1 : (int)smp.top_k;
  const int32_t x = i <= mb ? tokens[(size_t)b * M + (i - 1)] : -1;
  const uint16_t* row = is_target ? target + ((size_t)b * (M + 1) + (i - 1)) * (size_t)V
                                  : draft + ((size_t)b * M + (i - 1)) * (size_t)V;
  RowRec* rec = rows + (size_t)b * R + slot;

  // 16-byte aligned window over the row: positions [head, head + V) are the row
  const int head = (int)(((uintptr_t)row & 15u) >> 1);
  const u32x4* vbase = (const u32x4*)(row - head);
  const int npos = head + V;
  const int nvec = (npos + 7) / 8;
  const int ntiles = (npos + kTile - 1) / kTile;

  WaveState s;
  s.reg = region[wave];
  s.n = 0;
  s.k = k;
  s.thr = -0x8000;
  s.strict = false;
  s.overflow = false;
  s.magmax = 0;

  // tiles fully inside the row take the unmasked path
  const int t_first_full = (head + kTile - 1) / kTile;
  const int t_end_full = (head + V) / kTile;
  u32x4 va[kVec], vb[kVec];
  load_tile_any(va, vbase, 0, nvec);
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 1 < ntiles) load_tile_any(vb, vbase, t + 1, nvec);
    if (t >= t_first_full && t < t_end_full) tile_process<true>(s, va, t, head, V);
    else tile_process<false>(s, va, t, head, V);
    if (t + 1 >= ntiles || s.overflow) break;
    if (t + 2 < ntiles) load_tile_any(va, vbase, t + 2, nvec);
    if (t + 1 >= t_first_full && t + 1 < t_end_full) tile_process<true>(s, vb, t + 1, head, V);
    else tile_process<false>(s, vb, t + 1, head, V);
    if (s.overflow) break;
  }
  if (s.overflow) {
    if (lane == 0) {
      RowRec r{};
      r.status = kRowFallback;
      *rec = r;
    }
    return;
  }
  row_finish(s, k, one_hot, smp, x, rec);
}

}  // namespace

void launch_rows_topk(const LaunchArgs& a, hipStream_t st) {
  if (a.dtype != SV_BF16) return;
  const size_t slots = (size_t)a.B * (2 * a.M + 1);
  const unsigned grid = (unsigned)((slots + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(k_rows_topk, dim3(grid), dim3(kWave * kWavesPerBlock), 0, st,
                     (const uint16_t*)a.target, (const uint16_t*)a.draft, a.tokens, a.m, a.rule,
                     a.sampling, a.sess_status, a.B, a.M, a.V, a.rows);
}

}  // namespace sv
