// sv_rows_generic.hip -- the generic row kernel: the exact profile of
// sv_rows_exact.hpp, one workgroup of kNT threads per row, for the binary32
// rows with top-p or top-k above 64 (the single-pass kernel takes every other
// row, and profiles a row it hands back itself).
#include <algorithm>

#include "sv_kernels.hpp"
#include "sv_rows_exact.hpp"

namespace sv {

namespace {

constexpr int kNT = 256;


// Does row slot slot_g need this kernel?
// With in-order reading (decided != null) only the window's positions of the
// sessions still undecided.
template <class Tr>
__device__ bool generic_row(int slot_g, const int32_t* m, const int32_t* rule,
                            const sv_sampling* sampling, const int32_t* sess_status, int M, int V,
                            const RowRec* rows, bool draft_logits, const int32_t* decided,
                            int win_lo, int win_w) {
  const int R = 2 * M + 1;
  const int b = slot_g / R;
  const int slot = slot_g - b * R;
  if (sess_status[b] != 0) return false;
  const int mb = m[b];
  const int rl = rule[b];
  const bool is_target = slot <= M;
  const int i = is_target ? slot + 1 : slot - M;  // 1-based position
  if (decided && (i < win_lo || i >= win_lo + win_w || (win_lo > 1 && decided[b] != 0)))
    return false;
  // draft rows are profiled only when draft logits are given (not with q rows)
  if (is_target ? (i > mb + 1) : (rl != SV_RULE_SPECULATIVE || i > mb || !draft_logits))
    return false;
  const sv_sampling smp = sampling[b];
  // the single-pass kernel's rows (a row it hands back, it profiles itself)
  return !row_uses_topk_kernel(Tr::kDtype, rl, smp) &&
         !row_uses_dense_kernel(Tr::kDtype, rl, smp, V);
}

// A grid of at most kMaxBlocks workgroups scans the row slots: each workgroup
// takes an equal share of consecutive slots, kNT at a time; each thread checks
// one slot, the slots that need this kernel are listed in LDS, and the
// workgroup profiles them one after another.
constexpr int kMaxBlocks = 1024;
template <class Tr>
__global__ __launch_bounds__(kNT) void k_rows_generic(
    const typename Tr::elem_t* __restrict__ target, const typename Tr::elem_t* __restrict__ draft,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ m,
    const int32_t* __restrict__ rule, const sv_sampling* __restrict__ sampling,
    const int32_t* __restrict__ sess_status, int B, int M, int V, RowRec* __restrict__ rows,
    uint32_t* __restrict__ draw_flag, uint32_t draw_token, const int32_t* __restrict__ decided,
    int win_lo, int win_w) {
  __shared__ exact::Smem<kNT> sm;
  __shared__ int32_t todo[kNT];
  __shared__ int32_t wave_cnt[kNT / kWave];
  const int R = 2 * M + 1;
  const int slots = B * R;
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  // this workgroup's slots: an equal share, so that few rows spread over many groups
  const int per = (slots + (int)gridDim.x - 1) / (int)gridDim.x;
  const int end = min(slots, ((int)blockIdx.x + 1) * per);
  for (int base = (int)blockIdx.x * per; base < end; base += kNT) {
    const int slot_g = base + (int)threadIdx.x;
    const bool need = slot_g < end &&
                      generic_row<Tr>(slot_g, m, rule, sampling, sess_status, M, V, rows,
                                      draft != nullptr, decided, win_lo, win_w);
    if (need) draw_flag[slot_g / R] = draw_token;  // a row without a listed support
    const uint64_t mask = __ballot(need);
    __syncthreads();  // the previous round's list is consumed
    if (lane == 0) wave_cnt[wid] = __builtin_popcountll(mask);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kNT / kWave; ++w) {
      before += w < wid ? wave_cnt[w] : 0;
      total += wave_cnt[w];
    }
    if (need)
      todo[before + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0))] = slot_g;
    __syncthreads();
    for (int t = 0; t < total; ++t) {
      const int sg = todo[t];
      const int b = sg / R;
      const int slot = sg - b * R;
      const bool is_target = slot <= M;
      const int i = is_target ? slot + 1 : slot - M;
      const int mb = m[b];
      const int32_t x = i <= mb ? tokens[(size_t)b * M + (i - 1)] : -1;
      const typename Tr::elem_t* row =
          is_target ? target + ((size_t)b * (M + 1) + (i - 1)) * (size_t)V
                    : draft + ((size_t)b * M + (i - 1)) * (size_t)V;
      exact::profile_row<Tr, kNT>(row, V, sampling[b], rule[b] == SV_RULE_GREEDY, x, rows + sg,
                                  &sm);
    }
  }
}

}  // namespace

void launch_rows_generic(const LaunchArgs& a, hipStream_t st) {
  // bf16 rows are all profiled by the single-pass kernel (a row it hands back
  // included): no launch
  if (a.dtype == SV_BF16) return;
  const size_t slots = (size_t)a.B * (2 * a.M + 1);
  const unsigned grid = (unsigned)std::min<size_t>(slots, kMaxBlocks);
  {
    hipLaunchKernelGGL(k_rows_generic<F32>, dim3(grid), dim3(kNT), 0, st,
                       (const uint32_t*)a.target, (const uint32_t*)a.draft, a.tokens, a.m, a.rule,
                       a.sampling, a.sess_status, a.B, a.M, a.V, a.rows, a.draw_flag,
                       a.draw_token, a.decided, a.win_lo, a.win_w);
  }
}

}  // namespace sv
