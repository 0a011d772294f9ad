// Per-query top-k selection over the visible indexer scores, with lowering of the chosen
// local indices to rows of the concatenated compressed buffer.
//
// "DeepSeek-V4 Attention Training Systems": top-k is a discrete per-query choice that the
// language-model loss does not train (section 3); the fused stack uses a radix top-k with
// a fixed-capacity, alignment-padded index list of global rows (sections 8.1, 8.2).
//
// Kernel design (gfx950): scores become order-preserving 32-bit keys (-0 folded into +0);
// an MSB-first radix select over 8-bit digits finds the exact k-th largest key, and one
// ordered pass emits every key above it plus the first `need` keys equal to it in
// ascending j order (ties go to the smaller j), so the output rows come out sorted and the
// kernels are deterministic.  Rows of up to 4096 visible scores take one wave each (keys
// in registers, no barriers); longer rows take a 512-lane workgroup.  No MFMA: the work is
// integer compare/count, bound by the one HBM read of the scores.
#include "attn_common.h"
#include "csa_launch.h"
#include "topk_wave.h"

namespace csa {

using attn::token_info_wave;

constexpr int kTopkSub = 8;   // sub-histograms per wave

// One workgroup of kTopkThreads lanes per query row for rows longer than a wave holds (see
// topk_row_wg), reading the row from HBM.
template <int KPL>
__global__ __launch_bounds__(kTopkThreads) void k_topk_wg(const float* __restrict__ scores,
                                                          int64_t ld, const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ cu_cmp, int B,
                                                          int r, int n_cap, int k, int k_cap,
                                                          int32_t* __restrict__ idx) {
  __shared__ TopkWgLds<KPL> sm;
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  int32_t* out = idx + (int64_t)t * k_cap;
  TokenInfo ti;
  const bool real = token_info(cu, B, t, ti);
  const int nv = real ? min((ti.p + 1) / r, n_cap) : 0;  // n_cap clamp keeps reads in the row
  const int row0 = real ? cu_cmp[ti.b] : 0;
  if (nv <= k) {  // every visible row is selected (also covers padding rows: nv = 0)
    for (int c = tid; c < k_cap; c += kTopkThreads) out[c] = c < nv ? row0 + c : -1;
    return;
  }
  const int n_it = (nv + kTopkThreads - 1) / kTopkThreads;
  topk_row_wg<KPL>(scores + (int64_t)t * ld, nv, n_it, k, row0, out, sm, nullptr);
  for (int c = k + tid; c < k_cap; c += kTopkThreads) out[c] = -1;
}

// One wave per query row for rows of up to 64 * KPL visible scores (no workgroup barriers):
// keys live in registers lane-interleaved (j = lane + 64 i); each 8-bit radix pass counts
// the keys matching the prefix into a wave-private LDS histogram split eight ways by lane
// (fewer same-address atomic collisions), the wave scans it from the top digit down and
// picks the digit holding the k-th largest key.  The ordered output pass walks the keys in
// j order 64 at a time: ballots give every lane its output position, so each step writes a
// contiguous run of selected rows (ascending, ties to the smaller j).  Rows are dispatched
// to a register footprint of 16, 32, 48 or 64 keys per lane by their visible count.  The
// register budget is held to three waves per SIMD: a wave waits ~5 us for its row to
// arrive from HBM, and three resident waves hide more of it than two (a few keys of the
// 64-key footprint then live in scratch; measured 0.268 -> 0.222 ms at 64K THD).
template <int KPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_topk_wave(const float* __restrict__ scores, int64_t ld,
                                                   const int32_t* __restrict__ cu,
                                                   const int32_t* __restrict__ cu_cmp, int B,
                                                   int r, int n_cap, int k, int k_cap, int T,
                                                   int32_t* __restrict__ idx) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[4][kTopkSub * kHistStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int32_t* out = idx + (int64_t)t * k_cap;
  TokenInfo ti;
  const bool real = token_info_wave(cu, B, t, ti);
  const int nv = real ? min((ti.p + 1) / r, n_cap) : 0;
  const int row0 = real ? cu_cmp[ti.b] : 0;
  if (nv <= k) {  // every visible row is selected (also covers padding rows: nv = 0)
    for (int c = lane; c < k_cap; c += 64) out[c] = c < nv ? row0 + c : -1;
    return;
  }
  const int n_it = __builtin_amdgcn_readfirstlane((nv + 63) >> 6);
  const float* row = scores + (int64_t)t * ld;
  if (KPL >= 16 && n_it <= 16) topk_row_wave<16, kTopkSub>(row, nv, n_it, k, row0, out, hist_all[wave], nullptr);
  else if (KPL >= 32 && n_it <= 32) topk_row_wave<32, kTopkSub>(row, nv, n_it, k, row0, out, hist_all[wave], nullptr);
  else if (KPL >= 48 && n_it <= 48) topk_row_wave<48, kTopkSub>(row, nv, n_it, k, row0, out, hist_all[wave], nullptr);
  else topk_row_wave<(KPL > 48 ? 64 : KPL), kTopkSub>(row, nv, n_it, k, row0, out, hist_all[wave], nullptr);
  for (int c = k + lane; c < k_cap; c += 64) out[c] = -1;
}

hipError_t launch_topk(const Shape& sh, const float* scores, int64_t ld, int32_t* idx,
                       hipStream_t s) {
  if (sh.T == 0) return hipSuccess;
  {
    const int n_cap = sh.max_seqlen / sh.r;
    const dim3 grid((sh.T + 3) / 4), block(256);
    if (n_cap <= 64 * 16) {
      hipLaunchKernelGGL(k_topk_wave<16>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B,
                         sh.r, n_cap, sh.k, sh.k_cap, sh.T, idx);
      return hipGetLastError();
    }
    if (n_cap <= 64 * 32) {
      hipLaunchKernelGGL(k_topk_wave<32>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B,
                         sh.r, n_cap, sh.k, sh.k_cap, sh.T, idx);
      return hipGetLastError();
    }
    if (n_cap <= 64 * 64) {
      hipLaunchKernelGGL(k_topk_wave<64>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B,
                         sh.r, n_cap, sh.k, sh.k_cap, sh.T, idx);
      return hipGetLastError();
    }
  }
  const int n_cap = sh.max_seqlen / sh.r;
  const dim3 grid(sh.T), block(kTopkThreads);
  if (n_cap <= 16 * kTopkThreads)
    hipLaunchKernelGGL(k_topk_wg<16>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B, sh.r,
                       n_cap, sh.k, sh.k_cap, idx);
  else if (n_cap <= 32 * kTopkThreads)
    hipLaunchKernelGGL(k_topk_wg<32>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B, sh.r,
                       n_cap, sh.k, sh.k_cap, idx);
  else
    hipLaunchKernelGGL(k_topk_wg<64>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B, sh.r,
                       n_cap, sh.k, sh.k_cap, idx);
  return hipGetLastError();
}

}  // namespace csa
