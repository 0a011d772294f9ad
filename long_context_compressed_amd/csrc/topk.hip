// Per-query top-k selection over the visible indexer scores, with lowering of the chosen
// local indices to rows of the concatenated compressed buffer.
//
// "DeepSeek-V4 Attention Training Systems": top-k is a discrete per-query choice that the
// language-model loss does not train (section 3); the fused stack uses a radix top-k with
// a fixed-capacity, alignment-padded index list of global rows (sections 8.1, 8.2).
//
// Kernel design (gfx950): one workgroup of 512 lanes per query row; the visible scores
// are read once from HBM into registers (ITEMS per lane, lane-interleaved so the loads
// coalesce) as order-preserving 32-bit keys.  An MSB-first radix select (4 passes of 8
// bits, LDS histograms) finds the exact k-th largest key; a single ordered pass then
// emits every key above it plus the first `need` keys equal to it in ascending j order
// (ties go to the smaller j), using a packed (greater, equal) block prefix count, so the
// output rows come out sorted and the kernel is deterministic.  No MFMA: the work is
// integer compare/count, bound by the one HBM read of the scores.
#include "attn_common.h"
#include "csa_launch.h"
#include "topk_wave.h"

namespace csa {

using attn::token_info_wave;

constexpr int kTopkThreads = 512;
constexpr int kTopkSub = 8;   // sub-histograms per wave

template <int ITEMS>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ scores,
                                                       int64_t ld, const int32_t* __restrict__ cu,
                                                       const int32_t* __restrict__ cu_cmp, int B,
                                                       int r, int n_cap, int k, int k_cap,
                                                       int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[kTopkThreads / 64];
  __shared__ uint32_t sel_digit, sel_above;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  const float* row = scores + (int64_t)t * ld;
  uint32_t key[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int j = tid + i * kTopkThreads;
    key[i] = j < nv ? order_key(row[j]) : 0u;
  }

  uint32_t prefix = 0, pmask = 0;
  uint32_t need = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int j = tid + i * kTopkThreads;
      if (j < nv && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane covers digits 255-4*lane .. 252-4*lane (descending digit order)
      uint32_t c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = hist[255 - (4 * lane + q)];
      const uint32_t s = c[0] + c[1] + c[2] + c[3];
      uint32_t run = wave_incl_scan(s) - s;   // keys with a larger digit than this lane's
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run < need && run + c[q] >= need) {
          sel_digit = 255u - (uint32_t)(4 * lane + q);
          sel_above = run;
        }
        run += c[q];
      }
    }
    __syncthreads();
    need -= sel_above;
    prefix |= sel_digit << shift;
    pmask |= 255u << shift;
  }
  const uint32_t thr = prefix;  // the k-th largest key; `need` (>= 1) keys equal to it are taken

  uint32_t base_gt = 0, base_eq = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int j = tid + i * kTopkThreads;
    const bool valid = j < nv;
    const bool gt = valid && key[i] > thr;
    const bool eq = valid && key[i] == thr;
    const uint32_t packed = (gt ? 1u : 0u) | (eq ? 0x10000u : 0u);
    const uint32_t incl = wave_incl_scan(packed);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t before = incl - packed, total = 0;
#pragma unroll
    for (int wv = 0; wv < kTopkThreads / 64; ++wv) {
      const uint32_t x = wave_tot[wv];
      if (wv < wave) before += x;
      total += x;
    }
    const uint32_t gt_before = base_gt + (before & 0xffffu);
    const uint32_t eq_before = base_eq + (before >> 16);
    if (gt || (eq && eq_before < need)) {
      const uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
      out[pos] = row0 + j;
    }
    base_gt += total & 0xffffu;
    base_eq += total >> 16;
    __syncthreads();
  }
  for (int c = k + tid; c < k_cap; c += kTopkThreads) out[c] = -1;
}

// One wave per query row for rows of up to 64 * KPL visible scores (no workgroup barriers):
// keys live in registers lane-interleaved (j = lane + 64 i); each 8-bit radix pass counts
// the keys matching the prefix into a wave-private LDS histogram split four ways by lane
// (fewer same-address atomic collisions), the wave scans it from the top digit down and
// picks the digit holding the k-th largest key.  The ordered output pass walks the keys in
// j order 64 at a time: ballots give every lane its output position, so each step writes a
// contiguous run of selected rows (ascending, ties to the smaller j).  Rows are dispatched
// to a register footprint of 16, 32, 48 or 64 keys per lane by their visible count.
template <int KPL>
__global__ __launch_bounds__(256) void k_topk_wave(const float* __restrict__ scores, int64_t ld,
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
  if (sh.T == 0) return hipSuccess;
  const int n_cap = sh.max_seqlen / sh.r;
  const dim3 grid(sh.T), block(kTopkThreads);
  if (n_cap <= 4 * kTopkThreads)
    hipLaunchKernelGGL(k_topk<4>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B, sh.r,
                       n_cap, sh.k, sh.k_cap, idx);
  else if (n_cap <= 16 * kTopkThreads)
    hipLaunchKernelGGL(k_topk<16>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B, sh.r,
                       n_cap, sh.k, sh.k_cap, idx);
  else
    hipLaunchKernelGGL(k_topk<64>, grid, block, 0, s, scores, ld, sh.cu, sh.cu_cmp, sh.B, sh.r,
                       n_cap, sh.k, sh.k_cap, idx);
  return hipGetLastError();
}

}  // namespace csa
