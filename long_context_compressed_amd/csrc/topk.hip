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

constexpr int kTopkThreads = 512;
constexpr int kTopkSub = 8;   // sub-histograms per wave

// One workgroup of 512 lanes per query row for rows longer than a wave holds (up to
// 64 KPL keys per lane, lane-interleaved j = tid + 512 i, so the loads coalesce).  Same
// selection as the wave kernel: the radix starts at the highest bit where the row's keys
// differ and stops once the k-th digit is taken whole; each wave counts into its own two
// padded sub-histograms and wave 0 sums them and picks the digit.  The ordered output
// needs every lane's position among the selected keys in j order: per (step i, wave) the
// counts of keys above and equal to the threshold are packed into one word, one exclusive
// scan over the 8 n_it words gives each (i, wave) its base, and ballots give the lane
// offsets, so the output pass runs without barriers.
template <int KPL>
__global__ __launch_bounds__(kTopkThreads) void k_topk_wg(const float* __restrict__ scores,
                                                          int64_t ld, const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ cu_cmp, int B,
                                                          int r, int n_cap, int k, int k_cap,
                                                          int32_t* __restrict__ idx) {
  constexpr int NW = kTopkThreads / 64;
  __shared__ __attribute__((aligned(16))) uint32_t hist[NW][2 * kHistStride];
  __shared__ uint32_t cnt[KPL * NW];
  __shared__ uint32_t red[2][NW], wtot[NW], pick[3];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const float* row = scores + (int64_t)t * ld;

  // every load is issued before the first use (indexes clamped into the row)
  float v[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i)
    if (i < n_it) v[i] = row[min(tid + kTopkThreads * i, nv - 1)];
  uint32_t key[KPL];
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    key[i] = 0u;                                  // 0 is below every real key
    if (i < n_it) {
      const uint32_t u = __float_as_uint(v[i] + 0.0f);   // -0 + 0 = +0
      const uint32_t kk = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
      key[i] = tid + kTopkThreads * i < nv ? kk : 0u;
    }
    kmax = max(kmax, key[i]);
    kmin = min(kmin, key[i] ? key[i] : 0xffffffffu);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
  }
  if (lane == 0) {
    red[0][wave] = kmax;
    red[1][wave] = kmin;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmax = max(kmax, red[0][w]);
    kmin = min(kmin, red[1][w]);
  }

  uint32_t prefix, pmask, need = (uint32_t)k, in_digit = 0;
  int shift;
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0u) {            // every visible key is equal: the first k in j order
    prefix = kmax;
    pmask = 0xffffffffu;
    shift = -1;
  } else {
    const int hb = 31 - __builtin_clz(diff);
    pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
    prefix = kmax & pmask;
    shift = max(hb - 7, 0);
  }
  uint32_t* my = &hist[wave][(lane & 1) * kHistStride];
  bool first = true;
#pragma unroll 1
  while (shift >= 0) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<uint4*>(&hist[wave][q * kHistStride + 4 * lane]) = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
    if (first) {   // padding keys (0) land in digit 0 and are taken off below
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (i < n_it) atomicAdd(&my[(key[i] >> shift) & 255u], 1u);
    } else if (prefix != 0u) {
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (i < n_it && (key[i] & pmask) == prefix) atomicAdd(&my[(key[i] >> shift) & 255u], 1u);
    } else {
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (i < n_it && key[i] != 0u && (key[i] & pmask) == prefix)
          atomicAdd(&my[(key[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane covers digits 255-4*lane .. 252-4*lane (descending digit order)
      uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 2 * NW; ++q) {
        const uint4 x = *reinterpret_cast<const uint4*>(
            &hist[q >> 1][(q & 1) * kHistStride + 4 * (63 - lane)]);
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
      }
      if (first && lane == 63) acc.x -= (uint32_t)(kTopkThreads * n_it - nv);
      const uint32_t c[4] = {acc.w, acc.z, acc.y, acc.x};
      const uint32_t s = c[0] + c[1] + c[2] + c[3];
      uint32_t run = wave_incl_scan(s) - s;   // keys with a larger digit than this lane's
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run < need && run + c[q] >= need) {
          pick[0] = 255u - (uint32_t)(4 * lane + q);
          pick[1] = run;
          pick[2] = c[q];
        }
        run += c[q];
      }
    }
    __syncthreads();
    const uint32_t digit = pick[0];
    need -= pick[1];
    in_digit = pick[2];
    prefix |= digit << shift;
    pmask |= 255u << shift;
    first = false;
    if (in_digit == need || shift == 0) break;   // the whole digit is taken, or exact key
    shift = max(shift - 8, 0);
  }

  // selected: keys whose masked value exceeds the prefix, plus the first `need` equal to it
  const uint32_t thr = prefix;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (i < n_it) {
      const uint32_t m = key[i] & pmask;
      const uint64_t bg = __ballot(key[i] != 0u && m > thr);
      const uint64_t be = __ballot(key[i] != 0u && m == thr);
      if (lane == 0) cnt[i * NW + wave] = (uint32_t)__popcll(bg) | ((uint32_t)__popcll(be) << 16);
    }
  }
  __syncthreads();
  {
    const uint32_t x = tid < n_it * NW ? cnt[tid] : 0u;
    const uint32_t incl = wave_incl_scan(x);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t before = incl - x;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    if (tid < n_it * NW) cnt[tid] = before;
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (i < n_it) {
      const uint32_t m = key[i] & pmask;
      const bool gt = key[i] != 0u && m > thr;
      const bool eq = key[i] != 0u && m == thr;
      const uint32_t base = cnt[i * NW + wave];
      const uint32_t gt_before = (base & 0xffffu) + lanes_below(__ballot(gt));
      const uint32_t eq_before = (base >> 16) + lanes_below(__ballot(eq));
      if (gt || (eq && eq_before < need))
        out[gt_before + min(eq_before, need)] = row0 + tid + kTopkThreads * i;
    }
  }
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
