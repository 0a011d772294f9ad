// Wave-level radix top-k of one query row, shared by the stand-alone top-k and the fused
// indexer-scores + top-k kernels ("DeepSeek-V4 Attention Training Systems", section 3
// selection; ties go to the smaller index).
#pragma once

#include "csa_device.h"

namespace csa {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                       // -0 and +0 are the same value
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending float <=> ascending key
}

// One wave per query row of up to 64 * KPL visible scores (no workgroup barriers):
// keys live in registers lane-interleaved (j = lane + 64 i); each 8-bit radix pass counts
// the keys matching the prefix into a wave-private LDS histogram split four ways by lane
// (fewer same-address atomic collisions), the wave scans it from the top digit down and
// picks the digit holding the k-th largest key.  The ordered output pass walks the keys in
// j order 64 at a time: ballots give every lane its output position, so each step writes a
// contiguous run of selected rows (ascending, ties to the smaller j).
// Radix select + ordered output of one row of nv (> k) visible scores, n_it = ceil(nv / 64)
// <= KPL keys per lane.  `row` may be global or LDS; when sel is non-null the score of every
// selected j is also stored to sel[j].
template <int KPL>
__device__ __forceinline__ void topk_row_wave(const float* __restrict__ row, int nv, int n_it,
                                              int k, int row0, int32_t* __restrict__ out,
                                              uint32_t (*hist)[256], float* __restrict__ sel) {
  const int lane = threadIdx.x & 63;
  uint32_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int j = lane + 64 * i;
    key[i] = (i < n_it && j < nv) ? order_key(row[j]) : 0u;   // 0 is below every real key
  }
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  const int sub = lane & 3;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(&hist[q][4 * lane]) = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (key[i] != 0u && (key[i] & pmask) == prefix)
        atomicAdd(&hist[sub][(key[i] >> shift) & 255u], 1u);
    __builtin_amdgcn_wave_barrier();
    // lane covers digits 255-4*lane .. 252-4*lane (descending digit order)
    uint32_t c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 255 - (4 * lane + q);
      c[q] = (hist[0][d] + hist[1][d]) + (hist[2][d] + hist[3][d]);
    }
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    uint32_t run = wave_incl_scan(s) - s;   // keys with a larger digit than this lane's
    int hit = -1;
    uint32_t above = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (hit < 0 && run < need && run + c[q] >= need) { hit = q; above = run; }
      run += c[q];
    }
    const uint64_t bal = __ballot(hit >= 0);
    const int src = __ffsll((unsigned long long)bal) - 1;
    const uint32_t digit = 255u - (uint32_t)(4 * src + __shfl(hit, src, 64));
    need -= __shfl(above, src, 64);
    prefix |= digit << shift;
    pmask |= 255u << shift;
  }
  const uint32_t thr = prefix;  // the k-th largest key; `need` (>= 1) keys equal to it are taken
  uint32_t base = 0, eq_seen = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const bool gt = key[i] > thr;
    const bool eq = key[i] == thr;
    const uint64_t beq = __ballot(eq);
    const uint32_t eq_before = eq_seen + (uint32_t)__popcll(beq & lt_mask);
    const bool take = gt || (eq && eq_before < need);
    const uint64_t bt = __ballot(take);
    if (take) {
      out[base + __popcll(bt & lt_mask)] = row0 + lane + 64 * i;
      if (sel) sel[lane + 64 * i] = row[lane + 64 * i];
    }
    base += (uint32_t)__popcll(bt);
    eq_seen += (uint32_t)__popcll(beq);
  }
}

}  // namespace csa
