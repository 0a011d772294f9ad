// Wave-level radix top-k of one query row, shared by the stand-alone top-k and the fused
// indexer-scores + top-k kernels ("DeepSeek-V4 Attention Training Systems", section 3
// selection; ties go to the smaller index).
#pragma once

#include "csa_device.h"

namespace csa {

// Keys: u = bits of (score + 0) (so -0 becomes +0), key = u ^ (sign ? 0xffffffff : 0x80000000),
// ascending in the score; key_value inverts it.
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Number of set bits of a wave mask below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Sub-histogram stride in 32-bit words: 256 digits plus 4 words, so the same digit of
// sub-histograms s and s' falls in different LDS banks.
constexpr int kHistStride = 260;
constexpr int kTopkThreads = 512;   // lanes of the workgroup top-k (rows beyond 4096 keys)

// One wave per query row of up to 64 * KPL visible scores (no workgroup barriers).  Keys
// live in registers lane-interleaved (j = lane + 64 i).  The radix select starts at the
// highest bit in which the row's keys differ (bits above it are common to all keys), takes
// 8-bit digits from there down, and counts the keys matching the prefix found so far into
// NSUB wave-private LDS sub-histograms (lane % NSUB picks one, fewer same-address atomic
// collisions).  The wave scans the histogram from the top digit and keeps the digit that
// holds the k-th largest key; it stops early once every key of that digit is selected.
// The ordered output pass walks the keys in j order 64 at a time: ballots give every lane
// its output position, so each step writes a contiguous run of selected rows (ascending,
// ties to the smaller j).
// Rows of nv (> k) visible scores, n_it = ceil(nv / 64) <= KPL keys per lane; `row` may be
// global or LDS and is read before `hist` (NSUB * kHistStride words) is first written, so
// the two may share storage.  When sel is non-null the score of every selected j is also
// stored to sel[j].
template <int KPL, int NSUB>
__device__ __forceinline__ void topk_row_wave(const float* __restrict__ row, int nv, int n_it,
                                              int k, int row0, int32_t* __restrict__ out,
                                              uint32_t* hist, float* __restrict__ sel) {
  const int lane = threadIdx.x & 63;
  uint32_t key[KPL];
  uint32_t kmax = 0u, kmin = 0xffffffffu;
  // every load is issued before the first use: the index is clamped into the row instead of
  // guarding each load with a per-lane branch (which would wait for each load in turn)
  float v[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i)
    if (i < n_it) v[i] = row[min(lane + 64 * i, nv - 1)];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    key[i] = 0u;                                  // 0 is below every real key
    if (i < n_it) {
      const uint32_t u = __float_as_uint(v[i] + 0.0f);   // -0 + 0 = +0
      const uint32_t kk = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
      key[i] = lane + 64 * i < nv ? kk : 0u;
    }
    kmax = max(kmax, key[i]);
    kmin = min(kmin, key[i] ? key[i] : 0xffffffffu);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
  }
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  kmin = __builtin_amdgcn_readfirstlane(kmin);
  __builtin_amdgcn_wave_barrier();

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
  uint32_t* my = hist + (lane % NSUB) * kHistStride;
  bool first = true;
#pragma unroll 1
  while (shift >= 0) {
#pragma unroll
    for (int q = 0; q < NSUB; ++q)
      *reinterpret_cast<uint4*>(&hist[q * kHistStride + 4 * lane]) = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
    if (first) {
      // every visible key shares the bits above the first digit; the 64 n_it - nv padding
      // keys (0) land in digit 0 and are taken off below
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (i < n_it) atomicAdd(&my[(key[i] >> shift) & 255u], 1u);
    } else if (prefix != 0u) {  // a padding key (0) cannot match a nonzero prefix
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (i < n_it && (key[i] & pmask) == prefix) atomicAdd(&my[(key[i] >> shift) & 255u], 1u);
    } else {
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (i < n_it && key[i] != 0u && (key[i] & pmask) == prefix)
          atomicAdd(&my[(key[i] >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    // lane covers digits 255-4*lane .. 252-4*lane (descending digit order)
    uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < NSUB; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(&hist[q * kHistStride + 4 * (63 - lane)]);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (first && lane == 63) acc.x -= (uint32_t)(64 * n_it - nv);
    const uint32_t c[4] = {acc.w, acc.z, acc.y, acc.x};
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    uint32_t run = wave_incl_scan(s) - s;   // keys with a larger digit than this lane's
    int hit = -1;
    uint32_t above = 0, cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (hit < 0 && run < need && run + c[q] >= need) { hit = q; above = run; cnt = c[q]; }
      run += c[q];
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t bal = __ballot(hit >= 0);
    const int src = __ffsll((unsigned long long)bal) - 1;
    const uint32_t digit = 255u - (uint32_t)(4 * src + __shfl(hit, src, 64));
    need -= (uint32_t)__shfl((int)above, src, 64);
    in_digit = (uint32_t)__shfl((int)cnt, src, 64);
    prefix |= digit << shift;
    pmask |= 255u << shift;
    first = false;
    if (in_digit == need || shift == 0) break;   // the whole digit is taken, or exact key
    shift = max(shift - 8, 0);
  }
  // selected: keys whose masked value exceeds the prefix, plus the first `need` equal to it
  const uint32_t thr = prefix;
  uint32_t base = 0;
  if (in_digit == need && thr != 0u) {
    // no tie to break (every key equal to the prefix is taken) and padding keys fall below
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      if (i < n_it) {
        const bool take = (key[i] & pmask) >= thr;
        const uint64_t bt = __ballot(take);
        if (take) {
          out[base + lanes_below(bt)] = row0 + lane + 64 * i;
          if (sel) sel[lane + 64 * i] = key_value(key[i]);
        }
        base += (uint32_t)__popcll(bt);
      }
    }
    return;
  }
  uint32_t eq_seen = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (i < n_it) {
      const uint32_t m = key[i] & pmask;
      const bool gt = key[i] != 0u && m > thr;
      const bool eq = key[i] != 0u && m == thr;
      const uint64_t beq = __ballot(eq);
      const uint32_t eq_before = eq_seen + lanes_below(beq);
      const bool take = gt || (eq && eq_before < need);
      const uint64_t bt = __ballot(take);
      if (take) {
        out[base + lanes_below(bt)] = row0 + lane + 64 * i;
        if (sel) sel[lane + 64 * i] = key_value(key[i]);
      }
      base += (uint32_t)__popcll(bt);
      eq_seen += (uint32_t)__popcll(beq);
    }
  }
}

// One workgroup of kTopkThreads lanes per query row for rows longer than a wave holds (up to
// KPL keys per lane, lane-interleaved j = tid + 512 i, so the loads coalesce).  Same
// selection as the wave kernel: the radix starts at the highest bit where the row's keys
// differ and stops once the k-th digit is taken whole; each wave counts into its own two
// padded sub-histograms and wave 0 sums them and picks the digit.  The ordered output
// needs every lane's position among the selected keys in j order: per (step i, wave) the
// counts of keys above and equal to the threshold are packed into one word, one exclusive
// scan over the 8 n_it words gives each (i, wave) its base, and ballots give the lane
// offsets, so the output pass runs without barriers.
// `row` (global or LDS) holds the nv (> k) visible scores; it is read before sm.hist is first
// written (after a workgroup barrier), so an LDS row may share storage with sm.  When sel is
// non-null the score of every selected j is also stored to sel[j].  idx entries k .. k_cap
// are left to the caller.
template <int KPL>
struct TopkWgLds {
  static constexpr int NW = kTopkThreads / 64;
  __attribute__((aligned(16))) uint32_t hist[NW][2 * kHistStride];
  uint32_t cnt[KPL * NW];
  uint32_t red[2][NW], wtot[NW], pick[3];
};

template <int KPL>
__device__ __forceinline__ void topk_row_wg(const float* __restrict__ row, int nv, int n_it,
                                            int k, int row0, int32_t* __restrict__ out,
                                            TopkWgLds<KPL>& sm, float* __restrict__ sel) {
  constexpr int NW = kTopkThreads / 64;
  auto& hist = sm.hist;
  auto& cnt = sm.cnt;
  auto& red = sm.red;
  auto& wtot = sm.wtot;
  auto& pick = sm.pick;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
      if (gt || (eq && eq_before < need)) {
        out[gt_before + min(eq_before, need)] = row0 + tid + kTopkThreads * i;
        if (sel) sel[tid + kTopkThreads * i] = key_value(key[i]);
      }
    }
  }
}


}  // namespace csa
