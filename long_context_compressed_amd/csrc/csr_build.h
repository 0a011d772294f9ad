// Compressed-row CSR of a chunk of queries (row -> the (query, slot) pairs that attend it),
// built in a count pass and, after an exclusive scan of the counts, a fill pass.  Shared by
// the attention backward and the indexer-loss backward, whose owner-side reductions read it
// ("DeepSeek-V4 Attention Training Systems", section 3 gradient ownership: every
// compressed row's gradient is the sum over the queries that selected it).
//
// A workgroup takes kCsrGroup consecutive queries.  Neighbouring queries of one sample
// select largely the same rows (all of them while n_vis <= k), so the pairs are first
// counted in an LDS histogram over the group's row span and each touched row then costs
// one global atomic per workgroup instead of one per pair; the fill pass reserves each
// row's range with that atomic and places the pairs by LDS atomics.  A group whose rows
// span more than kCsrSpan (it straddles samples, or samples are very long) falls back to
// one global atomic per pair.  The order of the pairs within a row's list is not fixed.
#pragma once

#include "csa_device.h"

namespace csa {

struct CsrBuild {
  const int32_t* idx;   // [T, k_cap] selected global rows, or null: slot s is visible row s
  const int32_t* cu;
  const int32_t* cu_cmp;
  const int32_t* nc;    // [T] candidate slots of each query
  int32_t* cnt;         // [rows] pair counts (count pass, +=; zeroed by the caller)
  int32_t* cur;         // [rows] next free list position (fill pass; the row offsets)
  int32_t* list;        // [pairs] (query - t0) * slots + slot
  int64_t slots;
  int t0, nT, B, r, n_cap, k_cap;
};

constexpr int kCsrGroup = 16;    // queries per workgroup
constexpr int kCsrSpan = 4096;   // compressed rows a workgroup counts in LDS

inline int csr_grid(int nT) { return (nT + kCsrGroup - 1) / kCsrGroup; }

// Workgroup of 256 lanes; blockIdx.x = query group.
template <bool FILL>
__device__ __forceinline__ void csr_group_pass(const CsrBuild& c) {
  __shared__ int32_t hist[kCsrSpan];
  __shared__ int32_t base[FILL ? kCsrSpan : 1];
  __shared__ int32_t q_row0[kCsrGroup], q_nv[kCsrGroup], q_n[kCsrGroup];
  __shared__ int32_t s_lo, s_hi;
  const int tid = threadIdx.x;
  const int g0 = blockIdx.x * kCsrGroup;
  if (tid == 0) {
    s_lo = 0x7fffffff;
    s_hi = -0x7fffffff;
  }
  __syncthreads();
  if (tid < kCsrGroup) {
    const int tl = g0 + tid;
    int row0 = 0, nv = 0, n = 0;
    TokenInfo ti;
    if (tl < c.nT && token_info(c.cu, c.B, c.t0 + tl, ti)) {
      row0 = c.cu_cmp[ti.b];
      nv = min((ti.p + 1) / c.r, c.n_cap);
      n = nv > 0 ? c.nc[c.t0 + tl] : 0;
      if (n > 0) {
        atomicMin(&s_lo, row0);
        atomicMax(&s_hi, row0 + nv);
      }
    }
    q_row0[tid] = row0;
    q_nv[tid] = nv;
    q_n[tid] = n;
  }
  __syncthreads();
  const int lo = s_lo, span = s_hi - s_lo;
  if (span <= 0) return;                       // no pair in the group (uniform)
  // global row of slot s of group query q, or -1 outside its visible range
  auto row_of = [&](int q, int s) {
    const int row0 = q_row0[q], nv = q_nv[q];
    const int gr = c.idx ? c.idx[(int64_t)(c.t0 + g0 + q) * c.k_cap + s] : row0 + s;
    return (gr >= row0 && gr < row0 + nv) ? gr : -1;
  };
  if (span > kCsrSpan) {                       // uniform: one global atomic per pair
    for (int q = 0; q < kCsrGroup; ++q)
      for (int s = tid; s < q_n[q]; s += 256) {
        const int gr = row_of(q, s);
        if (gr < 0) continue;
        if (!FILL) {
          atomicAdd(&c.cnt[gr], 1);
        } else {
          const int pos = atomicAdd(&c.cur[gr], 1);
          c.list[pos] = (g0 + q) * (int32_t)c.slots + s;
        }
      }
    return;
  }
  // every valid pair (q, s, row) of the group, f(q, s, row); the slots of kQB queries x kSI
  // slots per lane are loaded together, so a lane waits for one load latency per batch
  // instead of one per slot
  int n_max = 0;
  for (int q = 0; q < kCsrGroup; ++q) n_max = max(n_max, q_n[q]);
  auto for_pairs = [&](auto&& f) {
    constexpr int kQB = 4, kSI = 4;
    for (int q0 = 0; q0 < kCsrGroup; q0 += kQB)
      for (int sb = 0; sb < n_max; sb += 256 * kSI) {
        int gr[kQB][kSI];
#pragma unroll
        for (int j = 0; j < kQB; ++j)
#pragma unroll
          for (int i = 0; i < kSI; ++i) {
            const int s = sb + tid + 256 * i;
            gr[j][i] = s < q_n[q0 + j] ? row_of(q0 + j, s) : -1;
          }
#pragma unroll
        for (int j = 0; j < kQB; ++j)
#pragma unroll
          for (int i = 0; i < kSI; ++i)
            if (gr[j][i] >= 0) f(q0 + j, sb + tid + 256 * i, gr[j][i]);
      }
  };
  for (int i = tid; i < span; i += 256) hist[i] = 0;
  __syncthreads();
  for_pairs([&](int, int, int gr) { atomicAdd(&hist[gr - lo], 1); });
  __syncthreads();
  if (!FILL) {
    for (int i = tid; i < span; i += 256) {
      const int v = hist[i];
      if (v) atomicAdd(&c.cnt[lo + i], v);
    }
    return;
  }
  for (int i = tid; i < span; i += 256) {
    const int v = hist[i];
    if (v) base[i] = atomicAdd(&c.cur[lo + i], v);
    hist[i] = 0;
  }
  __syncthreads();
  for_pairs([&](int q, int s, int gr) {
    const int pos = base[gr - lo] + atomicAdd(&hist[gr - lo], 1);
    c.list[pos] = (g0 + q) * (int32_t)c.slots + s;
  });
}

}  // namespace csa
