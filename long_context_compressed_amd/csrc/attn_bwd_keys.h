// Key-major accumulation of the shared-row gradients of the attention backward.
//
// Method ("DeepSeek-V4 Attention Training Systems", section 8.2: the backward needs no dense
// matrix; section 3, gradient ownership: a compressed row's gradient is the sum over the
// queries that attend it).  With the per-(query, slot) values scale*dS and P of the 64 heads
// already formed by the dq pass, the gradient of a shared row x is
//   d row_x = sum_t sum_h (scale dS[t,h,x] q[t,h] + P[t,h,x] dO[t,h]),
// a contraction over (query, head, {dS, P}) of the per-query operand [q_t; dO_t]
// (128 x 512).  Here it runs as a dense masked product per work item: a block of up to kb
// consecutive rows of one sample (compressed rows, or raw window rows) against a range of
// up to kCq consecutive queries of that sample; the (query, row) pairs a query does not
// attend contribute zero.  Items of one block write fp32 partial sums that a reduction adds
// in a fixed order, so the result does not depend on scheduling.
//
// This file holds the enumeration of the work items, shared by the device planner and the
// host bound on their number.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define CSA_HD __host__ __device__
#else
#define CSA_HD
#endif

namespace csa {
namespace keys {

constexpr int kKeysMax = 256;   // rows per item: kb = 128 (attention) or 256 (indexer keys)
constexpr int kCq = 256;     // queries per item

// Item kinds: compressed rows of a CSA_SPARSE layer (slots found in the idx row), compressed
// rows of a CSA_DENSE layer (slot = visible row), raw window rows.
constexpr int kKindSel = 0, kKindDense = 1, kKindWin = 2;

// One sample's share of a backward query chunk: local query positions [pa, pb).
struct SampleChunk {
  int s0, L, pa, pb;
};

CSA_HD inline SampleChunk sample_chunk(int s0, int L, int t0, int nT) {
  SampleChunk sc;
  sc.s0 = s0;
  sc.L = L;
  sc.pa = t0 - s0 > 0 ? t0 - s0 : 0;
  sc.pb = t0 + nT - s0 < L ? t0 + nT - s0 : L;
  return sc;
}

// ---- compressed rows: block k holds local rows [kb k, kb (k + 1)) of the rows visible to some
// query of the chunk; query p sees rows < min((p + 1) / r, n_cap).
CSA_HD inline int cmp_rows(const SampleChunk& sc, int r, int n_cap) {
  const int v = sc.pb / r;
  return v < n_cap ? v : n_cap;
}
CSA_HD inline int cmp_blocks(const SampleChunk& sc, int r, int n_cap, int kb) {
  return (cmp_rows(sc, r, n_cap) + kb - 1) / kb;
}
CSA_HD inline int n_chunks(const SampleChunk& sc) { return (sc.pb - sc.pa + kCq - 1) / kCq; }
// first query of the chunk that sees row kb k
CSA_HD inline int cmp_qlo(const SampleChunk& sc, int r, int k, int kb) {
  const int f = r * (kb * k + 1) - 1;
  return f > sc.pa ? f : sc.pa;
}
// first query chunk (of kCq queries from pa) holding a query that sees block k
CSA_HD inline int cmp_clo(const SampleChunk& sc, int r, int k, int kb) {
  return (cmp_qlo(sc, r, k, kb) - sc.pa) / kCq;
}

// ---- window rows: block m holds local raw rows [kb m, kb (m + 1)); row u is seen by the
// queries u .. u + W - 1 of its sample.
CSA_HD inline int win_mlo(const SampleChunk& sc, int W, int kb) {
  const int u = sc.pa - W + 1;
  return (u > 0 ? u : 0) / kb;
}
CSA_HD inline int win_mhi(const SampleChunk& sc, int kb) { return (sc.pb + kb - 1) / kb; }
struct WinBlock {
  int nk, qlo, qhi, pieces;
};
CSA_HD inline WinBlock win_block(const SampleChunk& sc, int W, int m, int kb) {
  WinBlock wb;
  wb.nk = sc.L - kb * m < kb ? sc.L - kb * m : kb;
  wb.qlo = kb * m > sc.pa ? kb * m : sc.pa;
  const int e = kb * m + wb.nk - 1 + W;
  wb.qhi = e < sc.pb ? e : sc.pb;
  wb.pieces = wb.qhi > wb.qlo ? (wb.qhi - wb.qlo + kCq - 1) / kCq : 0;
  return wb;
}

// Upper bound on the items of one chunk of nT queries (B samples, rows per sample at most
// n_cap compressed rows, window W, blocks of kb rows); partial slots and reduction records are
// at most as many.  Compressed: every sample has at most n_cap / kb + 1 blocks, each in at
// most (its queries in the chunk) / kCq + 1 items.  Window: a sample's blocks that its chunk
// queries see number at most (its queries + W - 1) / kb + 2, each in at most
// ceil((kb - 1 + W) / kCq) items.
CSA_HD inline int64_t item_cap(int mode, int B, int nT, int n_cap, int W, int kb) {
  const int64_t bc = B < nT ? B : nT;
  int64_t n = 0;
  if (mode != 2) n += (int64_t)(n_cap / kb + 1) * ((int64_t)nT / kCq + bc);
  if (W > 0)
    n += (((int64_t)nT + bc * (W - 1)) / kb + 2 * bc) * ((kb - 1 + W + kCq - 1) / kCq);
  return n;
}

}  // namespace keys

#ifdef __HIPCC__
}  // namespace csa
#include <hip/hip_runtime.h>
namespace csa {

// Operands of the key-major pass of one query chunk [t0, t0 + nT).
struct KeysArgs {
  const uint16_t* q;        // [T, 64, 512] bf16
  const uint16_t* dout;     // [T, 64, 512] bf16
  const uint16_t* pds;      // [nT, n_slots, 128]: scale*dS (64 heads) then P (64 heads)
  const int32_t* idx;       // [T, k_cap] (CSA_SPARSE) or null
  const int32_t* nc;        // [T] compressed candidate count of each query
  const int32_t* cu;
  const int32_t* cu_cmp;
  const uint16_t* zeros;    // >= 16 zero bytes
  int4* items;              // [cap] key0, nkeys | kind << 16, first query, queries
  int32_t* item_part;       // [cap] partial slot of the item
  int4* red;                // [cap] key0, nkeys | kind << 16, first partial slot, slots
  float* part;              // [cap, kb, D]
  int32_t* counters;        // [0] items, [1] reduction records, [2] repeated-row flag (zeroed)
  float* dkv_cmp;
  float* dkv;
  int64_t n_slots, cap;
  int t0, nT, B, r, n_cap, W, k_cap, mode;
  int kb;   // rows per block: 128 (attention) or 256 (indexer keys)
  int D;    // width of the gradient rows (and of the partial rows)
  int KC;   // coefficients per (query, slot): 128 (attention: dS | P) or 64 (indexer: E)
};
hipError_t launch_attn_bwd_keys(const KeysArgs& a, hipStream_t s);       // the work items
hipError_t launch_attn_bwd_keys_sums(const KeysArgs& a, hipStream_t s);  // sums, reduction
// Indexer-key gradients: dkI[j] += sum_t sum_h E[t, h, j] qI[t, h] (q = qI [T, 64, 128],
// pds = E [nT, n_slots, 64] bf16, dkv_cmp = dkI, D = 128, KC = 64, W = 0).
hipError_t launch_kl_keys_sums(const KeysArgs& a, hipStream_t s);
#endif

}  // namespace csa
