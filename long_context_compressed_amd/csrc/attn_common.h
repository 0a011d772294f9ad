// Shared pieces of the matrix-core attention kernels (bf16, H = 64 heads sharing one
// D = 512 K=V row): operand types, the token -> workgroup mapping, candidate slots.
#pragma once

#include "csa_device.h"

namespace csa {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kH = 64;
constexpr int kD = 512;
constexpr int kChunk = 256;   // tokens per XCD chunk

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane j supplies the
// address of row rowbase + j/4, columns colbase + 4(j%4) .. +3 of a row-major bf16 tile;
// lane i then receives column colbase + i of rows rowbase .. rowbase + 3.
__device__ __forceinline__ v4i16 ld_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
}

__device__ __forceinline__ bf16x8 join8(v4i16 lo, v4i16 hi) {
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// Workgroup -> token: XCD x = bid % 8 takes 256-token chunks x, x+8, x+16, ...
__device__ __forceinline__ int token_of_block(int bid) {
  const int x = bid & 7, j = bid >> 3;
  return (j / kChunk) * (8 * kChunk) + x * kChunk + (j % kChunk);
}

__host__ __forceinline__ int64_t token_grid(int64_t n) {
  return ((n + 8 * kChunk - 1) / (8 * kChunk)) * 8 * kChunk;
}

// First -1 of an idx row (k_cap if none); every thread of the block gets it.
__device__ __forceinline__ int leading_valid(const int32_t* __restrict__ row, int k_cap, int* s_tmp) {
  if (threadIdx.x == 0) *s_tmp = k_cap;
  __syncthreads();
  for (int c = threadIdx.x; c < k_cap; c += blockDim.x)
    if (row[c] < 0) atomicMin(s_tmp, c);
  __syncthreads();
  const int n = *s_tmp;
  __syncthreads();
  return n;
}

// An idx row of up to NPT * blockDim.x entries read into registers with every load in
// flight at once (a copy loop that stores each entry before loading the next waits one
// load latency per pass); store_idx_lds then writes it to LDS.  Entries past k_cap are 0.
template <int NPT>
__device__ __forceinline__ void load_idx_regs(const int32_t* __restrict__ row, int k_cap,
                                              int (&v)[NPT]) {
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int c = threadIdx.x + blockDim.x * i;
    v[i] = c < k_cap ? row[c] : 0;
  }
}
template <int NPT>
__device__ __forceinline__ void store_idx_lds(int32_t* dst, int k_cap, const int (&v)[NPT]) {
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int c = threadIdx.x + blockDim.x * i;
    if (c < k_cap) dst[c] = v[i];
  }
}

// leading_valid of an idx row that the calling block has copied into LDS (row); the first
// barrier publishes the copy, so the row is read from global memory once.
__device__ __forceinline__ int leading_valid_lds(const int32_t* row, int k_cap, int* s_tmp) {
  if (threadIdx.x == 0) *s_tmp = k_cap;
  __syncthreads();
  for (int c = threadIdx.x; c < k_cap; c += blockDim.x)
    if (row[c] < 0) atomicMin(s_tmp, c);
  __syncthreads();
  const int n = *s_tmp;
  __syncthreads();
  return n;
}

// Sample of packed row t (false for capacity padding, t >= cu[B]).  The wave reads up to 64
// entries of cu_seqlens at once and counts those <= t, so the lookup costs one load latency
// per 64 samples instead of a chain of dependent loads.  Given the compressed offsets
// cu_cmp, the same pass also reads the sample's first compressed row into ti.c0.  Every
// lane of the wave must call it.
__device__ __forceinline__ bool token_info_wave(const int32_t* __restrict__ cu, int B, int t,
                                                TokenInfo& ti,
                                                const int32_t* __restrict__ cu_cmp = nullptr) {
  const int lane = threadIdx.x & 63;
  int cnt = 0, lo = 0, hi = 0, c0 = 0;   // cnt = #{i <= B : cu[i] <= t}
  for (int base = 0; base <= B; base += 64) {
    const int i = base + lane;
    const int v = i <= B ? cu[i] : 0x7fffffff;
    const int vc = (cu_cmp && i <= B) ? cu_cmp[i] : 0;
    const uint64_t le = __ballot(v <= t);
    const int n = __popcll(le);
    if (n == 0) break;
    cnt += n;
    // cu[cnt - 1] and cu[cnt] (if still within this group of 64)
    const int j = cnt - 1 - base;
    lo = __shfl(v, j, 64);
    c0 = __shfl(vc, j, 64);
    hi = j + 1 < 64 ? __shfl(v, j + 1, 64) : 0x7fffffff;
    if (n < 64) break;
  }
  if (cnt == 0 || cnt > B) return false;
  if (hi == 0x7fffffff) hi = cu[cnt];
  ti.b = cnt - 1;
  ti.start = lo;
  ti.len = hi - lo;
  ti.p = t - lo;
  ti.c0 = c0;
  return true;
}

// Candidate slots of a query: compressed candidates in [0, n_c), masked padding in
// [n_c, n_cs), window rows in [n_cs, n_cs + n_w).
struct CandSet {
  int n_c, n_cs, n_w, row0, nv, win0;
};

// Row id of slot c: >= 0 a compressed row, <= -2 the raw row -2 - id, -1 no row.
__device__ __forceinline__ int slot_row(const int32_t* __restrict__ idx_t, int mode,
                                        const CandSet& cs, int c) {
  if (c < cs.n_c) {
    const int g = mode == 1 ? cs.row0 + c : idx_t[c];
    return (g >= cs.row0 && g < cs.row0 + cs.nv) ? g : -1;
  }
  if (c < cs.n_cs) return -1;
  if (c < cs.n_cs + cs.n_w) return -2 - (cs.win0 + (c - cs.n_cs));
  return -1;
}

// 16-byte chunk swizzle of 1 KiB LDS rows: physical chunk = logical chunk ^ swz(row), a
// bijection on the low four row bits.  Sixteen consecutive rows read at one logical chunk
// (ds_read_b128) hit sixteen distinct 16-byte bank groups, and four aligned rows read at two
// adjacent chunks (ds_read_b64_tr_b16) hit eight, in both halves of a 64-bank LDS.
__device__ __forceinline__ int swz(int row) {
  return ((row & 3) << 1) | ((row >> 2) & 1) | (row & 8);
}

}  // namespace attn
}  // namespace csa
