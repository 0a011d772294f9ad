// Key-major shared-row gradients of the matrix-core attention backward (bf16, H = 64 heads
// sharing one D = 512 K=V row), gfx950.
//
// Method ("DeepSeek-V4 Attention Training Systems", section 8.2, backward without a dense
// matrix; section 3, gradient ownership): after the dq pass has stored scale*dS and P of
// every (query, candidate slot) for the 64 heads, the gradient of a shared row x is
//   d row_x = sum_t [scale dS[t, :, x] | P[t, :, x]] . [q_t; dO_t]        (128-deep per query)
// Each work item (a block of <= 128 consecutive rows of one sample against <= 256 consecutive
// queries of it, enumerated by k_attn_bwd_keys_plan) forms this product on MFMA with the rows
// as the M dimension, d as N and (query, head, {dS, P}) as K: per query the [q_t; dO_t] rows
// (128 x 1 KiB, contiguous) and, for each row of the block that the query attends, its 256-byte
// dS|P slot are loaded global -> LDS, four k-steps of 32 per query, three k-steps in flight.
// Rows the query does not attend load zeros.  No per-pair row gradient is ever stored: the
// workgroup keeps its 128 x 512 fp32 sums in registers for all its queries and writes them
// once, with plain stores, to a partial slot that k_attn_bwd_keys_reduce adds to the rows in
// item order (also for a block with one item: a read-modify-write of the rows here would wait
// out one memory round trip per value).
//
// A row listed twice in one query's idx row (allowed by the sparse layout: each listing is a
// candidate of its own) is taken once here, at its first slot; k_attn_bwd_keys_dups adds the
// other listings when the planner's scan saw any.
#include <math.h>

#include <type_traits>

#include "attn_bwd_keys.h"
#include "attn_common.h"
#include "csa_launch.h"

// M0 is named as clobbered by the LDS-DMA asm below; the compiler keeps no value in it here.
#pragma clang diagnostic ignored "-Winline-asm"

namespace csa {

using namespace attn;
using namespace keys;

namespace {

constexpr int kMaxBlk = 2048;   // compressed blocks of one sample the planner holds in LDS

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// global_load_lds_dwordx4: lane l's 16 bytes land at LDS byte offset lds + 16 l.
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m), "v"(src) : "memory", "m0");
}

// global_load_lds_dword: lane l's 4 bytes land at LDS byte offset lds + 4 l.
__device__ __forceinline__ void dma4(const void* src, const void* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Exclusive prefix of v over the 256 lanes of the workgroup; total in `total`.
__device__ __forceinline__ int wg_scan(int v, int* sh, int& total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int x = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  total = sh[255];
  const int incl = sh[tid];
  __syncthreads();
  return incl - v;
}

}  // namespace

// ---- the work items of one query chunk (one workgroup of 256 lanes)
// Per sample: compressed blocks in query-chunk-major order (the items that share a query
// chunk are consecutive, so that they run side by side on one XCD and share its L2 for the
// [q; dO] rows), then the window blocks in row order.  Partial slots are numbered block-major
// (a block's items are consecutive) for the reduction.
__global__ __launch_bounds__(256) void k_attn_bwd_keys_plan(KeysArgs a) {
  __shared__ int sc_s[256];
  __shared__ int clo_s[kMaxBlk], pbase_s[kMaxBlk];
  const int tid = threadIdx.x;
  const int64_t cap = a.cap;
  int n_items = 0, n_parts = 0, n_red = 0;
  for (int b = 0; b < a.B; ++b) {
    const int s0 = a.cu[b];
    const SampleChunk sc = sample_chunk(s0, a.cu[b + 1] - s0, a.t0, a.nT);
    if (sc.pa >= sc.pb) continue;
    if (a.mode != 2) {
      const int c0 = a.cu_cmp[b];
      const int rows = cmp_rows(sc, a.r, a.n_cap), nblk = cmp_blocks(sc, a.r, a.n_cap, a.kb);
      const int nch = n_chunks(sc);
      const int kind = a.mode == 0 ? kKindSel : kKindDense;
      for (int k0 = 0; k0 < nblk; k0 += 256) {
        const int k = k0 + tid;
        const bool in = k < nblk;
        const int clo = in ? cmp_clo(sc, a.r, k, a.kb) : 0;
        const int ni = in ? nch - clo : 0, v = ni;
        int tot, rtot;
        const int pre = wg_scan(v, sc_s, tot);
        const int rpre = wg_scan(v > 0 ? 1 : 0, sc_s, rtot);
        if (in) {
          clo_s[k] = clo;
          pbase_s[k] = v > 0 ? n_parts + pre : -1;
        }
        if (v > 0 && n_red + rpre < cap)
          a.red[n_red + rpre] = make_int4(c0 + a.kb * k, min(a.kb, rows - a.kb * k) | (kind << 16),
                                          n_parts + pre, ni);
        n_parts += tot;
        n_red += rtot;
      }
      __syncthreads();
      for (int cb = 0; cb < nch; cb += 256) {
        const int c = cb + tid;
        int K = 0;   // blocks seen by chunk c: those with clo <= c (clo grows with k)
        if (c < nch) {
          int lo = 0, hi = nblk;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (clo_s[mid] <= c) lo = mid + 1;
            else hi = mid;
          }
          K = lo;
        }
        int tot;
        const int pre = wg_scan(K, sc_s, tot);
        for (int k = 0; k < K; ++k) {
          const int64_t e = (int64_t)n_items + pre + k;
          if (e >= cap) break;
          const int qa = max(cmp_qlo(sc, a.r, k, a.kb), sc.pa + kCq * c);
          const int qb = min(sc.pb, sc.pa + kCq * (c + 1));
          a.items[e] = make_int4(c0 + a.kb * k, min(a.kb, rows - a.kb * k) | (kind << 16),
                                 s0 + qa, qb - qa);
          a.item_part[e] = pbase_s[k] >= 0 ? pbase_s[k] + (c - clo_s[k]) : -1;
        }
        n_items += tot;
      }
      __syncthreads();   // clo_s and pbase_s are rewritten for the next sample
    }
    if (a.W > 0) {
      const int mlo = win_mlo(sc, a.W, a.kb), nm = win_mhi(sc, a.kb) - mlo;
      for (int m0 = 0; m0 < nm; m0 += 256) {
        const int m = mlo + m0 + tid;
        WinBlock wb = {0, 0, 0, 0};
        if (m0 + tid < nm) wb = win_block(sc, a.W, m, a.kb);
        const int np = wb.pieces, v = np;
        int tot, ptot, rtot;
        const int pre = wg_scan(np, sc_s, tot);
        const int ppre = wg_scan(v, sc_s, ptot);
        const int rpre = wg_scan(v > 0 ? 1 : 0, sc_s, rtot);
        for (int e2 = 0; e2 < np; ++e2) {
          const int64_t e = (int64_t)n_items + pre + e2;
          if (e >= cap) break;
          const int qa = wb.qlo + kCq * e2;
          a.items[e] = make_int4(s0 + a.kb * m, wb.nk | (kKindWin << 16), s0 + qa,
                                 min(kCq, wb.qhi - qa));
          a.item_part[e] = v > 0 ? n_parts + ppre + e2 : -1;
        }
        if (v > 0 && n_red + rpre < cap)
          a.red[n_red + rpre] = make_int4(s0 + a.kb * m, wb.nk | (kKindWin << 16), n_parts + ppre, np);
        n_items += tot;
        n_parts += ptot;
        n_red += rtot;
      }
    }
  }
  if (tid == 0) {
    a.counters[0] = (int)min((int64_t)n_items, cap);
    a.counters[1] = (int)min((int64_t)n_red, cap);
  }
}

// ---- one work item per workgroup: 8 waves, wave w owns d = 64w .. 64w+63 of all 128 rows.
// KI: idx entries per lane of the query's idx row (0 unless the rows are found in idx rows).
template <int KI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_attn_bwd_keys(KeysArgs a) {
  constexpr int kKeys = 128;   // rows per block (a.kb)
  __shared__ __attribute__((aligned(16))) uint16_t Bs[3][32][kD];     // [q; dO] k-step rows
  __shared__ __attribute__((aligned(16))) uint16_t As[3][kKeys][32];  // dS|P of the rows
  __shared__ __attribute__((aligned(16))) int32_t idx_s[KI > 0 ? 512 * KI : 1];
  __shared__ int32_t slot_s[2][kKeys];
  __shared__ int32_t nc_s[kCq];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // XCD x = blockIdx % 8 takes items x * per .. x * per + per - 1 in order
  const int n_items = a.counters[0];
  const int per = (n_items + 7) >> 3;
  const int jb = (int)(blockIdx.x >> 3);
  if (jb >= per) return;
  const int item = (int)(blockIdx.x & 7) * per + jb;
  if (item >= n_items) return;
  const int4 it = a.items[item];
  const int key0 = it.x, nkeys = it.y & 0xffff, kind = it.y >> 16, q0 = it.z, nq = it.w;
  const int part = a.item_part[item];
  if (part < 0 || part >= a.cap || nq <= 0 || nq > kCq) return;
  TokenInfo ti;
  token_info_wave(a.cu, a.B, q0, ti, kind == kKindWin ? nullptr : a.cu_cmp);
  const int s0 = ti.start, c0 = ti.c0;
  for (int i = tid; i < nq; i += 512) nc_s[i] = a.nc[q0 + i];

  // slot map of query tq, stage 0: its idx row into LDS and the map reset (selected rows)
  auto prep0 = [&](int tq) {
    if (KI > 0 && kind == kKindSel) {
      const int32_t* row = a.idx + (int64_t)(q0 + tq) * a.k_cap;
#pragma unroll
      for (int e = 0; e < KI; ++e) {
        const int base = 64 * (8 * e + wave);
        if (base < a.k_cap) dma4(row + base + lane, &idx_s[base]);
      }
      if (tid < kKeys) slot_s[tq & 1][tid] = 0x7fffffff;
    }
  };
  // stage 1: slot of each row of the block for query tq (-1 / INT_MAX: not attended)
  auto prep1 = [&](int tq) {
    const int t = q0 + tq, p = t - s0, nct = nc_s[tq];
    if (kind == kKindSel) {
      if (KI > 0) {
        for (int c = tid; c < nct; c += 512) {
          const int j = idx_s[c] - key0;
          if (j >= 0 && j < nkeys) {
            const int old = atomicMin(&slot_s[tq & 1][j], c);
            if (old != 0x7fffffff) a.counters[2] = 1;   // a row listed twice
          }
        }
      }
    } else if (tid < kKeys) {
      int s = -1;
      if (tid < nkeys) {
        if (kind == kKindDense) {
          const int jl = key0 - c0 + tid, nv = min((p + 1) / a.r, a.n_cap);
          if (jl < nv) s = jl;
        } else {
          const int u = key0 + tid, nw = min(a.W, p + 1), w0 = t - nw + 1;
          if (u >= w0 && u <= t) s = nct + (u - w0);
        }
      }
      slot_s[tq & 1][tid] = s;
    }
  };
  // k-step s (query s / 4, k-step s % 4) into buffer s % 3: wave w loads [q; dO] rows
  // 4w .. 4w+3 of the k-step (1 KiB each, chunk-swizzled; part jj < 4) and the dS|P columns of
  // rows 16w .. 16w+15 (64 bytes each; lane l: row 16w + l/4, physical chunk l%4; part 4)
  auto b_src = [&](int s) {
    const int i = s & 3;
    return (i < 2 ? a.q : a.dout) + ((int64_t)(q0 + (s >> 2)) * kH + 32 * (i & 1)) * kD;
  };
  auto issue_b = [&](int s, const uint16_t* src, int jj) {
    const int r = 4 * wave + jj;
    dma16(src + (int64_t)r * kD + 8 * (lane ^ swz(r)), &Bs[s % 3][r][0]);
  };
  auto a_src = [&](int s) {
    const int tq = s >> 2, i = s & 3;
    const int sl = slot_s[tq & 1][16 * wave + (lane >> 2)];
    const int lc = (lane & 3) ^ (lane >> 4);
    return (sl >= 0 && sl != 0x7fffffff)
               ? a.pds + ((int64_t)(q0 + tq - a.t0) * a.n_slots + sl) * 128 + 32 * i + 8 * lc
               : a.zeros;
  };
  auto issue_a = [&](int s, const uint16_t* src) { dma16(src, &As[s % 3][16 * wave][0]); };
  auto issue = [&](int s) {
    const uint16_t* src = b_src(s);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) issue_b(s, src, jj);
    issue_a(s, a_src(s));
  };

  // B operand: [q; dO] rows 8g .. 8g+7 of the k-step at d = 64w + 16nt + c16, read transposed;
  // A operand: dS|P of row 16mt + c16, k 8g .. 8g+7 (physical chunk g ^ (c16 / 4))
  const int trr = 8 * g + (c16 >> 2), tre = (c16 & 3) >> 1, troff = 4 * (c16 & 1);
  const int lo_s = 8 * ((8 * wave + tre) ^ swz(trr)), hi_s = 8 * ((8 * wave + tre) ^ swz(trr + 4));
  const int aoff = 8 * (g ^ (c16 >> 2));
  f32x4 acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int S = 4 * nq;
  prep0(0);
  wait_vmem();
  __syncthreads();
  prep1(0);
  __syncthreads();
  issue(0);
  if (S > 1) issue(1);
  // k-step s; MORE: k-step s + 2 exists (its loads are issued between this step's MFMAs, so
  // that a load waiting for the address unit overlaps the MFMAs in flight)
  auto body = [&](auto more_c, int s) {
    constexpr bool kMore = decltype(more_c)::value;
    const int tq = s >> 2, i = s & 3, buf = s % 3;
    // every wave issues 5 loads per k-step: all but the next k-step's are done
    if (s + 1 < S) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else wait_vmem();
    __syncthreads();
    if (i == 0 && tq + 1 < nq) prep0(tq + 1);
    if (i == 1 && tq + 1 < nq) prep1(tq + 1);
    const uint16_t* bsrc = kMore ? b_src(s + 2) : nullptr;
    const uint16_t* asrc = kMore ? a_src(s + 2) : nullptr;
    bf16x8 bv[4], av[8];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      bv[nt] = join8(ld_tr(&Bs[buf][trr][troff + (lo_s ^ (16 * nt))]),
                     ld_tr(&Bs[buf][trr + 4][troff + (hi_s ^ (16 * nt))]));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) av[mt] = ld16(&As[buf][16 * mt + c16][aoff]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma16(av[mt], bv[nt], acc[mt][nt]);
      if (kMore && mt < 4) issue_b(s + 2, bsrc, mt);
      if (kMore && mt == 4) issue_a(s + 2, asrc);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int s = 0;
  for (; s + 2 < S; ++s) body(std::true_type(), s);
  for (; s < S; ++s) body(std::false_type(), s);
  // rows 16mt + 4g + i, d = 64w + 16nt + c16
  float* dst = a.part + (int64_t)part * kKeys * kD;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * g + i;
      if (row >= nkeys) continue;
      float* o = dst + (int64_t)row * kD + 64 * wave + c16;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) o[16 * nt] = acc[mt][nt][i];
    }
}

// ---- every block: rows += sum of its partial slots, in slot order.
// Work unit = (block record, 8 rows); lane: row 8u' + tid / 32, columns (tid % 32) D/32 ..
// (D = 512 or 128: 4 or 1 float4 per lane).
__global__ __launch_bounds__(256) void k_attn_bwd_keys_reduce(KeysArgs a) {
  const int kUnits = a.kb / 8;
  const int n_units = a.counters[1] * kUnits;
  const int nv4 = a.D / 128;
  for (int w = blockIdx.x; w < n_units; w += gridDim.x) {
    const int4 rd = a.red[w / kUnits];
    const int key0 = rd.x, nkeys = rd.y & 0xffff, kind = rd.y >> 16, pf = rd.z, np = rd.w;
    const int row = 8 * (w % kUnits) + (threadIdx.x >> 5), d = nv4 * 4 * (threadIdx.x & 31);
    if (row >= nkeys || pf < 0 || pf + np > a.cap) continue;
    float4 s[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) s[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = 0; p < np; ++p) {
      const float4* src =
          reinterpret_cast<const float4*>(a.part + ((int64_t)(pf + p) * a.kb + row) * a.D + d);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (v < nv4) {
          const float4 x = src[v];
          s[v].x += x.x; s[v].y += x.y; s[v].z += x.z; s[v].w += x.w;
        }
      }
    }
    float4* o = reinterpret_cast<float4*>((kind == kKindWin ? a.dkv : a.dkv_cmp) +
                                          (int64_t)(key0 + row) * a.D + d);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v < nv4) {
        float4 x = o[v];
        x.x += s[v].x; x.y += s[v].y; x.z += s[v].z; x.w += s[v].w;
        o[v] = x;
      }
    }
  }
}

// ---- rows listed more than once in a query's idx row: the key-major pass took each such row
// at its first slot; add the contributions of the later slots (rare; only when flagged).
// Coefficient k of a slot multiplies row k of [q_t; dO_t] (KC = 128: the attention's dS | P)
// or row k of qI_t (KC = 64: the indexer loss's E).
__global__ __launch_bounds__(256) void k_attn_bwd_keys_dups(KeysArgs a) {
  __shared__ int32_t row_s[2048];
  __shared__ int32_t dup_s[2048];
  __shared__ int n_dup;
  if (a.counters[2] == 0) return;
  const int tid = threadIdx.x;
  for (int tl = blockIdx.x; tl < a.nT; tl += gridDim.x) {
    const int t = a.t0 + tl;
    TokenInfo ti;
    if (!token_info(a.cu, a.B, t, ti)) continue;
    const int c0 = a.cu_cmp[ti.b], nv = min((ti.p + 1) / a.r, a.n_cap);
    const int nct = min(a.nc[t], 2048);
    for (int c = tid; c < nct; c += 256) row_s[c] = a.idx[(int64_t)t * a.k_cap + c];
    if (tid == 0) n_dup = 0;
    __syncthreads();
    for (int c = tid; c < nct; c += 256) {
      const int j = row_s[c];
      if (j < c0 || j >= c0 + nv) continue;
      bool dup = false;
      for (int c2 = 0; c2 < c && !dup; ++c2) dup = row_s[c2] == j;
      if (dup) dup_s[atomicAdd(&n_dup, 1)] = c;
    }
    __syncthreads();
    const int nd = n_dup;
    const uint16_t* bt = a.q + (int64_t)t * 64 * a.D;
    const uint16_t* gt = a.KC == 128 ? a.dout + (int64_t)t * 64 * a.D : nullptr;
    for (int e = 0; e < nd; ++e) {
      const int c = dup_s[e], j = row_s[c];
      const uint16_t* ps = a.pds + ((int64_t)tl * a.n_slots + c) * a.KC;
      for (int d = tid; d < a.D; d += 256) {
        float s = 0.f;
        for (int h = 0; h < 64; ++h) {
          s += bf2f(ps[h]) * bf2f(bt[h * a.D + d]);
          if (gt) s += bf2f(ps[64 + h]) * bf2f(gt[h * a.D + d]);
        }
        atomicAdd(a.dkv_cmp + (int64_t)j * a.D + d, s);
      }
    }
    __syncthreads();
  }
}

// ---- indexer-key gradients, one work item per workgroup: dkI[j] += sum_t E[t, :, j] qI_t for
// the item's 256 rows and queries (the same items, slot maps and partial slots as the
// attention's compressed rows, no window); per query two k-steps of 32 heads: the qI rows
// 32i .. 32i+31 (256 bytes each) and the rows' 64-byte E pieces, three k-steps in flight.
// 4 waves, wave w owns d = 32w .. 32w+31 of all 256 rows.
template <int KI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_kl_keys(KeysArgs a) {
  constexpr int kDI = 128, kKeys = 256;   // rows per block (a.kb)
  __shared__ __attribute__((aligned(16))) uint16_t Bs[3][32][kDI];    // qI k-step rows
  __shared__ __attribute__((aligned(16))) uint16_t As[3][kKeys][32];  // E of the rows
  __shared__ __attribute__((aligned(16))) int32_t idx_s[KI > 0 ? 256 * KI : 1];
  __shared__ int32_t slot_s[2][kKeys];
  __shared__ int32_t nc_s[kCq];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int n_items = a.counters[0];
  const int per = (n_items + 7) >> 3;
  const int jb = (int)(blockIdx.x >> 3);
  if (jb >= per) return;
  const int item = (int)(blockIdx.x & 7) * per + jb;
  if (item >= n_items) return;
  const int4 it = a.items[item];
  const int key0 = it.x, nkeys = it.y & 0xffff, kind = it.y >> 16, q0 = it.z, nq = it.w;
  const int part = a.item_part[item];
  if (part < 0 || part >= a.cap || nq <= 0 || nq > kCq) return;
  TokenInfo ti;
  token_info_wave(a.cu, a.B, q0, ti, a.cu_cmp);
  const int s0 = ti.start, c0 = ti.c0;
  for (int i = tid; i < nq; i += 256) nc_s[i] = a.nc[q0 + i];

  auto prep0 = [&](int tq) {
    if (KI > 0 && kind == kKindSel) {
      const int32_t* row = a.idx + (int64_t)(q0 + tq) * a.k_cap;
#pragma unroll
      for (int e = 0; e < KI; ++e) {
        const int base = 64 * (4 * e + wave);
        if (base < a.k_cap) dma4(row + base + lane, &idx_s[base]);
      }
      if (tid < kKeys) slot_s[tq & 1][tid] = 0x7fffffff;
    }
  };
  auto prep1 = [&](int tq) {
    const int t = q0 + tq, p = t - s0, nct = nc_s[tq];
    if (kind == kKindSel) {
      if (KI > 0) {
        for (int c = tid; c < nct; c += 256) {
          const int j = idx_s[c] - key0;
          if (j >= 0 && j < nkeys) {
            const int old = atomicMin(&slot_s[tq & 1][j], c);
            if (old != 0x7fffffff) a.counters[2] = 1;   // a row listed twice
          }
        }
      }
    } else if (tid < kKeys) {
      int s = -1;
      if (tid < nkeys) {
        const int jl = key0 - c0 + tid, nv = min((p + 1) / a.r, a.n_cap);
        if (jl < nv) s = jl;
      }
      slot_s[tq & 1][tid] = s;
    }
  };
  // k-step s (query s / 2, heads 32 (s % 2) ..) into buffer s % 3.  qI parts 0, 1: rows
  // 8w + 4jj .. +3 (lane l: row + l/16, physical chunk l%16); E parts 0 .. 3: the 64-byte E
  // pieces of rows 64w + 16jj .. +15 (lane l: row + l/4, physical chunk l%4)
  auto b_src = [&](int s) { return a.q + ((int64_t)(q0 + (s >> 1)) * 64 + 32 * (s & 1)) * kDI; };
  auto issue_b = [&](int s, const uint16_t* src, int jj) {
    const int r0 = 8 * wave + 4 * jj, r = r0 + (lane >> 4);
    dma16(src + (int64_t)r * kDI + 8 * ((lane & 15) ^ swz(r)), &Bs[s % 3][r0][0]);
  };
  auto a_src = [&](int s, int jj) {
    const int tq = s >> 1, i = s & 1;
    const int sl = slot_s[tq & 1][64 * wave + 16 * jj + (lane >> 2)];
    const int lc = (lane & 3) ^ (lane >> 4);
    return (sl >= 0 && sl != 0x7fffffff)
               ? a.pds + ((int64_t)(q0 + tq - a.t0) * a.n_slots + sl) * 64 + 32 * i + 8 * lc
               : a.zeros;
  };
  auto issue_a = [&](int s, const uint16_t* src, int jj) {
    dma16(src, &As[s % 3][64 * wave + 16 * jj][0]);
  };
  auto issue = [&](int s) {
    const uint16_t* src = b_src(s);
    issue_b(s, src, 0);
    issue_b(s, src, 1);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) issue_a(s, a_src(s, jj), jj);
  };

  const int trr = 8 * g + (c16 >> 2), tre = (c16 & 3) >> 1, troff = 4 * (c16 & 1);
  const int lo_s = 8 * ((4 * wave + tre) ^ swz(trr)), hi_s = 8 * ((4 * wave + tre) ^ swz(trr + 4));
  const int aoff = 8 * (g ^ (c16 >> 2));
  f32x4 acc[16][2];
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The loads of k-step s + 2 are issued in k-step s, so the slot map of query tq + 2 is
  // formed in query tq's k-steps (idx row loaded in the first, mapped in the second) and
  // first read in query tq + 1's first k-step: maps of queries 0 and 1 before the loop.
  const int S = 2 * nq;
  for (int q = 0; q < 2 && q < nq; ++q) {
    prep0(q);
    wait_vmem();
    __syncthreads();
    prep1(q);
    __syncthreads();
  }
  issue(0);
  if (S > 1) issue(1);
  auto body = [&](auto more_c, int s) {
    constexpr bool kMore = decltype(more_c)::value;
    const int tq = s >> 1, i = s & 1, buf = s % 3;
    // every wave issues 6 loads per k-step (an idx row's loads come before them): all but
    // the next k-step's are done
    if (s + 1 < S) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else wait_vmem();
    __syncthreads();
    if (i == 0 && tq + 2 < nq) prep0(tq + 2);
    if (i == 1 && tq + 2 < nq) prep1(tq + 2);
    if (kMore) issue(s + 2);
    bf16x8 bv[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      bv[nt] = join8(ld_tr(&Bs[buf][trr][troff + (lo_s ^ (16 * nt))]),
                     ld_tr(&Bs[buf][trr + 4][troff + (hi_s ^ (16 * nt))]));
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
      const bf16x8 av = ld16(&As[buf][16 * mt + c16][aoff]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma16(av, bv[nt], acc[mt][nt]);
    }
  };
  int s = 0;
  for (; s + 2 < S; ++s) body(std::true_type(), s);
  for (; s < S; ++s) body(std::false_type(), s);
  // rows 16mt + 4g + i, d = 32w + 16nt + c16
  float* dst = a.part + (int64_t)part * kKeys * kDI;
#pragma unroll
  for (int mt = 0; mt < 16; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * g + i;
      if (row >= nkeys) continue;
      float* o = dst + (int64_t)row * kDI + 32 * wave + c16;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) o[16 * nt] = acc[mt][nt][i];
    }
}

hipError_t launch_attn_bwd_keys(const KeysArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_attn_bwd_keys_plan, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_keys_sums(const KeysArgs& a, hipStream_t s) {
  if (a.kb != 128) return hipErrorInvalidValue;
  const int64_t grid = ((a.cap + 7) / 8) * 8;
  if (a.mode != 0)
    hipLaunchKernelGGL(k_attn_bwd_keys<0>, dim3((unsigned)grid), dim3(512), 0, s, a);
  else if (a.k_cap <= 1024)
    hipLaunchKernelGGL(k_attn_bwd_keys<2>, dim3((unsigned)grid), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_bwd_keys<4>, dim3((unsigned)grid), dim3(512), 0, s, a);
  const int64_t rgrid = a.cap * (a.kb / 8) < 2048 ? a.cap * (a.kb / 8) : 2048;
  hipLaunchKernelGGL(k_attn_bwd_keys_reduce, dim3((unsigned)(rgrid > 0 ? rgrid : 1)), dim3(256), 0, s, a);
  if (a.mode == 0) hipLaunchKernelGGL(k_attn_bwd_keys_dups, dim3(1024), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kl_keys_sums(const KeysArgs& a, hipStream_t s) {
  if (a.kb != 256) return hipErrorInvalidValue;
  const int64_t grid = ((a.cap + 7) / 8) * 8;
  if (a.mode != 0)
    hipLaunchKernelGGL(k_kl_keys<0>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else if (a.k_cap <= 1024)
    hipLaunchKernelGGL(k_kl_keys<4>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_kl_keys<8>, dim3((unsigned)grid), dim3(256), 0, s, a);
  const int64_t rgrid = a.cap * (a.kb / 8) < 2048 ? a.cap * (a.kb / 8) : 2048;
  hipLaunchKernelGGL(k_attn_bwd_keys_reduce, dim3((unsigned)(rgrid > 0 ? rgrid : 1)), dim3(256), 0, s, a);
  if (a.mode == 0) hipLaunchKernelGGL(k_attn_bwd_keys_dups, dim3(1024), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
