// Matrix-core (MFMA) sparse attention backward for bf16 operands, H = 64 heads sharing one
// D = 512 K=V row (MQA), on gfx950.
//
// Method ("DeepSeek-V4 Attention Training Systems", section 8.2): from the saved O and
// log-sum-exp, recompute P over each query's candidates and return dq, the gradients of
// the shared compressed rows and raw window rows (key and value contributions summed, as
// one row is both), and the optional sink gradient.
#include <math.h>

#include "attn_bwd_keys.h"
#include "attn_common.h"
#include "csa_launch.h"
#include "csr_build.h"

// M0 is named as clobbered by the LDS-DMA asm below; the compiler keeps no value in it here.
#pragma clang diagnostic ignored "-Winline-asm"

namespace csa {

using namespace attn;

// The backward is processed in chunks of query tokens (so the workspace stays bounded);
// per chunk:
// Kernel 1 (k_attn_bwd_dq_mfma): one workgroup per query token.  Per block of 32
// candidates the rows are gathered into swizzled LDS rows by direct global->LDS loads (the
// next block's rows one per two k-steps of the current block's S^T loop); wave w recomputes
// S^T and dP^T for heads 16w..16w+15 on MFMA (A = rows from LDS, B = its Q / dO slice
// resident in registers), forms P = e^{S - LSE} and dS = P (dP - Dt) in fp32 and writes
// scale*dS and P (bf16) to an LDS tile [slot][head]; after a barrier wave w accumulates
// dq[:, 128w .. 128w+127] += (scale dS) K over all 64 heads, with dS read transposed from
// the tile as the A operand and the row tile read transposed (ds_read_b64_tr_b16) as the B
// operand; the tile is also stored as the dS|P rows kernel 2 reads.
// Kernel 2 (k_attn_bwd_dkv_mfma): one workgroup per query token, two per CU, wave w owns
// d-slice 128w..128w+127.  Q, then dO, of the token are staged in LDS and read transposed
// into registers; per block of 32 candidates the row gradients
// (d row)^T = [Q; dO]^T [scale dS | P]^T are formed on MFMA (lane = candidate, 4
// consecutive d) and stored as bf16 to a staging buffer, one 1 KiB vector per
// (query, candidate) pair, with plain stores.
// Then the owner of each shared row sums its staged vectors in fp32: a CSR of the
// compressed rows (row -> contributing (query, slot) pairs) is built from the candidate
// lists, and window rows find their contributors directly (the next W-1 queries).
// Stores + an owner-side gather replace fp32 atomics, which run at a fraction of the
// store bandwidth on this part.

namespace {

constexpr int kDW = 128;          // d per wave, kernel 2
constexpr int kNB1 = 32;          // candidates per block, kernel 1
constexpr int kKS = kD + 16;      // row stride (bf16) of LDS row tiles
constexpr int kNB2 = 64;          // slot padding of the per-query staging rows
constexpr int kNB3 = 32;          // candidates per block, kernel 2
constexpr int kPTS = 144;         // row stride (bf16) of the dS | P tile (conflict-free reads)

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One 16-byte-per-lane global -> LDS load (global_load_lds_dwordx4): lane l's 16 bytes land
// at LDS byte offset lds_row + 16 l.  Issued through asm so that the compiler does not order
// LDS reads of the other tile buffer behind it; completion is awaited with wait_vmem().
__device__ __forceinline__ void dma_row16(const void* src, const void* lds_row) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_row);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(src) : "memory", "m0");
}
constexpr int64_t kStageBudget = 96ll << 30;   // bytes of pds + staging per chunk
constexpr int kIdxLds = 2048;                   // idx entries of a query staged in LDS (kernel 1)

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* kv_cmp;
  const uint16_t* kv;
  const int32_t* idx;
  const float* sink;
  const int32_t* cu;
  const int32_t* cu_cmp;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  float* dkv_cmp;
  float* dkv;
  float* dsink;
  uint16_t* pds;     // [chunk][n_slots][128]: scale*dS (64 heads) then P (64 heads)
  uint16_t* stage;   // [chunk][n_slots][512]: bf16 row gradient of each (query, slot)
  int32_t* nc;       // [T] compressed candidate count of each query
  int32_t* cnt;      // [Tc_cap] contributors per compressed row (this chunk)
  int32_t* off;      // [Tc_cap] CSR offsets
  int32_t* cur;      // [Tc_cap] CSR fill cursors
  int32_t* list;     // [chunk * n_c_max] (query - t0) * n_slots + slot
  int64_t n_slots;
  int t0, nT, Tc_cap;
  int B, T, r, n_cap, W, k_cap, mode;
  float scale, scale_log2;
};

// ti from token_info_wave with the compressed offsets; idx_lds: the query's idx row copied
// into LDS by the calling block (published by the scan's first barrier), or null
__device__ __forceinline__ CandSet make_cands(const BwdArgs& b, int t, const TokenInfo& ti,
                                              int* s_tmp, const int32_t* idx_lds) {
  CandSet cs;
  cs.row0 = ti.c0;
  cs.nv = min((ti.p + 1) / b.r, b.n_cap);
  cs.n_w = min(b.W, ti.p + 1);
  cs.win0 = t - cs.n_w + 1;
  if (b.mode == 1) cs.n_c = cs.nv;
  else if (b.mode == 2) cs.n_c = 0;
  else if (idx_lds) cs.n_c = leading_valid_lds(idx_lds, b.k_cap, s_tmp);
  else cs.n_c = leading_valid(b.idx + (int64_t)t * b.k_cap, b.k_cap, s_tmp);
  cs.n_cs = cs.n_c;
  return cs;
}

// Pointer to the row of candidate slot c, or nullptr for a masked / absent slot.
__device__ __forceinline__ const uint16_t* cand_ptr(const BwdArgs& b, int t, const CandSet& cs,
                                                    int c) {
  const int id = slot_row(b.mode == 0 ? b.idx + (int64_t)t * b.k_cap : nullptr, b.mode, cs, c);
  if (id == -1) return nullptr;
  return id >= 0 ? b.kv_cmp + (int64_t)id * kD : b.kv + (int64_t)(-2 - id) * kD;
}

// Global compressed row of slot c (< n_c) of query t, or -1 if it is outside the visible range.
__device__ __forceinline__ int cmp_row(const BwdArgs& b, int t, int row0, int nv, int c) {
  const int gr = b.mode == 1 ? row0 + c : b.idx[(int64_t)t * b.k_cap + c];
  return (gr >= row0 && gr < row0 + nv) ? gr : -1;
}

}  // namespace

// IDX_LDS: the query's idx row (k_cap <= kIdxLds) is staged in LDS once, so that the block
// loop reads its next slots from LDS instead of issuing a global load per block.
template <bool IDX_LDS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_attn_bwd_dq_mfma(BwdArgs b) {
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][kNB1][kD];       // swizzled 1 KiB rows
  __shared__ __attribute__((aligned(16))) uint16_t PT[2][kNB1][kPTS];     // [slot][dS | P]
  __shared__ int32_t idx_s[IDX_LDS ? kIdxLds : 1];
  __shared__ int s_tmp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int tl = token_of_block(blockIdx.x);
  if (tl >= b.nT) return;
  const int t = b.t0 + tl;
  TokenInfo ti;
  if (!token_info_wave(b.cu, b.B, t, ti, b.cu_cmp)) {
    uint4* o = reinterpret_cast<uint4*>(b.dq + (int64_t)t * kH * kD);
    for (int e = tid; e < kH * kD / 8; e += 256) o[e] = make_uint4(0, 0, 0, 0);
    if (tid == 0) b.nc[t] = 0;
    return;
  }
  const int h = 16 * wave + c16;  // this lane's head for S^T / dP^T (n index)

  // the idx row first (into registers; to LDS once the operands are in flight), then the B
  // operands Q[h][32ks + 8g ..] and dO[h][...] and Dt = dO . O for head h
  const int32_t* idx_t = b.mode == 0 ? b.idx + (int64_t)t * b.k_cap : nullptr;
  int iv[IDX_LDS ? kIdxLds / 256 : 1];
  if (IDX_LDS && b.mode == 0) load_idx_regs(idx_t, b.k_cap, iv);
  bf16x8 qb[16], gb[16];
  const int64_t rowq = ((int64_t)t * kH + h) * kD;
  const float lse_t = b.lse[(int64_t)t * kH + h];
  float dt = 0.f;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    qb[ks] = ld16(b.q + rowq + 32 * ks + 8 * g);
    gb[ks] = ld16(b.dout + rowq + 32 * ks + 8 * g);
    float ov[8], gv[8];
    load8(b.o + rowq + 32 * ks + 8 * g, ov);
    load8(b.dout + rowq + 32 * ks + 8 * g, gv);
#pragma unroll
    for (int i = 0; i < 8; ++i) dt = fmaf(ov[i], gv[i], dt);
  }
  if (IDX_LDS && b.mode == 0) store_idx_lds(idx_s, b.k_cap, iv);   // published by make_cands
  // raw idx entry of slot 32 blk + (lane & 31)
  auto raw_of = [&](int blk) {
    const int c = kNB1 * blk + (lane & 31);
    if (b.mode != 0 || c >= b.k_cap) return 0;
    return IDX_LDS ? idx_s[c] : idx_t[c];
  };
  const CandSet cs = make_cands(b, t, ti, &s_tmp, IDX_LDS && b.mode == 0 ? idx_s : nullptr);
  int raw_cur = raw_of(0), raw_nxt = raw_of(1);
  if (tid == 0) b.nc[t] = cs.n_c;
  const int n_tot = cs.n_c + cs.n_w;
  const int nblk = (n_tot + kNB1 - 1) / kNB1;
  dt += __shfl_xor(dt, 16, 64);
  dt += __shfl_xor(dt, 32, 64);
  const float lse2 = lse_t * 1.44269504088896341f;

  f32x4 dq[4][8];   // heads 16mt + 4g + i, d = 128 wave + 16nt + c16
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) dq[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // row id of slot 32 blk + (lane & 31): >= 0 compressed row, <= -2 raw row -2 - id, -1 none
  auto rid_of = [&](int blk, int raw) {
    const int c = kNB1 * blk + (lane & 31);
    if (blk >= nblk) return -1;
    if (c < cs.n_c) {
      const int gr = b.mode == 1 ? cs.row0 + c : raw;
      return (gr >= cs.row0 && gr < cs.row0 + cs.nv) ? gr : -1;
    }
    if (c < n_tot) return -2 - (cs.win0 + (c - cs.n_c));
    return -1;
  };
  // wave w gathers rows 8w .. 8w+7 of a block (one 1 KiB row per instruction, lane l fills
  // physical chunk l); an absent slot loads the query's own raw row (finite, masked)
  auto issue_row = [&](int rid, int buf, int j) {
    const int r = 8 * wave + j;
    const int id = __builtin_amdgcn_readlane(rid, r);
    const uint16_t* src = id >= 0 ? b.kv_cmp + (int64_t)id * kD
                                  : b.kv + (int64_t)(id == -1 ? t : -2 - id) * kD;
    dma_row16(src + 8 * (lane ^ swz(r)), &Kt[buf][r][0]);
  };
  auto issue = [&](int rid, int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_row(rid, buf, j);
  };
  // per-lane LDS offsets (elements): S^T A operand rows 16mt + c16, logical chunk 4ks + g
  int eq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) eq[q] = 8 * ((4 * q + g) ^ swz(c16));
  // dq product, wave w = d slice 128w .. 128w+127 for all 64 heads, k = the block's 32 slots:
  //  A = dS (transposed read of PT[slot][head]), rows 8g + c16/4 (lo) and +4 (hi);
  //  B = row tile read transposed, the same rows, column 128w + 16nt + 4(c16 & 3) at
  //      128w + (16nt ^ 8((c16 & 3)/2 ^ s)) + 4(c16 & 1) with s the row's swizzle
  const int trr = 8 * g + (c16 >> 2), tre = (c16 & 3) >> 1, troff = 4 * (c16 & 1);
  const int klo_s = 8 * (tre ^ swz(trr)), khi_s = 8 * (tre ^ swz(trr + 4));

  uint16_t* pds_t = b.pds + (int64_t)tl * b.n_slots * 128;
  auto store_pds = [&](int blk) {   // slots of block blk from PT[blk & 1], 16-byte stores
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid + 256 * k, s = e >> 4, cc = e & 15;
      *reinterpret_cast<uint4*>(pds_t + (int64_t)(kNB1 * blk + s) * 128 + 8 * cc) =
          *reinterpret_cast<const uint4*>(&PT[blk & 1][s][8 * cc]);
    }
  };

  int rid_cur = rid_of(0, raw_cur), rid_nxt = rid_of(1, raw_nxt);
  if (nblk > 0) issue(rid_cur, 0);
  wait_vmem();
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    const uint32_t valid = (uint32_t)__ballot(rid_cur != -1);
    const bool more = blk + 1 < nblk;
    const int raw_nn = raw_of(blk + 2);
    if (blk > 0) store_pds(blk - 1);
    // ---- S^T, dP^T for 32 candidates x this wave's 16 heads (operands read 3 steps ahead)
    f32x4 st[2], gt[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) st[mt] = gt[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      const uint16_t* rb = &Kt[buf][c16][0];
      auto seg = [&](int ks, int mt) { return ld16(rb + 16 * mt * kD + 128 * (ks >> 2) + eq[ks & 3]); };
      constexpr int kPre = 3;
      bf16x8 av[kPre][2];
#pragma unroll
      for (int j = 0; j < kPre; ++j)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) av[j][mt] = seg(j, mt);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          st[mt] = mfma16(av[ks % kPre][mt], qb[ks], st[mt]);
          gt[mt] = mfma16(av[ks % kPre][mt], gb[ks], gt[mt]);
        }
        if (ks + kPre < 16) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) av[ks % kPre][mt] = seg(ks + kPre, mt);
        }
        // the next block's rows, one per two k-steps, between the MFMAs
        if (more && (ks & 1)) issue_row(rid_nxt, buf ^ 1, ks >> 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- P, scale*dS for slots 16mt + 4g + i, head h -> PT (bf16)
    uint32_t dsw[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float pv[4], dv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cl = 16 * mt + 4 * g + i;
        const bool ok = (valid >> cl) & 1;
        pv[i] = ok ? __builtin_amdgcn_exp2f(st[mt][i] * b.scale_log2 - lse2) : 0.f;
        dv[i] = ok ? b.scale * pv[i] * (gt[mt][i] - dt) : 0.f;
      }
      dsw[2 * mt] = pack_bf16x2(dv[0], dv[1]);
      dsw[2 * mt + 1] = pack_bf16x2(dv[2], dv[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cl = 16 * mt + 4 * g + i;
        const uint32_t wd = dsw[2 * mt + (i >> 1)], wp = pack_bf16x2(pv[i], 0.f);
        PT[buf][cl][h] = (uint16_t)((i & 1) ? (wd >> 16) : (wd & 0xffffu));
        PT[buf][cl][64 + h] = (uint16_t)(wp & 0xffffu);
      }
    }
    __syncthreads();   // dS of all heads in PT[buf]
    // ---- dq[h][d] += sum_c dS[h][c] K[c][d] over this block's 32 slots
    {
      bf16x8 da[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        da[mt] = join8(ld_tr(&PT[buf][trr][16 * mt + 4 * (c16 & 3)]),
                       ld_tr(&PT[buf][trr + 4][16 * mt + 4 * (c16 & 3)]));
      const uint16_t* klo = &Kt[buf][trr][128 * wave + troff];
      const uint16_t* khi = &Kt[buf][trr + 4][128 * wave + troff];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bf16x8 kb = join8(ld_tr(klo + ((16 * nt) ^ klo_s)), ld_tr(khi + ((16 * nt) ^ khi_s)));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) dq[mt][nt] = mfma16(da[mt], kb, dq[mt][nt]);
      }
    }
    wait_vmem();
    __syncthreads();
    rid_cur = rid_nxt;
    rid_nxt = rid_of(blk + 2, raw_nn);
  }
  if (nblk > 0) store_pds(nblk - 1);
  // ---- dq (bf16) through LDS as [head][d] (swizzled rows), then full-row stores
  uint16_t* dqt = &Kt[0][0][0];   // 64 rows x 1 KiB = both tile buffers
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hr = 16 * mt + 4 * g + i;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int d = 128 * wave + 16 * nt + c16;
        dqt[hr * kD + 8 * ((d >> 3) ^ swz(hr)) + (d & 7)] =
            (uint16_t)(pack_bf16x2(dq[mt][nt][i], 0.f) & 0xffffu);
      }
    }
  __syncthreads();
  uint16_t* dqp = b.dq + (int64_t)t * kH * kD;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = tid + 256 * k, hr = e >> 6, cc = e & 63;
    *reinterpret_cast<uint4*>(dqp + hr * kD + 8 * cc) =
        *reinterpret_cast<const uint4*>(&dqt[hr * kD + 8 * (cc ^ swz(hr))]);
  }
  if (b.sink && b.dsink && g == 0)
    atomicAdd(b.dsink + h, -expf(b.sink[h] - lse_t) * dt);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_attn_bwd_dkv_mfma(BwdArgs b) {
  // LDS, sized for two workgroups per CU: Q, then dO, of the token staged in turn (64 rows
  // each, read transposed into registers); then one output tile of 32 rows x 1 KiB and two
  // dS|P tiles of 32 rows x 256 bytes (all rows chunk-swizzled)
  __shared__ __attribute__((aligned(16))) uint16_t lds[kH * kKS];
  uint16_t (*QO)[kKS] = reinterpret_cast<uint16_t (*)[kKS]>(lds);
  uint16_t (*OT)[kD] = reinterpret_cast<uint16_t (*)[kD]>(lds);
  uint16_t (*PS)[kNB3][128] = reinterpret_cast<uint16_t (*)[kNB3][128]>(lds + kNB3 * kD);
  static_assert(kNB3 * kD + 2 * kNB3 * 128 <= kH * kKS, "output and dS|P tiles fit");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int tl = token_of_block(blockIdx.x);
  if (tl >= b.nT) return;
  const int t = b.t0 + tl;
  TokenInfo ti;
  if (!token_info_wave(b.cu, b.B, t, ti)) return;
  const int n_tot = b.nc[t] + min(b.W, ti.p + 1);
  const int nblk = (n_tot + kNB3 - 1) / kNB3;
  const uint16_t* pds_t = b.pds + (int64_t)tl * b.n_slots * 128;
  uint16_t* stg_t = b.stage + (int64_t)tl * b.n_slots * kD;
  const int dw = wave * kDW;
  const int jr = c16 >> 2, jc = 4 * (c16 & 3);
  // [Q; dO] read transposed: MFMA A operand with m = d, k = head slot (Q heads in k-steps
  // 0, 1; dO heads in k-steps 2, 3), staged 64 rows at a time
  bf16x8 bo[8][4];   // [tile of d][k-step over the 128 head slots]
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint16_t* src = (half == 0 ? b.q : b.dout) + (int64_t)t * kH * kD;
    if (half) __syncthreads();       // every wave has read the Q rows
#pragma unroll 8
    for (int j = 0; j < 16; ++j) {
      const int row = 16 * wave + j;
      dma_row16(src + row * kD + 8 * lane, &QO[row][0]);
    }
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const v4i16 lo = ld_tr(&QO[32 * k2 + 8 * g + jr][dw + 16 * nt + jc]);
        const v4i16 hi = ld_tr(&QO[32 * k2 + 8 * g + 4 + jr][dw + 16 * nt + jc]);
        bo[nt][2 * half + k2] = join8(lo, hi);
      }
  }
  __syncthreads();   // QO no longer read: its space becomes the output and dS|P tiles
  // dS|P rows of block blk into PS[buf]: 4 rows of 256 bytes per instruction, wave w rows
  // 8w .. 8w+7, lane l fills physical chunk l % 16 of row 4i + l / 16
  auto issue = [&](int blk, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * wave + 4 * i + (lane >> 4);
      dma_row16(pds_t + (int64_t)(kNB3 * blk + r) * 128 + 8 * ((lane & 15) ^ swz(r)),
                &PS[buf][8 * wave + 4 * i][0]);
    }
  };
  // B operand reads: row 16mt + c16, logical chunk 4ks + g
  int eq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) eq[q] = 8 * ((4 * q + g) ^ swz(c16));
  if (nblk > 0) issue(0, 0);
  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1, c0 = kNB3 * blk;
    // this block's dS|P rows: after block 0 the only younger memory operations are the
    // previous (full) block's 8 row stores, which may stay in flight
    if (blk == 0) wait_vmem();
    else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __syncthreads();
    if (blk + 1 < nblk) issue(blk + 1, buf ^ 1);
    // row gradients of candidates c0 + 16mt + c16 -> OT[16mt + c16][d], chunk-swizzled
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int row = 16 * mt + c16;
      bf16x8 av[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) av[ks] = ld16(&PS[buf][row][eq[ks]]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) x = mfma16(bo[nt][ks], av[ks], x);
        // lane holds d = dw + 16nt + 4g .. +3 (logical chunk (dw + 16nt)/8 + g/2)
        const int ck = ((dw + 16 * nt) >> 3) + (g >> 1);
        *reinterpret_cast<uint2*>(&OT[row][8 * (ck ^ swz(row)) + 4 * (g & 1)]) =
            make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
      }
    }
    __syncthreads();
    // full-row 16-byte stores: wave w writes rows w, w+4, ...
    const int nrow = min(kNB3, n_tot - c0);
    for (int r = wave; r < nrow; r += 4)
      *reinterpret_cast<uint4*>(stg_t + (int64_t)(c0 + r) * kD + 8 * lane) =
          *reinterpret_cast<const uint4*>(&OT[r][8 * (lane ^ swz(r))]);
  }
}

// ---- CSR of the compressed rows of a chunk: count, scan, fill
__global__ __launch_bounds__(256) void k_bwd_fill_zero(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

template <bool FILL>
__global__ __launch_bounds__(256) void k_bwd_csr_pass(BwdArgs b) {
  CsrBuild g;
  g.idx = b.mode == 0 ? b.idx : nullptr; g.cu = b.cu; g.cu_cmp = b.cu_cmp; g.nc = b.nc;
  g.cnt = b.cnt; g.cur = b.cur; g.list = b.list; g.slots = b.n_slots; g.t0 = b.t0;
  g.nT = b.nT; g.B = b.B; g.r = b.r; g.n_cap = b.n_cap; g.k_cap = b.k_cap;
  csr_group_pass<FILL>(g);
}

// exclusive scan of cnt[0 .. n) into off and cur (one workgroup of 1024 lanes)
__global__ __launch_bounds__(1024) void k_bwd_csr_scan(BwdArgs b, int n) {
  __shared__ int part[1024];
  const int per = (n + 1023) / 1024;
  const int lo = threadIdx.x * per, hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += b.cnt[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;
  for (int i = lo; i < hi; ++i) {
    b.off[i] = run;
    b.cur[i] = run;
    run += b.cnt[i];
  }
}

// ---- owner-side reductions: 4 groups of 64 lanes, each lane owns 8 consecutive floats
__device__ __forceinline__ void add_staged(const uint16_t* src, float (&acc)[8]) {
  float v[8];
  load8(src, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] += v[i];
}

__device__ __forceinline__ void finish_row(float (&acc)[8], float* __restrict__ dst, float* red) {
  const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) red[(q * 64 + lane) * 9 + i] = acc[i];
  __syncthreads();
  if (q == 0) {
    float o[8];
    load8(dst + 8 * lane, o);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      o[i] += (acc[i] + red[(64 + lane) * 9 + i]) + (red[(128 + lane) * 9 + i] + red[(192 + lane) * 9 + i]);
    store8(dst + 8 * lane, o);
  }
}

__global__ __launch_bounds__(256) void k_bwd_reduce_cmp(BwdArgs b) {
  __shared__ float red[256 * 9];
  const int j = blockIdx.x;
  const int n = b.cnt[j];
  if (n == 0) return;
  const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int* lst = b.list + b.off[j];
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // wave q takes list entries 64q .. 64q + 63, then 64q + 256 .., each batch read with one
  // coalesced load and broadcast from registers; 8 staged rows in flight per wave
  for (int base = 64 * q; base < n; base += 256) {
    const int my = base + lane < n ? lst[base + lane] : 0;
    const int m = min(64, n - base);
    for (int k = 0; k < m; k += 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = __shfl(my, k + u, 64);
        v[u] = k + u < m ? *reinterpret_cast<const uint4*>(b.stage + (int64_t)e * kD + 8 * lane)
                         : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float f[8];
        load8(reinterpret_cast<const uint16_t*>(&v[u]), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += f[i];
      }
    }
  }
  finish_row(acc, b.dkv_cmp + (int64_t)j * kD, red);
}

// raw rows u in [u_lo, u_lo + gridDim.x): contributors are the queries t in [u, u + W - 1]
// of u's sample that lie in this chunk; u is slot nc[t] + (u - first window row of t)
__global__ __launch_bounds__(256) void k_bwd_reduce_win(BwdArgs b, int u_lo) {
  __shared__ float red[256 * 9];
  const int u = u_lo + blockIdx.x;
  TokenInfo ti;
  if (!token_info(b.cu, b.B, u, ti)) return;
  const int t_lo = max(u, b.t0);
  const int t_hi = min(min(u + b.W - 1, ti.start + ti.len - 1), b.t0 + b.nT - 1);
  if (t_lo > t_hi) return;
  const int q = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  // wave q takes contributors t_lo + q, t_lo + q + 4, ..., eight staged rows in flight
  for (int t0 = t_lo + q; t0 <= t_hi; t0 += 32) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = t0 + 4 * k;
      v[k] = make_uint4(0, 0, 0, 0);
      if (t <= t_hi) {
        const int p = t - ti.start;
        const int win0 = t - min(b.W, p + 1) + 1;
        const int64_t slot = (int64_t)(t - b.t0) * b.n_slots + b.nc[t] + (u - win0);
        v[k] = *reinterpret_cast<const uint4*>(b.stage + slot * kD + 8 * lane);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float f[8];
      load8(reinterpret_cast<const uint16_t*>(&v[k]), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
  }
  finish_row(acc, b.dkv + (int64_t)u * kD, red);
}

namespace {

struct BwdPlan {
  bool keys;   // shared-row gradients by the key-major pass (else staged rows + CSR sums)
  int64_t n_slots, n_c_max, chunk, Tc_cap, cap;
  size_t off_pds, off_stage, off_nc, off_cnt, off_off, off_cur, off_list;
  size_t off_items, off_ipart, off_red, off_part, total;
};

// The key-major pass does dense masked products over every (query, row) pair a query sees,
// where the staged path moves one 1 KiB row gradient per attended pair through HBM twice;
// it is taken unless a query attends only a small share of the compressed rows it sees
// (top-k well below the visible count), for all-visible and window-only layers, and while the
// per-sample block tables fit.
bool keys_path(const Shape& sh) {
  const int64_t n_cap = sh.r > 0 ? sh.max_seqlen / sh.r : 0;
  if (sh.mode == 2) return true;
  if (n_cap / 128 + 1 > 2048) return false;
  if (sh.mode == 1) return true;
  return sh.k_cap <= 2048 && n_cap <= 6ll * sh.k_cap;
}

// Workspace layout for chunks of `chunk` query tokens.
BwdPlan bwd_layout(const Shape& sh, int64_t chunk) {
  BwdPlan p = {};
  p.keys = keys_path(sh);
  p.n_c_max = sh.mode == 0 ? sh.k_cap : (sh.mode == 1 ? sh.max_seqlen / sh.r : 0);
  p.n_slots = ((p.n_c_max + sh.W + kNB2 - 1) / kNB2) * kNB2;
  p.chunk = chunk;
  p.Tc_cap = sh.r > 0 ? sh.T / sh.r + 1 : 1;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o = 0;
  p.off_pds = o;   o = al(o + (size_t)p.chunk * p.n_slots * 128 * 2);
  p.off_nc = o;    o = al(o + (size_t)sh.T * 4);
  if (p.keys) {
    const int n_cap = sh.mode == 2 ? 0 : sh.max_seqlen / sh.r;
    p.cap = keys::item_cap(sh.mode, sh.B, (int)chunk, n_cap, sh.W, 128);
    p.off_cnt = o;   o = al(o + 128 * 4);   // 64 counters, then 256 zero bytes
    p.off_items = o; o = al(o + (size_t)p.cap * 16);
    p.off_ipart = o; o = al(o + (size_t)p.cap * 4);
    p.off_red = o;   o = al(o + (size_t)p.cap * 16);
    p.off_part = o;  o = al(o + (size_t)p.cap * 128 * kD * 4);
  } else {
    p.off_stage = o; o = al(o + (size_t)p.chunk * p.n_slots * kD * 2);
    p.off_cnt = o;   o = al(o + (size_t)p.Tc_cap * 4);
    p.off_off = o;   o = al(o + (size_t)p.Tc_cap * 4);
    p.off_cur = o;   o = al(o + (size_t)p.Tc_cap * 4);
    p.off_list = o;  o = al(o + (size_t)p.chunk * (p.n_c_max > 0 ? p.n_c_max : 1) * 4);
  }
  p.total = o;
  return p;
}

// The largest chunk whose layout fits in `budget` bytes (the layout grows with the chunk):
// every query at once if that fits, else the largest whole multiple of the XCD token mapping
// (8 * kChunk tokens), else of the CSR group; at least one group (its total then exceeds a
// budget below the minimum; the caller checks).
BwdPlan bwd_plan(const Shape& sh, size_t budget) {
  const int64_t T = sh.T > 0 ? sh.T : 1;
  BwdPlan p = bwd_layout(sh, T);
  if (p.total <= budget || T <= kCsrGroup) return p;
  auto largest = [&](int64_t unit, int64_t hi) {   // largest m * unit < hi that fits, or 0
    int64_t lo = 0, up = (hi - 1) / unit;            // answer in [lo, up] units
    while (lo < up) {
      const int64_t mid = (lo + up + 1) / 2;
      if (bwd_layout(sh, mid * unit).total <= budget) lo = mid;
      else up = mid - 1;
    }
    return lo * unit;
  };
  int64_t ch = largest(8 * kChunk, T);
  if (ch == 0) ch = largest(kCsrGroup, T < 8 * kChunk ? T : 8 * kChunk);
  if (ch == 0) ch = kCsrGroup;
  return bwd_layout(sh, ch);
}

// Preferred workspace: chunks of up to kStageBudget bytes of per-pair storage (one chunk for
// a 64K batch: one launch tail per kernel per step).
size_t bwd_preferred(const Shape& sh) {
  const BwdPlan one = bwd_layout(sh, 1);
  const int64_t per_tok = one.n_slots * (one.keys ? 128 * 2 : (128 + kD) * 2);
  int64_t ch = kStageBudget / per_tok;
  ch = (ch / (8 * kChunk)) * (8 * kChunk);
  if (ch < 8 * kChunk) ch = 8 * kChunk;
  return bwd_layout(sh, ch < sh.T ? ch : (sh.T > 0 ? sh.T : 1)).total;
}

}  // namespace

size_t attn_bwd_workspace_mfma(const Shape& sh) {
  if (sh.dtype != 1 || sh.H != kH || sh.D != kD) return 0;
  return bwd_preferred(sh);
}

size_t attn_bwd_workspace_min_mfma(const Shape& sh) {
  if (sh.dtype != 1 || sh.H != kH || sh.D != kD) return 0;
  return bwd_layout(sh, sh.T < kCsrGroup ? (sh.T > 0 ? sh.T : 1) : kCsrGroup).total;
}

hipError_t launch_attn_bwd_mfma(const Shape& sh, const AttnIO& io, hipStream_t s, bool* handled) {
  *handled = false;
  if (sh.dtype != 1 || sh.H != kH || sh.D != kD) return hipSuccess;
  *handled = true;
  const size_t pref = bwd_preferred(sh);
  const BwdPlan pl = bwd_plan(sh, io.ws_bytes < pref ? io.ws_bytes : pref);
  if (pl.total > io.ws_bytes) return hipErrorInvalidValue;   // below the minimum: host-checked
  char* ws = (char*)io.ws;
  BwdArgs b;
  b.q = (const uint16_t*)io.q;
  b.kv_cmp = (const uint16_t*)io.kv_cmp;
  b.kv = (const uint16_t*)io.kv;
  b.idx = io.idx;
  b.sink = io.sink;
  b.cu = sh.cu;
  b.cu_cmp = sh.cu_cmp;
  b.o = (const uint16_t*)io.o;
  b.lse = io.lse;
  b.dout = (const uint16_t*)io.dout;
  b.dq = (uint16_t*)io.dq;
  b.dkv_cmp = io.dkv_cmp;
  b.dkv = io.dkv;
  b.dsink = io.dsink;
  b.pds = (uint16_t*)(ws + pl.off_pds);
  b.stage = (uint16_t*)(ws + pl.off_stage);
  b.nc = (int32_t*)(ws + pl.off_nc);
  b.cnt = (int32_t*)(ws + pl.off_cnt);
  b.off = (int32_t*)(ws + pl.off_off);
  b.cur = (int32_t*)(ws + pl.off_cur);
  b.list = (int32_t*)(ws + pl.off_list);
  b.n_slots = pl.n_slots;
  b.Tc_cap = (int)pl.Tc_cap;
  b.B = sh.B;
  b.T = sh.T;
  b.r = sh.r;
  b.n_cap = sh.max_seqlen / sh.r;
  b.W = sh.W;
  b.k_cap = sh.k_cap;
  b.mode = sh.mode;
  b.scale = sh.scale;
  b.scale_log2 = sh.scale * 1.44269504088896341f;
  KeysArgs ka = {};
  if (pl.keys) {
    ka.q = b.q;
    ka.dout = b.dout;
    ka.pds = b.pds;
    ka.idx = sh.mode == 0 ? io.idx : nullptr;
    ka.nc = b.nc;
    ka.cu = sh.cu;
    ka.cu_cmp = sh.cu_cmp;
    ka.counters = (int32_t*)(ws + pl.off_cnt);
    ka.zeros = (const uint16_t*)(ws + pl.off_cnt + 64 * 4);
    ka.items = (int4*)(ws + pl.off_items);
    ka.item_part = (int32_t*)(ws + pl.off_ipart);
    ka.red = (int4*)(ws + pl.off_red);
    ka.part = (float*)(ws + pl.off_part);
    ka.dkv_cmp = io.dkv_cmp;
    ka.dkv = io.dkv;
    ka.n_slots = pl.n_slots;
    ka.cap = pl.cap;
    ka.B = sh.B;
    ka.r = sh.r;
    ka.n_cap = sh.mode == 2 ? 0 : sh.max_seqlen / sh.r;
    ka.W = sh.W;
    ka.k_cap = sh.k_cap;
    ka.mode = sh.mode;
    ka.D = kD;
    ka.KC = 128;
    ka.kb = 128;
  }
  for (int64_t t0 = 0; t0 < sh.T; t0 += pl.chunk) {
    b.t0 = (int)t0;
    b.nT = (int)(sh.T - t0 < pl.chunk ? sh.T - t0 : pl.chunk);
    const int64_t grid = token_grid(b.nT);
    if (pl.keys) {
      ka.t0 = b.t0;
      ka.nT = b.nT;
      hipLaunchKernelGGL(k_bwd_fill_zero, dim3(1), dim3(256), 0, s, ka.counters, 128);
      hipError_t e = launch_attn_bwd_keys(ka, s);
      if (e != hipSuccess) return e;
    }
    if (sh.mode != 0 || sh.k_cap <= kIdxLds)
      hipLaunchKernelGGL(k_attn_bwd_dq_mfma<true>, dim3((unsigned)grid), dim3(256), 0, s, b);
    else
      hipLaunchKernelGGL(k_attn_bwd_dq_mfma<false>, dim3((unsigned)grid), dim3(256), 0, s, b);
    if (pl.keys) {
      hipError_t e = launch_attn_bwd_keys_sums(ka, s);
      if (e != hipSuccess) return e;
      continue;
    }
    hipLaunchKernelGGL(k_attn_bwd_dkv_mfma, dim3((unsigned)grid), dim3(256), 0, s, b);
    if (sh.mode != 2) {
      hipLaunchKernelGGL(k_bwd_fill_zero, dim3(64), dim3(256), 0, s, b.cnt, b.Tc_cap);
      hipLaunchKernelGGL(k_bwd_csr_pass<false>, dim3(csr_grid(b.nT)), dim3(256), 0, s, b);
      hipLaunchKernelGGL(k_bwd_csr_scan, dim3(1), dim3(1024), 0, s, b, b.Tc_cap);
      hipLaunchKernelGGL(k_bwd_csr_pass<true>, dim3(csr_grid(b.nT)), dim3(256), 0, s, b);
      hipLaunchKernelGGL(k_bwd_reduce_cmp, dim3(b.Tc_cap), dim3(256), 0, s, b);
    }
    const int u_lo = b.t0 - sh.W + 1 > 0 ? b.t0 - sh.W + 1 : 0;
    const int u_hi = b.t0 + b.nT;          // exclusive
    hipLaunchKernelGGL(k_bwd_reduce_win, dim3(u_hi - u_lo), dim3(256), 0, s, b, u_lo);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa
