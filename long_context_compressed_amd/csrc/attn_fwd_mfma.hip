// Matrix-core (MFMA) sparse attention forward for bf16 operands, H = 64 heads sharing one
// D = 512 K=V row (MQA), on gfx950.
//
// Method ("DeepSeek-V4 Attention Training Systems", sections 2 and 8.2): each query
// attends its selected (or all visible) compressed rows plus its local raw window; the
// forward returns O, the log-sum-exp and, optionally, the log-sum-exp over the compressed
// candidates alone (the normalizer of the selected-set indexer teacher, section 3).
//
// Design: one workgroup of 8 waves per query token (two per SIMD, so one wave's gathers,
// softmax and waits overlap the other's MFMAs; 256 registers each); candidates are processed
// in blocks of 64 rows, double-buffered in LDS.
//   * Rows are gathered with direct global->LDS loads (global_load_lds_dwordx4, one 1 KiB
//     row per wave instruction) one block ahead, spread over the S^T k-steps so that they
//     land while the current block computes; the query's idx row is staged in LDS once.
//     LDS rows are 1 KiB with a 16-byte chunk swizzle, so both the row-segment reads of
//     S = Q K^T and the transposed reads of P V are bank-conflict free.
//   * S^T: wave (hh, ch) computes heads 16hh..16hh+15 against candidates 32ch..32ch+31 of
//     the block on v_mfma_f32_16x16x32_bf16 (A = row segments from LDS, B = the query's Q
//     of its 16 heads resident in registers).
//   * Online softmax per head with a lazily rescaled running max: the max is only moved
//     when it grows by more than 2^8, so most blocks skip the O rescale.  P (bf16) goes to
//     LDS.
//   * O^T: wave w owns d = 64w..64w+63 for all 64 heads: A = the row tile read transposed
//     (ds_read_b64_tr_b16), B = P^T from LDS.
//   * O is normalised, transposed through LDS and written with full-row 16-byte stores.
// Tokens map to workgroups so that each XCD walks contiguous 256-token chunks (its L2 then
// holds the compressed rows of one sample).
#include <math.h>

#include "attn_common.h"
#include "csa_launch.h"

// M0 is named as clobbered by the LDS-DMA asm below; the compiler keeps no value in it here.
#pragma clang diagnostic ignored "-Winline-asm"

namespace csa {

using namespace attn;

namespace {

constexpr int kNB = 64;        // candidates per block
constexpr int kPS = 72;        // P tile row stride (bf16)
constexpr float kLazy = 8.f;   // growth (log2 units) of the running max tolerated before rescaling
constexpr int kIdxLds = 2048;    // idx entries of a query staged in LDS
constexpr int kFwdWaves = 8;   // two waves per SIMD: each holds Q of 16 heads and 1/8 of O
constexpr int kFwdHeadGroups = 4;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* kv_cmp;
  const uint16_t* kv;
  const int32_t* idx;
  const float* sink;
  const int32_t* cu;
  const int32_t* cu_cmp;
  uint16_t* out;
  uint16_t* out_rot;  // optional: out inverse-rotated at the query position
  float* lse;
  float* lse_cmp;    // optional log-sum-exp over the compressed candidates only
  float* t_logits;   // optional compressed-candidate logits [T, H, ld_t]
  int64_t ld_t;
  int B, T, r, n_cap, W, k_cap, mode;
  float scale;
  float scale_log2;  // softmax scale * log2(e)
  int rope_dim;      // rotary band of out_rot
  double rope_l2t;   // log2(theta)
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// at most 2 vector memory operations outstanding (they complete in issue order)
__device__ __forceinline__ void wait_vmem_2() { asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); }

// One 16-byte-per-lane global -> LDS load (global_load_lds_dwordx4); lane l's 16 bytes land
// at LDS byte offset lds + 16 l.  Issued through asm so that the compiler does not order the
// LDS reads of the other tile buffer behind it: completion is awaited explicitly with
// wait_vmem() before the barrier that publishes the tile.
__device__ __forceinline__ void dma_row16(const void* src, const void* lds_row) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_row);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(src) : "memory", "m0");
}

// The same with the row address as a scalar base plus a per-lane byte offset (saddr form).
__device__ __forceinline__ void dma_row16_s(uint64_t row, uint32_t lane_off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(lane_off), "s"(row) : "memory", "m0");
}

}  // namespace

// NW waves per query: NHG head groups of HPW = 64/NHG heads times NCH = NW/NHG candidate
// groups of CPW = 64/NCH candidates for S^T, and d slices of DPW = 512/NW columns for O^T.
// IDX_LDS: the query's idx row (k_cap <= kIdxLds) is staged in LDS once, so that the block
// loop reads its next slots from LDS instead of issuing a global load per block.
template <int NW, int NHG, bool IDX_LDS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void k_attn_fwd_mfma(FwdArgs a) {
  constexpr int NT = NW * 64, NCH = NW / NHG, CPW = kNB / NCH, MQ = CPW / 16, DPW = kD / NW,
                MP = DPW / 16, RPW = kNB / NW, HPW = kH / NHG, NT2 = HPW / 16;
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kNB][kD];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[kH][kPS];
  __shared__ float mx_s[NCH][kH];
  __shared__ float alpha_s[kH];
  __shared__ float lsum_s[NCH][kH], lsnap_s[NCH][kH];
  __shared__ float mrun_s[kH], msnap_s[kH], fin_s[kH];
  __shared__ int resc_s[NHG];
  __shared__ int s_tmp;
  __shared__ float2 rope_s[kD / 2];   // cos, sin of the output rotation's pairs
  __shared__ int32_t idx_s[IDX_LDS ? kIdxLds : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int hh = wave % NHG, ch = wave / NHG;   // head group, candidate group
  const int t = token_of_block(blockIdx.x);
  if (t >= a.T) return;

  TokenInfo ti;
  if (!token_info_wave(a.cu, a.B, t, ti, a.cu_cmp)) {
    uint4* o = reinterpret_cast<uint4*>(a.out + (int64_t)t * kH * kD);
    for (int e = tid; e < kH * kD / 8; e += NT) o[e] = make_uint4(0, 0, 0, 0);
    if (a.out_rot) {
      uint4* orot = reinterpret_cast<uint4*>(a.out_rot + (int64_t)t * kH * kD);
      for (int e = tid; e < kH * kD / 8; e += NT) orot[e] = make_uint4(0, 0, 0, 0);
    }
    if (tid < kH) a.lse[(int64_t)t * kH + tid] = 0.f;
    if (a.lse_cmp && tid < kH) a.lse_cmp[(int64_t)t * kH + tid] = -INFINITY;
    return;
  }
  // the idx row first (into registers; to LDS once Q is in flight), so the first block's
  // gather waits for the idx loads alone, then Q^T as the B operand:
  // qb[nt][ks] = Q[HPW hh + 16nt + c16][32ks + 8g .. +7]
  const int32_t* idx_t = a.mode == 0 ? a.idx + (int64_t)t * a.k_cap : nullptr;
  int iv[IDX_LDS ? kIdxLds / NT : 1];
  if (IDX_LDS && a.mode == 0) load_idx_regs(idx_t, a.k_cap, iv);
  bf16x8 qb[NT2][16];
  {
    const uint16_t* qt = a.q + ((int64_t)t * kH + HPW * hh + c16) * kD + 8 * g;
#pragma unroll
    for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qb[nt][ks] = ld16(qt + 16 * nt * kD + 32 * ks);
  }
  if (IDX_LDS && a.mode == 0) store_idx_lds(idx_s, a.k_cap, iv);   // published by leading_valid_lds
  // raw idx entries of slot 64 b + lane; converted to row ids once the candidate counts are known
  auto raw_of = [&](int b) {
    const int c = kNB * b + lane;
    if (a.mode != 0 || c >= a.k_cap) return 0;
    return IDX_LDS ? idx_s[c] : idx_t[c];
  };
  if (a.out_rot) {
    // angles of the output's inverse rotation at this query's position, formed while the
    // Q loads are in flight: pair i on lane i / NW of wave i % NW (at most kD / 2 <= NT pairs)
    static_assert(kD / 2 <= NT, "one pair per thread");
    const int i = wave + NW * lane;
    if (i < a.rope_dim / 2) {
      float c, s;
      rope_cs(ti.p, i, a.rope_dim, a.rope_l2t, true, c, s);
      rope_s[i] = make_float2(c, s);
    }
  }

  CandSet cs;
  cs.row0 = ti.c0;
  cs.nv = min((ti.p + 1) / a.r, a.n_cap);
  cs.n_w = min(a.W, ti.p + 1);
  cs.win0 = t - cs.n_w + 1;
  if (a.mode == 1) cs.n_c = cs.nv;
  else if (a.mode == 2) cs.n_c = 0;
  else if (IDX_LDS) cs.n_c = leading_valid_lds(idx_s, a.k_cap, &s_tmp);   // publishes idx_s
  else cs.n_c = leading_valid(idx_t, a.k_cap, &s_tmp);
  int raw_cur = raw_of(0);
  int raw_nxt = raw_of(1);
  // compressed slots padded to whole blocks, so a block never mixes compressed and window
  // rows and the compressed-only normalizer can be read off after the last compressed block
  cs.n_cs = ((cs.n_c + kNB - 1) / kNB) * kNB;
  const int nblk = (cs.n_cs + cs.n_w + kNB - 1) / kNB;

  f32x4 o[MP][4];   // O^T: d = DPW wave + 16 mt + 4g + i, head = 16 nt + c16
#pragma unroll
  for (int mt = 0; mt < MP; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  float m_run[NT2], l_part[NT2], m_snap[NT2], l_snap[NT2];
#pragma unroll
  for (int nt = 0; nt < NT2; ++nt) {
    m_run[nt] = m_snap[nt] = -INFINITY;
    l_part[nt] = l_snap[nt] = 0.f;
  }

  // row-segment reads of S^T: logical chunk 4ks + g of row CPW ch + 16 mq + c16 sits at
  // physical chunk 16 (ks / 4) + ((4 (ks % 4) + g) ^ swz(c16))
  int eq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) eq[q] = 8 * ((4 * q + g) ^ swz(c16));
  // transposed reads of P V: logical chunk DPW/8 wave + 2 mt + (c16 & 3) / 2 of rows
  // 32ks + 8g + c16/4 (lo) and +4 (hi), at physical chunk (DPW/8 wave + e + 2 mt) ^ s; the
  // three terms occupy disjoint bits, so 8 (that) = 8 ((DPW/8 wave + e) ^ s) ^ 16 mt
  const int tr_e = (c16 & 3) >> 1, tr_off = 4 * (c16 & 1);
  const int klo = 8 * (((DPW / 8) * wave + tr_e) ^ swz(8 * (g & 1) + (c16 >> 2)));
  const int khi = 8 * (((DPW / 8) * wave + tr_e) ^ swz(8 * (g & 1) + 4 + (c16 >> 2)));

  // row id of slot 64 b + lane: >= 0 compressed row, <= -2 raw row -2 - id, -1 none
  auto rid_of = [&](int b, int raw) {
    const int c = kNB * b + lane;
    if (b >= nblk) return -1;
    if (c < cs.n_c) {
      const int gr = a.mode == 1 ? cs.row0 + c : raw;
      return (gr >= cs.row0 && gr < cs.row0 + cs.nv) ? gr : -1;
    }
    if (c < cs.n_cs) return -1;
    if (c < cs.n_cs + cs.n_w) return -2 - (cs.win0 + (c - cs.n_cs));
    return -1;
  };
  // gather block rows RPW wave .. RPW wave + RPW - 1 into tile[buf] (lane l fills physical
  // chunk l); an absent slot loads the query's own raw row (finite, masked out by the softmax)
  auto issue_row = [&](int rid, int buf, int j) {
    const int r = RPW * wave + j;
    const int id = __builtin_amdgcn_readlane(rid, r);
    const uint16_t* src = id >= 0 ? a.kv_cmp + (int64_t)id * kD
                                  : a.kv + (int64_t)(id == -1 ? t : -2 - id) * kD;
    dma_row16(src + 8 * (lane ^ swz(r)), &tile[buf][r][0]);
  };
  auto issue = [&](int rid, int buf) {
#pragma unroll
    for (int j = 0; j < RPW; ++j) issue_row(rid, buf, j);
  };
  // the next block's rows are gathered one per S^T k-step, so the loads overlap the MFMAs
  // instead of stalling the wave at the block start: lane l holds the source of slot l, row
  // RPW wave + j is read with two lane reads; swz(row) depends on the row's low 4 bits only
  static_assert(RPW == 16 || RPW == 8, "one row per one or two S^T k-steps");
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const uint32_t tile_lds = (uint32_t)(uintptr_t)&tile[0][0][0];
  auto row_addr = [&](int rid) {
    return (uint64_t)(uintptr_t)(rid >= 0 ? a.kv_cmp + (int64_t)rid * kD
                                          : a.kv + (int64_t)(rid == -1 ? t : -2 - rid) * kD);
  };

  int rid_cur = rid_of(0, raw_cur);
  int rid_nxt = rid_of(1, raw_nxt);
  if (nblk > 0) issue(rid_cur, 0);
  wait_vmem();
  __syncthreads();

  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    const uint64_t valid = __ballot(rid_cur != -1);
    const bool more = b + 1 < nblk;
    const uint64_t nsrc = row_addr(rid_nxt);
    const uint32_t nlds = __builtin_amdgcn_readfirstlane(tile_lds + (buf ^ 1) * (kNB * kD * 2) +
                                                         RPW * wave * (kD * 2));
    auto gather = [&](int j) {   // row RPW wave + j of the next block
      const int r = RPW * wave + j;
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)nsrc, r);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(nsrc >> 32), r);
      dma_row16_s(((uint64_t)hi << 32) | lo, lane16 ^ (16u * swz(RPW * wave + j)), nlds + j * (kD * 2));
    };
    const int raw_nn = raw_of(b + 2);   // consumed after this block's final wait

    // ---- S^T: candidates CPW ch + 16 mq + 4g + i, heads HPW hh + 16nt + c16
    f32x4 st[MQ][NT2];
#pragma unroll
    for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
      for (int nt = 0; nt < NT2; ++nt) st[mq][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      // operands read kPre k-steps ahead of the MFMAs that consume them
      const uint16_t* rb = &tile[buf][CPW * ch + c16][0];
      auto seg = [&](int ks, int mq) { return ld16(rb + 16 * mq * kD + 128 * (ks >> 2) + eq[ks & 3]); };
      constexpr int kPre = 3;
      bf16x8 av[kPre][MQ];
#pragma unroll
      for (int j = 0; j < kPre; ++j)
#pragma unroll
        for (int mq = 0; mq < MQ; ++mq) av[j][mq] = seg(j, mq);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mq = 0; mq < MQ; ++mq)
#pragma unroll
          for (int nt = 0; nt < NT2; ++nt) st[mq][nt] = mfma16(av[ks % kPre][mq], qb[nt][ks], st[mq][nt]);
        if (more && (RPW == 16 || (ks & 1))) gather(RPW == 16 ? ks : ks >> 1);
        if (ks + kPre < 16) {
#pragma unroll
          for (int mq = 0; mq < MQ; ++mq) av[ks % kPre][mq] = seg(ks + kPre, mq);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // compressed blocks: keep the logits for the indexer teacher (16-byte stores of four
    // consecutive slots of one head)
    const bool t_store = a.t_logits && kNB * b < cs.n_cs;
    if (t_store) {
#pragma unroll
      for (int nt = 0; nt < NT2; ++nt) {
        float* dst = a.t_logits + ((int64_t)t * kH + HPW * hh + 16 * nt + c16) * a.ld_t +
                     kNB * b + CPW * ch + 4 * g;
#pragma unroll
        for (int mq = 0; mq < MQ; ++mq)
          *reinterpret_cast<f32x4*>(dst + 16 * mq) = st[mq][nt] * a.scale;
      }
    }
    // candidate validity of this lane's slots
    const uint32_t vbits = (uint32_t)(valid >> (CPW * ch + 4 * g));
    float s[NT2][4 * MQ];
#pragma unroll
    for (int nt = 0; nt < NT2; ++nt) {
      float mloc = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4 * MQ; ++j) {
        const int bit = 16 * (j >> 2) + (j & 3);
        s[nt][j] = ((vbits >> bit) & 1) ? st[j >> 2][nt][j & 3] * a.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, s[nt][j]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      if (g == 0) mx_s[ch][HPW * hh + 16 * nt + c16] = mloc;
    }
    __syncthreads();

    // ---- softmax of this block: P (bf16) and the per-head rescale factors
    bool any_resc = false;
#pragma unroll
    for (int nt = 0; nt < NT2; ++nt) {
      const int h = HPW * hh + 16 * nt + c16;
      float mb = mx_s[0][h];
#pragma unroll
      for (int c = 1; c < NCH; ++c) mb = fmaxf(mb, mx_s[c][h]);
      float alpha = 1.f;
      if (mb > m_run[nt] + kLazy) {
        alpha = __builtin_amdgcn_exp2f(m_run[nt] - mb);
        m_run[nt] = mb;
        any_resc = true;
      }
      float p[4 * MQ], sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4 * MQ; ++j) {
        const int bit = 16 * (j >> 2) + (j & 3);
        p[j] = ((vbits >> bit) & 1) ? __builtin_amdgcn_exp2f(s[nt][j] - m_run[nt]) : 0.f;
        sum += p[j];
      }
      l_part[nt] = l_part[nt] * alpha + sum;
#pragma unroll
      for (int mq = 0; mq < MQ; ++mq)
        *reinterpret_cast<uint2*>(&Ps[h][CPW * ch + 16 * mq + 4 * g]) =
            make_uint2(pack_bf16x2(p[4 * mq], p[4 * mq + 1]), pack_bf16x2(p[4 * mq + 2], p[4 * mq + 3]));
      if (ch == 0 && g == 0) alpha_s[h] = alpha;
      if (kNB * (b + 1) == cs.n_cs) {
        m_snap[nt] = m_run[nt];
        l_snap[nt] = l_part[nt];
      }
    }
    if (ch == 0) {
      const uint64_t r = __ballot(any_resc);
      if (lane == 0) resc_s[hh] = r != 0;
    }
    __syncthreads();

    // ---- O^T[d, h] = alpha_h O^T + V^T P^T over this block
    bool resc = false;
#pragma unroll
    for (int k = 0; k < NHG; ++k) resc = resc || resc_s[k];
    if (resc) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float al = alpha_s[16 * nt + c16];
#pragma unroll
        for (int mt = 0; mt < MP; ++mt) o[mt][nt] *= al;
      }
    }
    {
      // unit u = (ks, mt) = (u / MP, u % MP); its transposed row reads are issued two units
      // ahead of its MFMAs, the P^T operands of k-step 1 during unit 0
      const uint16_t* vb = &tile[buf][8 * g + (c16 >> 2)][tr_off];
      static_assert(DPW % 16 == 0 && DPW <= 128, "d slices of whole 16-column tiles");
      auto tr_lo = [&](int u) { return ld_tr(vb + 32 * (u / MP) * kD + ((16 * (u % MP)) ^ klo)); };
      auto tr_hi = [&](int u) { return ld_tr(vb + (32 * (u / MP) + 4) * kD + ((16 * (u % MP)) ^ khi)); };
      bf16x8 pb[2][4];
      v4i16 vlo[2], vhi[2];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) pb[0][nt] = ld16(&Ps[16 * nt + c16][8 * g]);
      vlo[0] = tr_lo(0);
      vhi[0] = tr_hi(0);
      vlo[1] = tr_lo(1);
      vhi[1] = tr_hi(1);
#pragma unroll
      for (int u = 0; u < 2 * MP; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        const int ks = u / MP, mt = u % MP;
        const bf16x8 va = join8(vlo[u & 1], vhi[u & 1]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[mt][nt] = mfma16(va, pb[ks][nt], o[mt][nt]);
        if (u + 2 < 2 * MP) {
          vlo[u & 1] = tr_lo(u + 2);
          vhi[u & 1] = tr_hi(u + 2);
        }
        if (u == 0) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) pb[1][nt] = ld16(&Ps[16 * nt + c16][32 + 8 * g]);
        }

      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next block's rows, gathered in the S^T loop: younger than them are only this block's
    // teacher-logit stores (NT2 x MQ = 2 per lane), which may stay in flight
    static_assert(NT2 * MQ == 2, "the wait below counts the teacher-logit stores");
    if (t_store) wait_vmem_2();
    else wait_vmem();
    __syncthreads();
    rid_cur = rid_nxt;
    rid_nxt = rid_of(b + 2, raw_nn);
  }

  // ---- finalize: per-head normalizers (with the optional sink), lse, lse_cmp
#pragma unroll
  for (int nt = 0; nt < NT2; ++nt) {
    float lt = l_part[nt], ls = l_snap[nt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    if (g == 0) {
      const int h = HPW * hh + 16 * nt + c16;
      lsum_s[ch][h] = lt;
      lsnap_s[ch][h] = ls;
      if (ch == 0) {
        mrun_s[h] = m_run[nt];
        msnap_s[h] = m_snap[nt];
      }
    }
  }
  __syncthreads();
  if (tid < kH) {
    const int h = tid;
    const float ln2 = 0.69314718055994531f;
    const float m = mrun_s[h];
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) l += lsum_s[c][h];
    float mf = m, lf = l;
    if (a.sink) {
      const float sk = a.sink[h] * 1.44269504088896341f;
      mf = fmaxf(m, sk);
      lf = (l > 0.f ? l * exp2f(m - mf) : 0.f) + exp2f(sk - mf);
    }
    a.lse[(int64_t)t * kH + h] = (mf + log2f(lf)) * ln2;
    fin_s[h] = l > 0.f ? exp2f(m - mf) / lf : 0.f;
    if (a.lse_cmp) {
      float lc = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) lc += lsnap_s[c][h];
      a.lse_cmp[(int64_t)t * kH + h] = lc > 0.f ? (msnap_s[h] + log2f(lc)) * ln2 : -INFINITY;
    }
  }
  __syncthreads();
  // O (bf16) -> LDS as [h][d] with the row swizzle, then full-row stores
  uint16_t* ot = &tile[0][0][0];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int h = 16 * nt + c16;
    const float f = fin_s[h];
#pragma unroll
    for (int mt = 0; mt < MP; ++mt) {
      const int d = DPW * wave + 16 * mt + 4 * g;
      *reinterpret_cast<uint2*>(&ot[h * kD + 8 * ((d >> 3) ^ swz(h)) + (d & 7)]) =
          make_uint2(pack_bf16x2(o[mt][nt][0] * f, o[mt][nt][1] * f),
                     pack_bf16x2(o[mt][nt][2] * f, o[mt][nt][3] * f));
    }
  }
  __syncthreads();
  uint16_t* op = a.out + (int64_t)t * kH * kD;
  if (a.out_rot) {
    // the inverse rotation at the query's position into storage of its own: chunks outside
    // the rotary band are stored twice, then the band's chunks are rotated by every lane
    // (a lane-divergent rotation inside the first loop would cost every wave the math)
    uint16_t* orp = a.out_rot + (int64_t)t * kH * kD;
    const int nb = a.rope_dim / 8, band0 = kD / 8 - nb;
#pragma unroll
    for (int k = 0; k < kH * kD / 8 / NT; ++k) {
      const int e = tid + NT * k;
      const int h = e >> 6, cc = e & 63;
      const uint4 v = *reinterpret_cast<const uint4*>(&ot[h * kD + 8 * (cc ^ swz(h))]);
      *reinterpret_cast<uint4*>(op + h * kD + 8 * cc) = v;
      if (cc < band0) *reinterpret_cast<uint4*>(orp + h * kD + 8 * cc) = v;
    }
    for (int e = tid; e < kH * nb; e += NT) {
      const int h = e / nb, c = e - h * nb, cc = band0 + c;
      const uint4 v = *reinterpret_cast<const uint4*>(&ot[h * kD + 8 * (cc ^ swz(h))]);
      float f[8];
      load8(reinterpret_cast<const uint16_t*>(&v), f);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 r = rope_s[4 * c + j];
        rotate_pair(f[2 * j], f[2 * j + 1], r.x, r.y);
      }
      store8(orp + h * kD + 8 * cc, f);
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < kH * kD / 8 / NT; ++k) {
    const int e = tid + NT * k;        // 16-byte chunk of the 64 x 512 output
    const int h = e >> 6, cc = e & 63;
    *reinterpret_cast<uint4*>(op + h * kD + 8 * cc) =
        *reinterpret_cast<const uint4*>(&ot[h * kD + 8 * (cc ^ swz(h))]);
  }
}

hipError_t launch_attn_fwd_mfma(const Shape& sh, const AttnIO& io, hipStream_t s, bool* handled) {
  *handled = false;
  if (sh.dtype != 1 || sh.H != kH || sh.D != kD) return hipSuccess;
  *handled = true;
  FwdArgs a;
  a.q = (const uint16_t*)io.q;
  a.kv_cmp = (const uint16_t*)io.kv_cmp;
  a.kv = (const uint16_t*)io.kv;
  a.idx = io.idx;
  a.sink = io.sink;
  a.cu = sh.cu;
  a.cu_cmp = sh.cu_cmp;
  a.out = (uint16_t*)io.out;
  a.out_rot = (uint16_t*)io.out_rot;
  a.rope_dim = sh.rope_dim;
  a.rope_l2t = sh.rope_dim > 0 ? log2((double)sh.rope_theta) : 0.0;
  a.lse = io.lse;
  a.lse_cmp = io.lse_cmp;
  a.t_logits = io.t_logits;
  a.ld_t = teacher_logits_ld(sh);
  a.scale = sh.scale;
  a.B = sh.B;
  a.T = sh.T;
  a.r = sh.r;
  a.n_cap = sh.max_seqlen / sh.r;
  a.W = sh.W;
  a.k_cap = sh.k_cap;
  a.mode = sh.mode;
  a.scale_log2 = sh.scale * 1.44269504088896341f;
  if (sh.mode != 0 || sh.k_cap <= kIdxLds)
    hipLaunchKernelGGL((k_attn_fwd_mfma<kFwdWaves, kFwdHeadGroups, true>), dim3((unsigned)token_grid(sh.T)),
                       dim3(kFwdWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn_fwd_mfma<kFwdWaves, kFwdHeadGroups, false>), dim3((unsigned)token_grid(sh.T)),
                       dim3(kFwdWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
