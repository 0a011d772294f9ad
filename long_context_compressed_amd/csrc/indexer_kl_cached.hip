// Indexer KL loss and its eager backward from cached teacher logits (gfx950, 64 teacher
// heads, bf16 64 x 128 indexer).
//
// "DeepSeek-V4 Attention Training Systems", section 3: L_I = sum_t KL(P_t || Q_t) over the
// candidate set C_t; the teacher is detached and gradients reach the indexer query, head
// weights and indexer keys only.  Section 8.2 recomputes the teacher logits inside the
// loss; when C_t is exactly the attention's compressed candidate set, the attention
// forward already formed those logits, and on a part with 288 GB of HBM keeping them
// (4 bytes per head and candidate) is cheaper than gathering every 1 KiB row again and
// repeating the QK product.  Teacher reading: P_t = mean over heads of the per-head
// softmax over C_t.
//
// Per query token one workgroup of 4 waves; candidate slots in blocks of 64:
//   * P_j: each thread reads 4 heads x 4 slots of the cached logits (16-byte loads),
//     forms e^{l - lse_h} and the head sum is finished across lanes and waves;
//   * Q_j from the index scores, KL_t, g_j = grad_scale (Q_j - P_j);
//   * z^T = kI qI^T on v_mfma_f32_16x16x32_bf16 (wave = 32 indexer heads x 32 slots; key
//     rows gathered into swizzled LDS by direct global->LDS loads one block ahead);
//   * E = g w 1[z>0], dw += g relu(z); dqI += E kI (E reused from registers as the A
//     operand, key rows read transposed);
//   * E (bf16, 64 heads) is written per (query, slot), 128 bytes; the key gradient
//     dkI[j] = sum_t sum_h E[t,h,j] qI[t,h] is then formed key-major (k_kl_keys: blocks of
//     128 compressed rows against the queries that see them, on MFMA, sums in registers),
//     with no per-pair key-gradient vector and no fp32 atomics.
#include <math.h>

#include "attn_common.h"
#include "attn_bwd_keys.h"
#include "csa_launch.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace csa {

using namespace attn;

namespace {

constexpr int kHT = 64;     // teacher heads
constexpr int kHI = 64;     // indexer heads
constexpr int kDI = 128;    // indexer width
constexpr int kNB = 64;     // slots per block
constexpr int kEST = 72;    // bf16 row stride of the E tile (slot-major, 64 heads + pad)
constexpr int64_t kStageBudget = 16ll << 30;   // bytes of E per chunk
constexpr int kIdxLds = 2048;                   // idx entries of a query staged in LDS

struct KlcArgs {
  const float* tl;          // cached teacher logits [T, 64, ld_t]
  int64_t ld_t;
  const float* tlse;        // teacher lse [T, 64] (natural log) or null
  const float* scores;
  int64_t ld;
  const int32_t* idx;       // null for the dense teacher
  const uint16_t* qI;
  const float* w;
  const uint16_t* kI;
  const int32_t* cu;
  const int32_t* cu_cmp;
  float gs;
  float* kl;
  float* dqI;
  float* dw;
  uint16_t* es;             // [chunk][k_slots][64] bf16: E of every (query, slot)
  int32_t* nc;              // [T] candidate count
  int64_t k_slots;
  int t0, nT;
  int B, T, r, n_cap, k_cap, grads;
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// at most 2 vector memory operations outstanding (they complete in issue order)
__device__ __forceinline__ void wait_vmem_2() { asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); }

__device__ __forceinline__ void dma_rows16(const void* src, const void* lds) {
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(a), "v"(src) : "memory", "m0");
}

// Sum over the workgroup's 4 waves in fp64 (the normalizers of the loss: an fp32 sum of a
// thousand terms of similar size carries a relative error of ~1e-7, as large as the KL of two
// near-uniform distributions is small).
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const double r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float u = __shfl_xor(v, o, 64);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))
                         : (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

}  // namespace

// IDX_LDS: the query's idx row and its student scores (C_t of at most kIdxLds slots: k_cap
// for the selected teacher, max_seqlen / ratio for the dense one) are staged in LDS,
// so that the block loop's only global loads are the cached logits and the key rows, neither
// needed in the block that issues it (a load consumed right away would make the wave wait
// for every older memory operation, the previous block's staged stores included).
template <bool IDX_LDS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_kl_cached(KlcArgs a) {
  __shared__ int32_t idx_s[IDX_LDS ? kIdxLds : 1];
  __shared__ float sc_s[IDX_LDS ? kIdxLds : 1];   // student scores of the slots
  __shared__ __attribute__((aligned(16))) uint16_t KIt[2][kNB][kDI];   // swizzled 256-byte rows
  __shared__ __attribute__((aligned(16))) uint16_t QIs[kHI][kDI];      // the query's qI, swizzled
  __shared__ __attribute__((aligned(16))) uint16_t EsT[kNB][kEST];
  __shared__ float Pp[2][4][kNB];   // per block parity: each wave's head-partial P of the slots
  __shared__ float gw_s[4][kNB];
  __shared__ float lse2_s[kHT];
  __shared__ double red_d[4];
  __shared__ float z_s;           // teacher mass over the blocks so far (wave 0)
  __shared__ float red[4];
  __shared__ int s_tmp;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int hh = wave & 1, ch = wave >> 1;
  const int tl = token_of_block(blockIdx.x);
  if (tl >= a.nT) return;
  const int t = a.t0 + tl;

  TokenInfo ti;
  const bool real = token_info_wave(a.cu, a.B, t, ti, a.cu_cmp);
  int row0 = 0, nv = 0, n_c = 0;
  const int32_t* idx_t = a.idx ? a.idx + (int64_t)t * a.k_cap : nullptr;
  if (real) {
    row0 = ti.c0;
    nv = min((ti.p + 1) / a.r, a.n_cap);
    if (IDX_LDS && idx_t) {
      int iv[IDX_LDS ? kIdxLds / 256 : 1];
      load_idx_regs(idx_t, a.k_cap, iv);
      store_idx_lds(idx_s, a.k_cap, iv);
    }
    if (!idx_t) n_c = nv;
    else if (IDX_LDS) n_c = leading_valid_lds(idx_s, a.k_cap, &s_tmp);   // publishes idx_s
    else n_c = leading_valid(idx_t, a.k_cap, &s_tmp);
  }
  if (tid == 0) a.nc[t] = n_c;
  if (n_c == 0) {
    if (tid == 0) a.kl[t] = 0.f;
    if (a.grads) {
      float4* d = reinterpret_cast<float4*>(a.dqI + (int64_t)t * kHI * kDI);
      for (int e = tid; e < kHI * kDI / 4; e += 256) d[e] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (tid < kHI) a.dw[(int64_t)t * kHI + tid] = 0.f;
    }
    return;
  }
  const float* srow = a.scores + (int64_t)t * a.ld;
  // local visible index of slot c, or -1 (outside C_t or the visible range)
  auto slot_local = [&](int c) -> int {
    if (c >= n_c) return -1;
    if (!idx_t) return c;
    const int gr = IDX_LDS ? idx_s[c] : idx_t[c];
    return (gr >= row0 && gr < row0 + nv) ? gr - row0 : -1;
  };

  // ---- loads of the query's resident operands, issued before the student scores so that
  // their latencies overlap: qI (the B operand of z; into LDS, wave w rows 16w .. 16w+15, 4
  // rows per instruction: lane l fills physical chunk l % 16 of row 4i + l / 16), weights,
  // teacher lse
  float wv[2];
  if (a.grads) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + (lane >> 4);
      dma_rows16(a.qI + ((int64_t)t * kHI + r) * kDI + 8 * ((lane & 15) ^ swz(r)),
                 &QIs[16 * wave + 4 * i][0]);
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) wv[nt] = a.w[(int64_t)t * kHI + 32 * hh + 16 * nt + c16];
  }
  const float tlse_v = (a.tlse && tid < kHT) ? a.tlse[(int64_t)t * kHT + tid] : 0.f;

  // ---- student log-sum-exp over C_t.  With up to kIdxLds slots the scores are read once,
  // all loads in flight together, and kept in LDS for the block loop (-inf marks a slot
  // outside C_t or the visible range); longer rows read them where they are used.
  // (IDX_LDS is launched only where every C_t has at most kIdxLds slots)
  constexpr bool sc_lds = IDX_LDS;
  float mx = -INFINITY;
  if (sc_lds) {
    constexpr int kPT = (IDX_LDS ? kIdxLds : 256) / 256;
    float sv[kPT];
#pragma unroll
    for (int i = 0; i < kPT; ++i) {
      const int j = slot_local(tid + 256 * i);
      sv[i] = j >= 0 ? srow[j] : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < kPT; ++i) {
      if (tid + 256 * i < n_c) sc_s[tid + 256 * i] = sv[i];
      mx = fmaxf(mx, sv[i]);
    }
  } else {
    for (int c = tid; c < n_c; c += 256) {
      const int j = slot_local(c);
      if (j >= 0) mx = fmaxf(mx, srow[j]);
    }
  }
  const float mS = block_reduce(mx, red, true);   // its barriers publish sc_s
  double sm = 0.0;
  for (int c = tid; c < n_c; c += 256) {
    if (sc_lds) {
      const float v = sc_s[c];
      if (v > -INFINITY) sm += (double)expf(v - mS);
    } else {
      const int j = slot_local(c);
      if (j >= 0) sm += (double)expf(srow[j] - mS);
    }
  }
  const float sS = (float)block_sum_f64(sm, red_d);
  // all slots out of the visible range (an invalid idx row): Q_t = 0 instead of NaN
  const float lseS = sS > 0.f ? mS + logf(sS) : INFINITY;

  // ---- teacher log-normalizer per head (log2 domain), from the forward or the cache
  const float* tl_t = a.tl + (int64_t)t * kHT * a.ld_t;
  if (a.tlse) {
    if (tid < kHT) lse2_s[tid] = tlse_v > -INFINITY ? tlse_v * 1.44269504088896341f : INFINITY;
  } else {
    // wave w: heads 16w..16w+15, one head at a time over all slots
    for (int hq = 0; hq < 16; ++hq) {
      const int h = 16 * wave + hq;
      float m = -INFINITY, l = 0.f;
      for (int c = lane; c < n_c; c += 64) {
        if (slot_local(c) < 0) continue;
        const float s2 = tl_t[(int64_t)h * a.ld_t + c] * 1.44269504088896341f;
        if (s2 > m) { l = l * exp2f(m - s2) + 1.f; m = s2; } else { l += exp2f(s2 - m); }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float mo = __shfl_xor(m, o, 64), lo = __shfl_xor(l, o, 64);
        const float mn = fmaxf(m, mo);
        if (mn != -INFINITY) { l = l * exp2f(m - mn) + lo * exp2f(mo - mn); m = mn; }
      }
      if (lane == 0) lse2_s[h] = l > 0.f ? m + log2f(l) : INFINITY;
    }
  }


  // key-row ids of a block: lane l <-> slot 64 b + l (global compressed row or -1)
  const int nblk = (n_c + kNB - 1) / kNB;
  auto row_of = [&](int b) {
    const int j = b < nblk ? slot_local(kNB * b + lane) : -1;
    return j >= 0 ? row0 + j : -1;
  };
  auto score_of = [&](int b) {
    const int j = b < nblk ? slot_local(kNB * b + lane) : -1;
    if (j < 0) return 0.f;
    return sc_lds ? sc_s[kNB * b + lane] : srow[j];
  };
  // wave w gathers rows 16w .. 16w+15 (4 rows of 256 bytes per instruction, lane l fills
  // physical chunk l % 16 of row 4i + l / 16); an absent slot's row is zero-filled
  auto issue = [&](int rid, int buf) {
    if (!a.grads) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + (lane >> 4);
      const int id = __shfl(rid, r, 64);
      if (id >= 0)
        dma_rows16(a.kI + (int64_t)id * kDI + 8 * ((lane & 15) ^ swz(r)),
                   &KIt[buf][16 * wave + 4 * i][0]);
      else
        *reinterpret_cast<uint4*>(&KIt[buf][r][8 * (lane & 15)]) = make_uint4(0, 0, 0, 0);
    }
  };

  f32x4 dq[2][8];   // dqI partial over this wave's slots: heads 32hh + 16nt + 4g + i, d 16nd + c16
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int nd = 0; nd < 8; ++nd) dq[nt][nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dw_acc[2] = {0.f, 0.f};
  // KL terms and the teacher's total mass Z = sum_j P_j (per block over the lanes, then over
  // the blocks in LDS): the loss is A / Z - log Z with A = sum_j P_j (log P_j - log Q_j),
  // i.e. the KL of P / Z, so the fp32 rounding of the per-head normalizers (which leaves
  // sum_j P_j = 1 + O(1e-7)) does not bias it (for near-uniform P and Q the KL itself is of
  // that order times the candidate count)
  float kl_acc = 0.f;
  if (tid == 0) z_s = 0.f;   // first read after the block loop's barriers

  // per-lane LDS offsets (elements) of the swizzled 256-byte key rows
  //  z^T A operand: row 32ch + 16mt + c16, logical chunk 4ks + g
  int za[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) za[ks] = 8 * ((4 * ks + g) ^ swz(c16));
  //  dqI B operand (transposed): rows 32ch + 4g + c16/4 (lo) and +16 (hi), logical chunk
  //  2 nd + (c16 & 3) / 2, element 4 (c16 & 1) within it; row bits 0-3 = 4g + c16/4 (mod 16)
  const int trr = 4 * g + (c16 >> 2);
  const int tre = (c16 & 3) >> 1, troff = 4 * (c16 & 1);

  int rid_cur = row_of(0), rid_nxt = row_of(1);
  float sc_cur = score_of(0), sc_nxt = score_of(1);
  issue(rid_cur, 0);
  wait_vmem();
  __syncthreads();

  // cached teacher logits of a block: thread = (heads 4 hq .. +3, slots 4 sq .. +3).  Block b
  // loads block b + 1's right after its first barrier and turns them into block b + 1's P at
  // its end, behind its own products.  Two register sets take turns over pairs of blocks, so no
  // set is copied while its loads are in flight (a rotating copy made every block end wait for
  // all its loads, and so did a student score that could come from global memory); past the
  // last block the loads repeat it, so every block issues the same loads.
  const int hq = tid >> 4, sq = tid & 15;
  auto load_logits = [&](int b, f32x4 (&v)[4]) {
    const int bb = b < nblk ? b : nblk - 1;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = *reinterpret_cast<const f32x4*>(tl_t + (int64_t)(4 * hq + k) * a.ld_t + kNB * bb +
                                             4 * sq);
  };
  f32x4 lg_a[4], lg_b[4];
  load_logits(0, lg_a);
  // block 0's logits complete before its P is formed
#pragma unroll
  for (int k = 0; k < 4; ++k) asm volatile("" :: "v"(lg_a[k]));

  // ---- teacher probabilities of block b's slots from its logits: this wave's 16 heads, per
  // slot, into Pp[b & 1][wave] (block b + 1's are formed at the end of block b, while block b's
  // products are still in flight, so that they are off the path to block b + 1's first barrier)
  auto teacher_p = [&](int b, const f32x4 (&lg)[4]) {
    float pj[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float l2 = lse2_s[4 * hq + k];
      const f32x4 v = lg[k];
#pragma unroll
      for (int i = 0; i < 4; ++i) pj[i] += __builtin_amdgcn_exp2f(v[i] * 1.44269504088896341f - l2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pj[i] += __shfl_xor(pj[i], 16, 64);
      pj[i] += __shfl_xor(pj[i], 32, 64);
    }
    if (g == 0) *reinterpret_cast<f32x4*>(&Pp[b & 1][wave][4 * sq]) = f32x4{pj[0], pj[1], pj[2], pj[3]};
  };
  teacher_p(0, lg_a);

  // block b: its logits' P is in Pp[b & 1]; lg_ld receives block b + 1's logits, whose P
  // this block forms at its end
  auto block = [&](int b, f32x4 (&lg_ld)[4]) {
    const int buf = b & 1;
    const int rid_nn = row_of(b + 2);
    // key rows of this block, issued during the previous block; younger than them are that
    // block's logit loads (consumed at its end) and, if this wave wrote E of any slot of it,
    // its 2 E stores, which may stay in flight (block 0: its rows were waited for before the
    // loop)
    if (IDX_LDS && a.grads && b > 0 && kNB * (b - 1) + 16 * wave < n_c) wait_vmem_2();
    else wait_vmem();
    __syncthreads();
    // the other key buffer was last read before the previous block's second barrier
    if (b + 1 < nblk) issue(rid_nxt, buf ^ 1);
    load_logits(b + 1, lg_ld);
    const float sc_nn = score_of(b + 2);   // used two blocks on

    // ---- per slot (lane l = slot 64 b + l): P, Q, KL and g; g w per wave in LDS
    float gl;
    {
      const bool in = rid_cur >= 0;
      const float P = ((Pp[buf][0][lane] + Pp[buf][1][lane]) + (Pp[buf][2][lane] + Pp[buf][3][lane])) *
                      (1.f / kHT);
      const float logQ = sc_cur - lseS;
      const float Q = in ? expf(logQ) : 0.f;
      // log P - log Q = log(P * s_S) - (s - m_S): no cancellation of two logs of the
      // candidate count when both distributions are close to uniform
      if (wave == 0) {
        if (in && P > 0.f) kl_acc += P * (logf(P * sS) - (sc_cur - mS));
        const float zb = wave_sum(in && P > 0.f ? P : 0.f);
        if (lane == 0) z_s += zb;
      }
      gl = in ? a.gs * (Q - P) : 0.f;
      gw_s[wave][lane] = gl;
    }
    if (a.grads) {
      // ---- z^T: slots 32ch + 16mt + 4g + i, indexer heads 32hh + 16nt + c16
      f32x4 z[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        z[mt][0] = z[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* rp = &KIt[buf][32 * ch + 16 * mt + c16][0];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 av = ld16(rp + za[ks]);
          // B: qI of heads 32hh + 16nt + c16 (row bits 0-3 = c16), d = 32ks + 8g .. +7
          const int qc = 8 * ((4 * ks + g) ^ swz(c16));
          z[mt][0] = mfma16(av, ld16(&QIs[32 * hh + c16][qc]), z[mt][0]);
          z[mt][1] = mfma16(av, ld16(&QIs[32 * hh + 16 + c16][qc]), z[mt][1]);
        }
      }
      // ---- E = g w 1[z > 0]; dw += g relu(z); E (bf16) to LDS as [slot][head]
      uint32_t ew[2][4];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          float e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = gw_s[wave][32 * ch + 16 * mt + 4 * g + i];
            const float zz = z[mt][nt][i];
            dw_acc[nt] = fmaf(gv, fmaxf(zz, 0.f), dw_acc[nt]);
            e[i] = zz > 0.f ? gv * wv[nt] : 0.f;
          }
          ew[nt][2 * mt] = pack_bf16x2(e[0], e[1]);
          ew[nt][2 * mt + 1] = pack_bf16x2(e[2], e[3]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t wd = ew[nt][2 * mt + (i >> 1)];
            EsT[32 * ch + 16 * mt + 4 * g + i][32 * hh + 16 * nt + c16] =
                (uint16_t)((i & 1) ? (wd >> 16) : (wd & 0xffffu));
          }
        }
      }
      // ---- dqI[h][d] += sum_c E[h][c] kI[c][d]: k-slot order {4g..4g+3, 16+4g..16+4g+3}
      {
        const uint16_t* klo = &KIt[buf][32 * ch + trr][troff];
        const uint16_t* khi = &KIt[buf][32 * ch + 16 + trr][troff];
        const int s_lo = swz(trr), s_hi = swz(16 + trr);
#pragma unroll
        for (int nd = 0; nd < 8; ++nd) {
          const int kq = 2 * nd + tre;
          const bf16x8 kb = join8(ld_tr(klo + 8 * (kq ^ s_lo)), ld_tr(khi + 8 * (kq ^ s_hi)));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const bf16x8 ea = __builtin_bit_cast(bf16x8, make_uint4(ew[nt][0], ew[nt][1], ew[nt][2], ew[nt][3]));
            dq[nt][nd] = mfma16(ea, kb, dq[nt][nd]);
          }
        }
      }
    }
    // Pp[buf ^ 1] was last read before this block's first barrier
    if (b + 1 < nblk) teacher_p(b + 1, lg_ld);
    __syncthreads();
    if (a.grads) {
      // ---- E rows of the block's slots (thread: slot tid / 4, heads 16 (tid % 4) .. +15):
      // two 16-byte stores from the slot-major LDS tile
      const int sl = tid >> 2, hq4 = 16 * (tid & 3), slot = kNB * b + sl;
      if (slot < n_c) {
        const uint4 e0 = *reinterpret_cast<const uint4*>(&EsT[sl][hq4]);
        const uint4 e1 = *reinterpret_cast<const uint4*>(&EsT[sl][hq4 + 8]);
        uint4* dst = reinterpret_cast<uint4*>(a.es + ((int64_t)tl * a.k_slots + slot) * kHI + hq4);
        dst[0] = e0;
        dst[1] = e1;
      }
    }
    rid_cur = rid_nxt;
    rid_nxt = rid_nn;
    sc_cur = sc_nxt;
    sc_nxt = sc_nn;
  };
  // pairs of blocks, then the one left
  int b = 0;
  for (; b + 1 < nblk; b += 2) {
    block(b, lg_b);
    block(b + 1, lg_a);
  }
  if (b < nblk) block(b, lg_b);

  // ---- outputs: kl, dw, dqI (the two slot halves ch = 0, 1 summed through LDS)
  if (wave == 0) {
    const double v = wave_sum_f64((double)kl_acc), z = (double)z_s;
    if (lane == 0) a.kl[t] = z > 0.0 ? (float)(v / z - log1p(z - 1.0)) : 0.f;
  }
  if (!a.grads) return;
  __syncthreads();
  float* dqs = reinterpret_cast<float*>(&KIt[0][0][0]);   // [64][128] fp32 = 32 KiB
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float d2 = dw_acc[nt];
    d2 += __shfl_xor(d2, 16, 64);
    d2 += __shfl_xor(d2, 32, 64);
    if (g == 0) Pp[0][ch][32 * hh + 16 * nt + c16] = d2;
  }
  if (ch == 0) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int nd = 0; nd < 8; ++nd)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dqs[(32 * hh + 16 * nt + 4 * g + i) * kDI + 16 * nd + c16] = dq[nt][nd][i];
  }
  __syncthreads();
  if (ch == 1) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int nd = 0; nd < 8; ++nd)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dqs[(32 * hh + 16 * nt + 4 * g + i) * kDI + 16 * nd + c16] += dq[nt][nd][i];
  }
  __syncthreads();
  if (tid < kHI) a.dw[(int64_t)t * kHI + tid] = Pp[0][0][tid] + Pp[0][1][tid];
  float4* dst = reinterpret_cast<float4*>(a.dqI + (int64_t)t * kHI * kDI);
  const float4* src = reinterpret_cast<const float4*>(dqs);
  for (int e = tid; e < kHI * kDI / 4; e += 256) dst[e] = src[e];
}

// ---- workspace plan and launch
namespace {

__global__ __launch_bounds__(256) void k_fill_zero_i32(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

struct KlcPlan {
  int64_t k_slots, chunk, cap;
  size_t off_es, off_nc, off_cnt, off_items, off_ipart, off_red, off_part, total;
};

bool klc_handles(const Shape& sh) {
  if (!(sh.H == kHT && sh.HI == kHI && sh.dI == kDI && sh.idx_dtype == 1 && sh.r > 0 &&
        ((sh.teacher == 1 && sh.mode == 0) || (sh.teacher == 2 && sh.mode == 1))))
    return false;
  // the key-major key gradients: idx rows held in LDS, per-sample block tables
  const int64_t n_cap = sh.max_seqlen / sh.r;
  return (sh.mode == 1 || sh.k_cap <= 2048) && n_cap / 256 + 1 <= 2048;
}

KlcPlan klc_layout(const Shape& sh, int64_t chunk) {
  KlcPlan p;
  p.k_slots = sh.mode == 0 ? sh.k_cap : sh.max_seqlen / sh.r;
  if (p.k_slots < 1) p.k_slots = 1;
  p.chunk = chunk;
  p.cap = keys::item_cap(sh.mode, sh.B, (int)chunk, sh.max_seqlen / sh.r, 0, 256);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o = 0;
  p.off_es = o;    o = al(o + (size_t)p.chunk * p.k_slots * kHI * 2);
  p.off_nc = o;    o = al(o + (size_t)sh.T * 4);
  p.off_cnt = o;   o = al(o + 128 * 4);   // 64 counters, then 256 zero bytes
  p.off_items = o; o = al(o + (size_t)p.cap * 16);
  p.off_ipart = o; o = al(o + (size_t)p.cap * 4);
  p.off_red = o;   o = al(o + (size_t)p.cap * 16);
  p.off_part = o;  o = al(o + (size_t)p.cap * 256 * kDI * 4);
  p.total = o;
  return p;
}

KlcPlan klc_plan(const Shape& sh) {
  const int64_t per_tok = (sh.mode == 0 ? sh.k_cap : sh.max_seqlen / sh.r) * kHI * 2;
  int64_t ch = kStageBudget / (per_tok > 0 ? per_tok : 1);
  ch = (ch / (8 * kChunk)) * (8 * kChunk);
  if (ch < 8 * kChunk) ch = 8 * kChunk;
  return klc_layout(sh, ch < sh.T ? ch : (sh.T > 0 ? sh.T : 1));
}

}  // namespace

size_t indexer_kl_cached_workspace(const Shape& sh) {
  return klc_handles(sh) ? klc_plan(sh).total : 0;
}

hipError_t launch_indexer_kl_cached(const Shape& sh, const KlIO& io, hipStream_t s, bool* handled) {
  *handled = false;
  if (!io.t_logits || !klc_handles(sh)) return hipSuccess;
  *handled = true;
  const KlcPlan pl = klc_plan(sh);
  if (pl.total > io.ws_bytes) return hipErrorInvalidValue;   // host-checked
  char* ws = (char*)io.ws;
  KlcArgs a;
  a.tl = io.t_logits;
  a.ld_t = teacher_logits_ld(sh);
  a.tlse = io.teacher_lse;
  a.scores = io.scores;
  a.ld = io.ld;
  a.idx = sh.teacher == 1 ? io.idx : nullptr;
  a.qI = (const uint16_t*)io.qI;
  a.w = io.w;
  a.kI = (const uint16_t*)io.kI;
  a.cu = sh.cu;
  a.cu_cmp = sh.cu_cmp;
  a.gs = io.grad_scale;
  a.kl = io.kl;
  a.dqI = io.dqI;
  a.dw = io.dw;
  a.es = (uint16_t*)(ws + pl.off_es);
  a.nc = (int32_t*)(ws + pl.off_nc);
  a.k_slots = pl.k_slots;
  a.B = sh.B;
  a.T = sh.T;
  a.r = sh.r;
  a.n_cap = sh.max_seqlen / sh.r;
  a.k_cap = sh.k_cap;
  a.grads = io.dqI != nullptr;
  KeysArgs k = {};
  k.q = a.qI;
  k.pds = a.es;
  k.idx = a.idx;
  k.nc = a.nc;
  k.cu = sh.cu;
  k.cu_cmp = sh.cu_cmp;
  k.counters = (int32_t*)(ws + pl.off_cnt);
  k.zeros = (const uint16_t*)(ws + pl.off_cnt + 64 * 4);
  k.items = (int4*)(ws + pl.off_items);
  k.item_part = (int32_t*)(ws + pl.off_ipart);
  k.red = (int4*)(ws + pl.off_red);
  k.part = (float*)(ws + pl.off_part);
  k.dkv_cmp = io.dkI;
  k.n_slots = pl.k_slots;
  k.cap = pl.cap;
  k.B = sh.B;
  k.r = sh.r;
  k.n_cap = a.n_cap;
  k.W = 0;
  k.k_cap = sh.k_cap;
  k.mode = sh.mode;
  k.D = kDI;
  k.KC = kHI;
  k.kb = 256;
  for (int64_t t0 = 0; t0 < sh.T; t0 += pl.chunk) {
    a.t0 = k.t0 = (int)t0;
    a.nT = k.nT = (int)(sh.T - t0 < pl.chunk ? sh.T - t0 : pl.chunk);
    if (a.grads) {
      hipLaunchKernelGGL(k_fill_zero_i32, dim3(1), dim3(256), 0, s, k.counters, 128);
      hipError_t e = launch_attn_bwd_keys(k, s);
      if (e != hipSuccess) return e;
    }
    if ((sh.mode == 0 ? (int64_t)sh.k_cap : a.n_cap) <= kIdxLds)
      hipLaunchKernelGGL(k_kl_cached<true>, dim3((unsigned)token_grid(a.nT)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(k_kl_cached<false>, dim3((unsigned)token_grid(a.nT)), dim3(256), 0, s, a);
    if (a.grads) {
      hipError_t e = launch_kl_keys_sums(k, s);
      if (e != hipSuccess) return e;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa
