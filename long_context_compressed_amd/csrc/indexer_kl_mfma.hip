// Matrix-core (MFMA) indexer KL loss with its eager backward on gfx950, for bf16 main
// operands (H = 64, D = 512) and a 64 x 128 indexer in bf16 or fp8.
//
// "DeepSeek-V4 Attention Training Systems", section 3: L_I = sum_t KL(P_t || Q_t) over the
// candidate set C_t (selected set, or all visible compressed entries in the dense-loss
// warm-up); the teacher is detached, gradients reach the indexer query, head weights and
// indexer keys only.  Section 8.2: teacher scores are recomputed, and the indexer-loss
// backward runs eagerly with the loss scale supplied by the caller (grad_scale).
// Teacher reading: P_t = mean over heads of the per-head softmax over C_t.
//
// One workgroup (4 waves) per query token; wave w owns heads 16w..16w+15.
//   pass 1: per block of 32 candidates the compressed KV rows are staged in LDS and
//           S^T = K Q^T is formed on MFMA; each lane keeps an online (max, sum) of its
//           head, merged across lane groups -> per-head teacher log-sum-exp;
//           the student log-sum-exp over C_t is a block reduction over the scores.
//   pass 2: S^T again -> per-head probabilities -> head sum across lanes and waves -> P_t;
//           Q_t from the scores; KL_t and g = grad_scale (Q_t - P_t);
//           z^T = kI qI^T on MFMA; E = g w 1[z>0]; dw += g relu(z) in registers;
//           dqI += E kI with E reused from registers as the A operand and the key tile
//           read transposed (ds_read_b64_tr_b16); dkI = E^T qI from LDS tiles, split by d
//           across waves, scatter-added with fp32 atomics.
// fp8 indexer: z (and so the ReLU mask) is formed from the e4m3 codes on the scaled fp8
// MFMA exactly as the score kernel forms it; the gradient products use bf16 tiles of the
// dequantized operands (code * fp32 scale, rounded once).
#include <math.h>

#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kH = 64, kD = 512, kHI = 64, kDI = 128;
constexpr int kNB = 32;
constexpr int kKS = kD + 16;    // bf16 row stride of the KV tile
constexpr int kIS = kDI + 8;    // bf16 row stride of the indexer tiles
constexpr int kES = 40;         // bf16 row stride of the E tile
constexpr int kChunk = 256;

struct KlArgs {
  const uint16_t* q;
  const uint16_t* kv_cmp;
  const float* scores;
  int64_t ld;
  const int32_t* idx;
  const float* teacher_lse;
  const void* qI;
  const float* qI_scale;
  const float* w;
  const void* kI;
  const float* kI_scale;
  const int32_t* cu;
  const int32_t* cu_cmp;
  float gs;
  float* kl;
  float* dqI;
  float* dw;
  float* dkI;
  int B, T, r, n_cap, k_cap, teacher, fp8, grads;
  float scale_log2;
};

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4i16 ld_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
}
__device__ __forceinline__ bf16x8 join8(v4i16 lo, v4i16 hi) {
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ int token_of_block(int bid) {
  const int x = bid & 7, j = bid >> 3;
  return (j / kChunk) * (8 * kChunk) + x * kChunk + (j % kChunk);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_indexer_kl_mfma(KlArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][kNB][kKS];
  __shared__ __attribute__((aligned(16))) uint16_t KIt[2][kNB][kIS];
  __shared__ __attribute__((aligned(16))) uint16_t QIt[kHI][kIS];
  __shared__ __attribute__((aligned(16))) uint16_t Es[kHI][kES];
  __shared__ __attribute__((aligned(16))) uint8_t KI8[2][kNB][kDI + 16];   // fp8 codes
  __shared__ float ksc_s[2][kNB];
  __shared__ float Pp[4][kNB];
  __shared__ float g_s[kNB];
  __shared__ float I_s[2][kNB];
  __shared__ int rowid_s[2][kNB];
  __shared__ float red[4];
  __shared__ double red_d[4];
  __shared__ int s_n;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int t = token_of_block(blockIdx.x);
  if (t >= a.T) return;
  TokenInfo ti;
  const bool real = token_info(a.cu, a.B, t, ti);
  int row0 = 0, nv = 0, n_c = 0;
  if (real) {
    row0 = a.cu_cmp[ti.b];
    nv = min((ti.p + 1) / a.r, a.n_cap);
    if (a.teacher == 2) {
      n_c = nv;
    } else {
      if (tid == 0) s_n = a.k_cap;
      __syncthreads();
      for (int c = tid; c < a.k_cap; c += 256)
        if (a.idx[(int64_t)t * a.k_cap + c] < 0) atomicMin(&s_n, c);
      __syncthreads();
      n_c = s_n;
    }
  }
  if (n_c == 0) {
    if (tid == 0) a.kl[t] = 0.f;
    if (a.grads) {
      for (int e = tid; e < kHI * kDI; e += 256) a.dqI[(int64_t)t * kHI * kDI + e] = 0.f;
      if (tid < kHI) a.dw[(int64_t)t * kHI + tid] = 0.f;
    }
    return;
  }
  const int32_t* idx_row = a.idx + (int64_t)t * a.k_cap;
  const float* srow = a.scores + (int64_t)t * a.ld;
  // local visible index of slot c (or -1)
  auto slot_local = [&](int c) -> int {
    if (c >= n_c) return -1;
    if (a.teacher == 2) return c;
    const int gr = idx_row[c];
    return (gr >= row0 && gr < row0 + nv) ? gr - row0 : -1;
  };

  // ---- student log-sum-exp over C_t
  float mx = -INFINITY;
  for (int c = tid; c < n_c; c += 256) {
    const int j = slot_local(c);
    if (j >= 0) mx = fmaxf(mx, srow[j]);
  }
  const float mS = block_max(mx, red);
  // the student normalizer, the KL terms and the teacher's mass Z = sum_j P_j in fp64: the
  // loss is A / Z - log Z with A = sum_j P_j (log P_j - log Q_j) (the KL of P / Z), unbiased by
  // the fp32 rounding of the normalizers when P and Q are both near-uniform
  double sm = 0.0;
  for (int c = tid; c < n_c; c += 256) {
    const int j = slot_local(c);
    if (j >= 0) sm += (double)expf(srow[j] - mS);
  }
  double smw = wave_sum_f64(sm);
  if ((tid & 63) == 0) red_d[tid >> 6] = smw;
  __syncthreads();
  const float sS = (float)((red_d[0] + red_d[1]) + (red_d[2] + red_d[3]));
  __syncthreads();
  // all slots out of the visible range (an invalid idx row): Q_t = 0 instead of NaN
  const float lseS = sS > 0.f ? mS + logf(sS) : INFINITY;

  // ---- resident operands: Q^T slice (teacher), indexer query tile (dequantized)
  const int h = 16 * wave + c16;
  bf16x8 qb[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qb[ks] = ld16(a.q + ((int64_t)t * kH + h) * kD + 32 * ks + 8 * g);
  if (a.grads) {
    for (int e = tid; e < kHI * (kDI / 8); e += 256) {
      const int hh = e / (kDI / 8), ch = e % (kDI / 8);
      uint4 v;
      if (!a.fp8) {
        v = *reinterpret_cast<const uint4*>((const uint16_t*)a.qI + ((int64_t)t * kHI + hh) * kDI + 8 * ch);
      } else {
        const uint2 cw = *reinterpret_cast<const uint2*>((const uint8_t*)a.qI + ((int64_t)t * kHI + hh) * kDI + 8 * ch);
        const float sc = a.qI_scale[(int64_t)t * kHI + hh];
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t wd = i < 2 ? cw.x : cw.y;
          const uint32_t b0 = (wd >> (16 * (i & 1))) & 0xffu, b1 = (wd >> (16 * (i & 1) + 8)) & 0xffu;
          o[i] = (uint32_t)f32_to_bf16_bits(e4m3_to_f32(b0) * sc) |
                 ((uint32_t)f32_to_bf16_bits(e4m3_to_f32(b1) * sc) << 16);
        }
        v = make_uint4(o[0], o[1], o[2], o[3]);
      }
      *reinterpret_cast<uint4*>(&QIt[hh][8 * ch]) = v;
    }
  }

  // ---- block loader, split in two halves: issue (global -> registers) right after the
  // barrier that starts a block, commit (registers -> LDS tiles) after the block computes,
  // so the loads of block c+1 overlap the MFMA work of block c
  uint4 pre_kv[8];
  int pre_j[8];
  float pre_I[8];
  uint4 pre_ki[2];
  float pre_sc[2];
  int pre_kj[2];
  auto issue = [&](int c0, bool second) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = slot_local(c0 + 4 * i + wave);
      pre_j[i] = j;
      pre_kv[i] = j >= 0 ? *reinterpret_cast<const uint4*>(a.kv_cmp + (int64_t)(row0 + j) * kD + 8 * lane)
                         : make_uint4(0, 0, 0, 0);
      pre_I[i] = (j >= 0 && lane == 0) ? srow[j] : 0.f;
    }
    if (second && a.grads) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int e = tid + 256 * i;
        const int row = e >> 4, ch = e & 15;
        const int j = slot_local(c0 + row);
        pre_kj[i] = j;
        pre_ki[i] = make_uint4(0, 0, 0, 0);
        pre_sc[i] = 0.f;
        if (j >= 0) {
          if (!a.fp8) {
            pre_ki[i] = *reinterpret_cast<const uint4*>((const uint16_t*)a.kI + (int64_t)(row0 + j) * kDI + 8 * ch);
          } else {
            const uint2 cw = *reinterpret_cast<const uint2*>((const uint8_t*)a.kI + (int64_t)(row0 + j) * kDI + 8 * ch);
            pre_ki[i] = make_uint4(cw.x, cw.y, 0, 0);
            pre_sc[i] = a.kI_scale[row0 + j];
          }
        }
      }
    }
  };
  auto commit = [&](int buf, bool second) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + wave;
      *reinterpret_cast<uint4*>(&Kt[buf][row][8 * lane]) = pre_kv[i];
      if (lane == 0) {
        rowid_s[buf][row] = pre_j[i] >= 0 ? row0 + pre_j[i] : -1;
        I_s[buf][row] = pre_I[i];
      }
    }
    if (second && a.grads) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int e = tid + 256 * i;
        const int row = e >> 4, ch = e & 15;
        uint4 v = pre_ki[i];
        if (a.fp8) {
          const uint2 cw = make_uint2(pre_ki[i].x, pre_ki[i].y);
          *reinterpret_cast<uint2*>(&KI8[buf][row][8 * ch]) = cw;
          if (ch == 0) ksc_s[buf][row] = pre_sc[i];
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t wd = q < 2 ? cw.x : cw.y;
            const uint32_t b0 = (wd >> (16 * (q & 1))) & 0xffu, b1 = (wd >> (16 * (q & 1) + 8)) & 0xffu;
            o[q] = (uint32_t)f32_to_bf16_bits(e4m3_to_f32(b0) * pre_sc[i]) |
                   ((uint32_t)f32_to_bf16_bits(e4m3_to_f32(b1) * pre_sc[i]) << 16);
          }
          v = make_uint4(o[0], o[1], o[2], o[3]);
        }
        *reinterpret_cast<uint4*>(&KIt[buf][row][8 * ch]) = v;
        (void)pre_kj;
      }
    }
  };

  // ---- pass 1: per-head teacher log-sum-exp over C_t (skipped when the forward supplied it)
  float m_h = -INFINITY, l_h = 0.f;
  int buf = 0;
  const bool have_lse = a.teacher_lse != nullptr;
  if (!have_lse) {
    issue(0, false);
    commit(0, false);
  }
  for (int c0 = 0; c0 < (have_lse ? 0 : n_c); c0 += kNB, buf ^= 1) {
    __syncthreads();
    const bool more = c0 + kNB < n_c;
    if (more) issue(c0 + kNB, false);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) st = mfma16(ld16(&Kt[buf][16 * mt + c16][32 * ks + 8 * g]), qb[ks], st);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (rowid_s[buf][16 * mt + 4 * g + i] < 0) continue;
        const float s2 = st[i] * a.scale_log2;
        if (s2 > m_h) {
          l_h = l_h * exp2f(m_h - s2) + 1.f;
          m_h = s2;
        } else {
          l_h += exp2f(s2 - m_h);
        }
      }
    }
    if (more) commit(buf ^ 1, false);
  }
  {  // merge the 4 lane groups of head h
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float mo = __shfl_xor(m_h, o, 64), lo = __shfl_xor(l_h, o, 64);
      const float mn = fmaxf(m_h, mo);
      if (mn != -INFINITY) {
        l_h = l_h * exp2f(m_h - mn) + lo * exp2f(mo - mn);
        m_h = mn;
      }
    }
  }
  float lse2 = l_h > 0.f ? m_h + log2f(l_h) : INFINITY;
  if (have_lse) {
    const float v = a.teacher_lse[(int64_t)t * kH + h];
    lse2 = v > -INFINITY ? v * 1.44269504088896341f : INFINITY;
  }

  // ---- pass 2
  bf16x8 qib[4];
  i32x8 qa8 = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  float sq_h = 1.f;
  if (a.grads && a.fp8) {
    const uint4* p = reinterpret_cast<const uint4*>((const uint8_t*)a.qI + ((int64_t)t * kHI + h) * kDI + 32 * g);
    const uint4 lo = p[0], hi = p[1];
    qa8 = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    sq_h = a.qI_scale[(int64_t)t * kHI + h];
  }
  f32x4 dqa[8];
  float dw_acc = 0.f, kl_acc = 0.f, z_acc = 0.f;
  const float wh = a.w[(int64_t)t * kHI + h];
  __syncthreads();   // QIt staged; pass-1 tiles no longer read
  if (a.grads) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qib[ks] = ld16(&QIt[h][32 * ks + 8 * g]);
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) dqa[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int jr = c16 >> 2, jc = 4 * (c16 & 3);
  buf = 0;
  issue(0, true);
  commit(0, true);
  for (int c0 = 0; c0 < n_c; c0 += kNB, buf ^= 1) {
    __syncthreads();
    const bool more = c0 + kNB < n_c;
    if (more) issue(c0 + kNB, true);
    // teacher probabilities of head h, summed over the wave's 16 heads
    float ps[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) st = mfma16(ld16(&Kt[buf][16 * mt + c16][32 * ks + 8 * g]), qb[ks], st);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = rowid_s[buf][16 * mt + 4 * g + i] >= 0 ? exp2f(st[i] * a.scale_log2 - lse2) : 0.f;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) p += __shfl_xor(p, o, 64);
        ps[mt][i] = p;
      }
    }
    if (c16 == 0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Pp[wave][16 * mt + 4 * g + i] = ps[mt][i];
    }
    __syncthreads();
    if (tid < kNB) {
      float gv = 0.f;
      if (rowid_s[buf][tid] >= 0) {
        const float P = ((Pp[0][tid] + Pp[1][tid]) + (Pp[2][tid] + Pp[3][tid])) * (1.f / kH);
        const float logQ = I_s[buf][tid] - lseS;
        const float Q = expf(logQ);
        // log P - log Q = log(P * s_S) - (I - m_S): no cancellation of two logs of the
        // candidate count when both distributions are close to uniform
        if (P > 0.f) {
          kl_acc += P * (logf(P * sS) - (I_s[buf][tid] - mS));
          z_acc += P;
        }
        gv = a.gs * (Q - P);
      }
      g_s[tid] = gv;
    }
    __syncthreads();
    if (a.grads) {
      // z^T = kI qI^T for this wave's 16 heads; E = g w 1[z>0]
      uint32_t ew[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!a.fp8) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) z = mfma16(ld16(&KIt[buf][16 * mt + c16][32 * ks + 8 * g]), qib[ks], z);
        } else {
          // z from the e4m3 codes exactly as the score kernel forms it, times both scales
          const uint4* kp = reinterpret_cast<const uint4*>(&KI8[buf][16 * mt + c16][32 * g]);
          const uint4 lo = kp[0], hi = kp[1];
          const i32x8 ka = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qa8, z, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] = z[i] * ksc_s[buf][16 * mt + 4 * g + i] * sq_h;
        }
        uint32_t e2[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = g_s[16 * mt + 4 * g + i];
          const float e = z[i] > 0.f ? gv * wh : 0.f;
          dw_acc = fmaf(gv, fmaxf(z[i], 0.f), dw_acc);
          const uint32_t eb = f32_to_bf16_bits(e);
          if (i & 1) e2[i >> 1] |= eb << 16;
          else e2[i >> 1] = eb;
        }
        ew[2 * mt] = e2[0];
        ew[2 * mt + 1] = e2[1];
        *reinterpret_cast<uint2*>(&Es[h][16 * mt + 4 * g]) = make_uint2(e2[0], e2[1]);
      }
      // dqI[h'][d] += sum_c E[h'][c] kI[c][d]; k-slot order {4g..4g+3, 16+4g..16+4g+3}
      const bf16x8 ea = __builtin_bit_cast(bf16x8, make_uint4(ew[0], ew[1], ew[2], ew[3]));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const v4i16 lo = ld_tr(&KIt[buf][4 * g + jr][16 * nt + jc]);
        const v4i16 hi = ld_tr(&KIt[buf][16 + 4 * g + jr][16 * nt + jc]);
        dqa[nt] = mfma16(ea, join8(lo, hi), dqa[nt]);
      }
      __syncthreads();
      // dkI[c][d] for d in 32 wave .. 32 wave + 31, contraction over all 64 heads
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 ev = join8(ld_tr(&Es[32 * ks + 8 * g + jr][16 * mt + jc]),
                                    ld_tr(&Es[32 * ks + 8 * g + 4 + jr][16 * mt + jc]));
            const int dcol = 32 * wave + 16 * nt + jc;
            const bf16x8 qv = join8(ld_tr(&QIt[32 * ks + 8 * g + jr][dcol]),
                                    ld_tr(&QIt[32 * ks + 8 * g + 4 + jr][dcol]));
            acc = mfma16(ev, qv, acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rid = rowid_s[buf][16 * mt + 4 * g + i];
            if (rid >= 0) atomicAdd(a.dkI + (int64_t)rid * kDI + 32 * wave + 16 * nt + c16, acc[i]);
          }
        }
    }
    if (more) commit(buf ^ 1, true);
  }
  // ---- outputs
  if (a.grads) {
    dw_acc += __shfl_xor(dw_acc, 16, 64);
    dw_acc += __shfl_xor(dw_acc, 32, 64);
    if (g == 0) a.dw[(int64_t)t * kHI + h] = dw_acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * wave + 4 * g + i;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) a.dqI[((int64_t)t * kHI + hh) * kDI + 16 * nt + c16] = dqa[nt][i];
    }
  }
  // kl: lanes 0..31 of wave 0 hold partial sums
  if (wave == 0) {
    const double v = wave_sum_f64(lane < kNB ? (double)kl_acc : 0.0);
    const double z = wave_sum_f64(lane < kNB ? (double)z_acc : 0.0);
    if (lane == 0) a.kl[t] = z > 0.0 ? (float)(v / z - log1p(z - 1.0)) : 0.f;
  }
}

hipError_t launch_indexer_kl_mfma(const Shape& sh, const KlIO& io, hipStream_t s, bool* handled) {
  *handled = false;
  if (sh.dtype != 1 || sh.H != kH || sh.D != kD || sh.HI != kHI || sh.dI != kDI ||
      sh.idx_dtype == 0)
    return hipSuccess;
  *handled = true;
  KlArgs a;
  a.q = (const uint16_t*)io.q;
  a.kv_cmp = (const uint16_t*)io.kv_cmp;
  a.scores = io.scores;
  a.ld = io.ld;
  a.idx = io.idx;
  a.teacher_lse = sh.teacher == 1 ? io.teacher_lse : nullptr;
  a.qI = io.qI;
  a.qI_scale = io.qI_scale;
  a.w = io.w;
  a.kI = io.kI;
  a.kI_scale = io.kI_scale;
  a.cu = sh.cu;
  a.cu_cmp = sh.cu_cmp;
  a.gs = io.grad_scale;
  a.kl = io.kl;
  a.dqI = io.dqI;
  a.dw = io.dw;
  a.dkI = io.dkI;
  a.B = sh.B;
  a.T = sh.T;
  a.r = sh.r;
  a.n_cap = sh.max_seqlen / sh.r;
  a.k_cap = sh.k_cap;
  a.teacher = sh.teacher;
  a.fp8 = sh.idx_dtype == 2;
  a.grads = io.dqI != nullptr;
  a.scale_log2 = sh.scale * 1.44269504088896341f;
  const int64_t chunks = ((int64_t)sh.T + 8 * kChunk - 1) / (8 * kChunk);
  hipLaunchKernelGGL(k_indexer_kl_mfma, dim3((unsigned)(chunks * 8 * kChunk)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
