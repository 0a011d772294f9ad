// Matrix-core (MFMA) lightning-indexer scores on gfx950 for d_I = 128, H_I = 64:
//   I[t, j] = sum_h w[t,h] relu(qI[t,h] . kI[row0 + j]),  j < n_vis(p)
// ("DeepSeek-V4 Attention Training Systems", section 3 indexer logits; section 9: the
// indexer query is FP8-eligible).
//
// One wave per query token (4 tokens per workgroup, no LDS, no barriers).  The token's
// 64 x 128 indexer query is resident in registers as the MFMA A operand; each step
// multiplies it with 64 visible compressed keys (B operand, 16-byte row loads), so the
// Z = qI kI^T tile [64 heads x 64 keys] lives in 16 accumulator tiles.  ReLU, the
// per-(token, head) weight and the head sum are done in registers: 16 heads inside each
// lane, then the 4 lane groups via cross-lane adds, in a fixed order (deterministic).
//   bf16: v_mfma_f32_16x16x32_bf16, 4 k-steps per tile.
//   fp8 (OCP e4m3 codes): v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales, one
//   instruction per tile; the per-row fp32 scales of qI and kI multiply the result.
#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kHI = 64;
constexpr int kDI = 128;

struct ScArgs {
  const void* qI;
  const float* qI_scale;
  const float* w;
  const void* kI;
  const float* kI_scale;
  const int32_t* cu;
  const int32_t* cu_cmp;
  float* scores;
  int64_t ld;
  int B, T, r, n_cap;
};

template <bool FP8>
__device__ __forceinline__ void scores_token(const ScArgs& a, int t) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  TokenInfo ti;
  if (!token_info(a.cu, a.B, t, ti)) return;
  const int nv = min((ti.p + 1) / a.r, a.n_cap);
  if (nv <= 0) return;
  const int row0 = a.cu_cmp[ti.b];
  float* out = a.scores + (int64_t)t * a.ld;

  // per-lane weights of the output rows h = 16mt + 4g + i (and fp8 query scales)
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * mt + 4 * g + i;
      float x = a.w[(int64_t)t * kHI + h];
      if (FP8) x *= a.qI_scale[(int64_t)t * kHI + h];
      wv[mt][i] = x;
    }

  if constexpr (!FP8) {
    const uint16_t* q = (const uint16_t*)a.qI + (int64_t)t * kHI * kDI;
    const uint16_t* k = (const uint16_t*)a.kI;
    bf16x8 qa[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qa[mt][ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(q + (16 * mt + c16) * kDI + 32 * ks + 8 * g));
    for (int j0 = 0; j0 < nv; j0 += 64) {
      bf16x8 kb[4][4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int j = j0 + 16 * nt + c16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (j < nv)
            v = *reinterpret_cast<const uint4*>(k + (int64_t)(row0 + j) * kDI + 32 * ks + 8 * g);
          kb[nt][ks] = __builtin_bit_cast(bf16x8, v);
        }
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kb[nt][ks], z, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) s = fmaf(wv[mt][i], fmaxf(z[i], 0.f), s);
        }
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        const int j = j0 + 16 * nt + c16;
        if (g == 0 && j < nv) out[j] = s + 0.0f;
      }
    }
  } else {
    const uint8_t* q = (const uint8_t*)a.qI + (int64_t)t * kHI * kDI;
    const uint8_t* k = (const uint8_t*)a.kI;
    i32x8 qa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint4* p = reinterpret_cast<const uint4*>(q + (16 * mt + c16) * kDI + 32 * g);
      const uint4 lo = p[0], hi = p[1];
      qa[mt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    for (int j0 = 0; j0 < nv; j0 += 64) {
      i32x8 kb[4];
      float ks_[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int j = j0 + 16 * nt + c16;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        float sc = 0.f;
        if (j < nv) {
          const uint4* p = reinterpret_cast<const uint4*>(k + (int64_t)(row0 + j) * kDI + 32 * g);
          lo = p[0];
          hi = p[1];
          sc = a.kI_scale[row0 + j];
        }
        kb[nt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        ks_[nt] = sc;
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
          // unit block scales (E8M0 127 = 2^0), A and B in fp8 e4m3 (format 0)
          z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kb[nt], z, 0, 0, 0, 127, 0,
                                                               127);
#pragma unroll
          for (int i = 0; i < 4; ++i) s = fmaf(wv[mt][i], fmaxf(z[i] * ks_[nt], 0.f), s);
        }
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        const int j = j0 + 16 * nt + c16;
        if (g == 0 && j < nv) out[j] = s + 0.0f;
      }
    }
  }
}

template <bool FP8>
__global__ __launch_bounds__(256) void k_index_scores_mfma(ScArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  scores_token<FP8>(a, t);
}

}  // namespace

hipError_t launch_index_scores_mfma(const Shape& sh, const void* qI, const float* qI_scale,
                                    const float* w, const void* kI, const float* kI_scale,
                                    float* scores, int64_t ld, hipStream_t s, bool* handled) {
  *handled = false;
  if (sh.HI != kHI || sh.dI != kDI || sh.idx_dtype == 0) return hipSuccess;
  *handled = true;
  ScArgs a;
  a.qI = qI;
  a.qI_scale = qI_scale;
  a.w = w;
  a.kI = kI;
  a.kI_scale = kI_scale;
  a.cu = sh.cu;
  a.cu_cmp = sh.cu_cmp;
  a.scores = scores;
  a.ld = ld;
  a.B = sh.B;
  a.T = sh.T;
  a.r = sh.r;
  a.n_cap = sh.max_seqlen / sh.r;
  const unsigned grid = (unsigned)((sh.T + 3) / 4);
  if (sh.idx_dtype == 2)
    hipLaunchKernelGGL(k_index_scores_mfma<true>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_index_scores_mfma<false>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
