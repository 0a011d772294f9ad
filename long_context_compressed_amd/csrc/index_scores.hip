// Lightning-indexer logits over the causally visible compressed rows:
//   I[t, j] = sum_h w[t,h] * relu(qI[t,h] . kI_cmp[cu_cmp[b] + j]),  j < n_vis(p)
// ("DeepSeek-V4 Attention Training Systems", section 3: indexer logits i_{t,j} from the
// indexer Q projection and the head-weight projection; section 4: visibility resets per
// sample).  This file holds the scalar-fp32 kernel used for fp32 operands and for shapes
// without a matrix-core kernel; bf16 / fp8 matrix-core kernels live in index_scores_mfma.hip.
#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

template <typename TI>
__device__ __forceinline__ float ld_idx(const TI* p);
template <>
__device__ __forceinline__ float ld_idx<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_idx<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }
template <>
__device__ __forceinline__ float ld_idx<uint8_t>(const uint8_t* p) { return e4m3_to_f32(*p); }

constexpr int kScJ = 32;  // compressed rows per workgroup

// One workgroup per (query t, block of 32 compressed rows).  qI[t] (dequantized to fp32)
// and the 32 key rows are staged in LDS (key rows padded by one word, conflict-free);
// lane (j, head group) accumulates w*relu(z) over its heads, then the 8 head-group
// partials of a row are added in a fixed order.
template <typename TI>
__global__ __launch_bounds__(256) void k_index_scores_generic(
    const TI* __restrict__ qI, const float* __restrict__ qI_scale, const float* __restrict__ w,
    const TI* __restrict__ kI, const float* __restrict__ kI_scale,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_cmp, int B, int r, int n_cap,
    int HI, int dI, float* __restrict__ scores, int64_t ld) {
  extern __shared__ float sm[];
  float* qs = sm;                       // [HI * dI]
  float* ks = qs + HI * dI;             // [kScJ][dI + 1]
  float* ws = ks + kScJ * (dI + 1);     // [HI]
  float* part = ws + HI;                // [8][kScJ]
  const int t = blockIdx.x;
  const int j0 = blockIdx.y * kScJ;
  TokenInfo ti;
  if (!token_info(cu, B, t, ti)) return;
  const int nv = min((ti.p + 1) / r, n_cap);
  if (j0 >= nv) return;
  const int row0 = cu_cmp[ti.b];
  const bool fp8 = qI_scale != nullptr;
  for (int e = threadIdx.x; e < HI * dI; e += 256) {
    float v = ld_idx<TI>(qI + (int64_t)t * HI * dI + e);
    if (fp8) v *= qI_scale[(int64_t)t * HI + e / dI];
    qs[e] = v;
  }
  for (int e = threadIdx.x; e < HI; e += 256) ws[e] = w[(int64_t)t * HI + e];
  for (int e = threadIdx.x; e < kScJ * dI; e += 256) {
    const int jl = e / dI, d = e - jl * dI;
    const int j = j0 + jl;
    float v = 0.f;
    if (j < nv) {
      v = ld_idx<TI>(kI + (int64_t)(row0 + j) * dI + d);
      if (fp8) v *= kI_scale[row0 + j];
    }
    ks[jl * (dI + 1) + d] = v;
  }
  __syncthreads();
  const int jl = threadIdx.x & (kScJ - 1);
  const int hg = threadIdx.x / kScJ;   // 8 head groups
  float acc = 0.f;
  for (int h = hg; h < HI; h += 8) {
    const float* qh = qs + h * dI;
    const float* kj = ks + jl * (dI + 1);
    float z = 0.f;
    for (int d = 0; d < dI; ++d) z = fmaf(qh[d], kj[d], z);
    acc = fmaf(ws[h], fmaxf(z, 0.f), acc);
  }
  part[hg * kScJ + jl] = acc;
  __syncthreads();
  if (threadIdx.x < kScJ && j0 + threadIdx.x < nv) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) s += part[g * kScJ + threadIdx.x];
    scores[(int64_t)t * ld + j0 + threadIdx.x] = s + 0.0f;   // -0 -> +0
  }
}


hipError_t launch_index_scores(const Shape& sh, const void* qI, const float* qI_scale,
                               const float* w, const void* kI, const float* kI_scale,
                               float* scores, int64_t ld, hipStream_t s) {
  if (sh.T == 0) return hipSuccess;
  bool handled = false;
  hipError_t e = launch_index_scores_mfma(sh, qI, qI_scale, w, kI, kI_scale, scores, ld, s,
                                          &handled);
  if (handled) return e;
  const int n_cap = sh.max_seqlen / sh.r;
  if (n_cap == 0) return hipSuccess;
  const dim3 grid(sh.T, (n_cap + kScJ - 1) / kScJ);
  const size_t lds = sizeof(float) * (sh.HI * sh.dI + kScJ * (sh.dI + 1) + sh.HI + 8 * kScJ);
  if (sh.idx_dtype == 0)
    hipLaunchKernelGGL(k_index_scores_generic<float>, grid, dim3(256), lds, s,
                       (const float*)qI, qI_scale, w, (const float*)kI, kI_scale, sh.cu,
                       sh.cu_cmp, sh.B, sh.r, n_cap, sh.HI, sh.dI, scores, ld);
  else if (sh.idx_dtype == 1)
    hipLaunchKernelGGL(k_index_scores_generic<uint16_t>, grid, dim3(256), lds, s,
                       (const uint16_t*)qI, qI_scale, w, (const uint16_t*)kI, kI_scale, sh.cu,
                       sh.cu_cmp, sh.B, sh.r, n_cap, sh.HI, sh.dI, scores, ld);
  else
    hipLaunchKernelGGL(k_index_scores_generic<uint8_t>, grid, dim3(256), lds, s,
                       (const uint8_t*)qI, qI_scale, w, (const uint8_t*)kI, kI_scale, sh.cu,
                       sh.cu_cmp, sh.B, sh.r, n_cap, sh.HI, sh.dI, scores, ld);
  return hipGetLastError();
}

}  // namespace csa
