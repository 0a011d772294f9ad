// Learned-score compressor, forward and adjoint ("DeepSeek-V4 Attention Training Systems":
// the compressor is a learned-score reduction that restarts at sample boundaries (sections
// 4 and 8.2), ratio-4 groups overlap their left neighbour for 8 source tokens while
// ratio-128 groups do not (section 5.1), and its positional parameter is fp32 (section 9)).
//
// Reading: per channel d, the compressed row of group j is
//   c[d] = sum_u w_u[d] x[t_u, d],  w[d] = softmax_u(score[t_u, d] + bias[p_u, d]),
// over the group's own r tokens (positions r .. 2r-1 when overlapping, else 0 .. r-1) and,
// when overlapping and j > 0, its left neighbour's r tokens (positions 0 .. r-1).
//
// Both directions are HBM streams: one thread per (compressed row, 8 channels), 16-byte
// loads of the value and score rows, fp32 math.  The forward takes the per-channel max in
// one pass over the source tokens and the exponentials and sums in a second (the rows are
// then in L1/L2).  The adjoint recomputes w and c and is launched twice: own tokens, then
// left-neighbour tokens, so every (token, channel) of dx and dscore has a single writer per
// launch (no atomics); the positional-parameter gradient is summed per workgroup in an LDS
// tile and added to the output once per workgroup.
#include <math.h>

#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

namespace {

constexpr int kBiasTile = 8192;   // adjoint: floats of the per-workgroup positional-gradient tile

struct Span {
  int t0, n, p0, own0;   // first source token, count, its position, first own token
};

// Group `row` (global compressed row) of the packed batch; false past the last row.
__device__ __forceinline__ bool group_span(const int32_t* __restrict__ cu,
                                           const int32_t* __restrict__ cu_cmp, int B, int r,
                                           bool overlap, int row, Span& sp) {
  if (row >= cu_cmp[B]) return false;
  const int b = upper_bound_i32(cu_cmp, B + 1, row) - 1;
  const int j = row - cu_cmp[b];
  const int own = cu[b] + j * r;
  sp.own0 = own;
  if (overlap && j > 0) {
    sp.t0 = own - r;
    sp.n = 2 * r;
    sp.p0 = 0;
  } else {
    sp.t0 = own;
    sp.n = r;
    sp.p0 = overlap ? r : 0;
  }
  return true;
}

// group_softmax for a span of exactly N tokens (the ratio-4 spans: 4 or 8): the loops are
// unrolled, so every token's loads are in flight together instead of one token at a time.
template <int N, typename T>
__device__ __forceinline__ void group_softmax_n(const T* __restrict__ x, const T* __restrict__ sc,
                                                const float* __restrict__ bias, int dim, int c8,
                                                const Span& sp, float (&m)[8], float (&l)[8],
                                                float (&c)[8]) {
  float s[N][8], bb[N][8], v[N][8];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    load8(sc + (int64_t)(sp.t0 + u) * dim + c8, s[u]);
    load8(bias + (int64_t)(sp.p0 + u) * dim + c8, bb[u]);
    load8(x + (int64_t)(sp.t0 + u) * dim + c8, v[u]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) { m[i] = -INFINITY; l[i] = 0.f; c[i] = 0.f; }
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], s[u][i] + bb[u][i]);
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = __expf(s[u][i] + bb[u][i] - m[i]);
      l[i] += e;
      c[i] = fmaf(e, v[u][i], c[i]);
    }
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] /= l[i];
}

// Per-channel max of the logits over the span, then the normalizer and the reduction.
template <typename T>
__device__ __forceinline__ void group_softmax(const T* __restrict__ x, const T* __restrict__ sc,
                                              const float* __restrict__ bias, int dim, int c8,
                                              const Span& sp, float (&m)[8], float (&l)[8],
                                              float (&c)[8]) {
  if (sp.n == 8) return group_softmax_n<8>(x, sc, bias, dim, c8, sp, m, l, c);
  if (sp.n == 4) return group_softmax_n<4>(x, sc, bias, dim, c8, sp, m, l, c);
#pragma unroll
  for (int i = 0; i < 8; ++i) { m[i] = -INFINITY; l[i] = 0.f; c[i] = 0.f; }
  for (int u = 0; u < sp.n; ++u) {
    float s[8], bb[8];
    load8(sc + (int64_t)(sp.t0 + u) * dim + c8, s);
    load8(bias + (int64_t)(sp.p0 + u) * dim + c8, bb);
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], s[i] + bb[i]);
  }
  for (int u = 0; u < sp.n; ++u) {
    float s[8], bb[8], v[8];
    load8(sc + (int64_t)(sp.t0 + u) * dim + c8, s);
    load8(bias + (int64_t)(sp.p0 + u) * dim + c8, bb);
    load8(x + (int64_t)(sp.t0 + u) * dim + c8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = __expf(s[i] + bb[i] - m[i]);
      l[i] += e;
      c[i] = fmaf(e, v[i], c[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] /= l[i];
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void k_compress_learned(const T* __restrict__ x,
                                                          const T* __restrict__ sc,
                                                          const float* __restrict__ bias,
                                                          int dim, const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ cu_cmp,
                                                          int B, int r, int overlap,
                                                          T* __restrict__ out, int64_t n_items) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_items) return;
  const int nch = dim / 8;
  const int row = (int)(e / nch), c8 = 8 * (int)(e % nch);
  Span sp;
  if (!group_span(cu, cu_cmp, B, r, overlap != 0, row, sp)) return;
  float m[8], l[8], c[8];
  group_softmax(x, sc, bias, dim, c8, sp, m, l, c);
  store8(out + (int64_t)row * dim + c8, c);
}

// part 0: the groups' own tokens; part 1: their left-neighbour tokens (overlap only).
// Workgroup (x, y): channels y cw .. y cw + cw - 1 (cw / 8 chunks per group row), group rows
// x gr .. x gr + gr - 1 of `per` consecutive groups each; the positional-parameter gradient
// of the workgroup is summed in an LDS tile [span][cw] and added to dbias once.
template <typename T>
__global__ __launch_bounds__(256) void k_compress_learned_bwd(
    const T* __restrict__ x, const T* __restrict__ sc, const float* __restrict__ bias,
    const float* __restrict__ dc, int dim, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cu_cmp, int B, int r, int overlap, int part, int cw, int per,
    float* __restrict__ dx, float* __restrict__ ds, float* __restrict__ dbias) {
  __shared__ float dbs[kBiasTile];
  const int span = overlap ? 2 * r : r;
  const int nchw = cw / 8, gr = 256 / nchw;
  for (int e = threadIdx.x; e < span * cw; e += 256) dbs[e] = 0.f;
  __syncthreads();
  const int lc = threadIdx.x % nchw, lr = threadIdx.x / nchw;
  const int c8 = (int)blockIdx.y * cw + 8 * lc;
  const int row_lo = ((int)blockIdx.x * gr + lr) * per;
  if (lr < gr) {
    for (int k = 0; k < per; ++k) {
      Span sp;
      if (!group_span(cu, cu_cmp, B, r, overlap != 0, row_lo + k, sp)) break;
      // tokens of this part: own tokens [own0, own0 + r), left tokens [t0, own0)
      const int u_lo = part == 0 ? sp.own0 - sp.t0 : 0;
      const int u_hi = part == 0 ? sp.n : sp.own0 - sp.t0;
      if (u_lo >= u_hi) continue;
      float m[8], l[8], c[8], g[8];
      group_softmax(x, sc, bias, dim, c8, sp, m, l, c);
      load8(dc + (int64_t)(row_lo + k) * dim + c8, g);
      if (u_hi - u_lo == 4) {
        // the ratio-4 parts: the four tokens' loads are all in flight before the first use
        constexpr int N = 4;
        float s[N][8], bb[N][8], v[N][8], ox[N][8], os[N][8];
#pragma unroll
        for (int q = 0; q < N; ++q) {
          const int u = u_lo + q;
          const int64_t off = (int64_t)(sp.t0 + u) * dim + c8;
          load8(sc + off, s[q]);
          load8(bias + (int64_t)(sp.p0 + u) * dim + c8, bb[q]);
          load8(x + off, v[q]);
          load8(dx + off, ox[q]);
          load8(ds + off, os[q]);
        }
#pragma unroll
        for (int q = 0; q < N; ++q) {
          const int u = u_lo + q;
          const int64_t off = (int64_t)(sp.t0 + u) * dim + c8;
          float* db = &dbs[(sp.p0 + u) * cw + 8 * lc];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float w = __expf(s[q][i] + bb[q][i] - m[i]) / l[i];
            ox[q][i] = fmaf(w, g[i], ox[q][i]);
            const float dz = w * (v[q][i] - c[i]) * g[i];
            os[q][i] += dz;
            atomicAdd(db + i, dz);
          }
          store8(dx + off, ox[q]);
          store8(ds + off, os[q]);
        }
        continue;
      }
      for (int u = u_lo; u < u_hi; ++u) {
        const int64_t off = (int64_t)(sp.t0 + u) * dim + c8;
        float s[8], bb[8], v[8], ox[8], os[8];
        load8(sc + off, s);
        load8(bias + (int64_t)(sp.p0 + u) * dim + c8, bb);
        load8(x + off, v);
        load8(dx + off, ox);
        load8(ds + off, os);
        float* db = &dbs[(sp.p0 + u) * cw + 8 * lc];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float w = __expf(s[i] + bb[i] - m[i]) / l[i];
          ox[i] = fmaf(w, g[i], ox[i]);
          const float dz = w * (v[i] - c[i]) * g[i];
          os[i] += dz;
          atomicAdd(db + i, dz);
        }
        store8(dx + off, ox);
        store8(ds + off, os);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < span * cw; e += 256) {
    const float v = dbs[e];
    if (v != 0.f) atomicAdd(dbias + (int64_t)(e / cw) * dim + (int)blockIdx.y * cw + e % cw, v);
  }
}

hipError_t launch_compress_learned(const Shape& sh, int dtype, const void* x, const void* score,
                                   const float* bias, int dim, int overlap, void* x_cmp,
                                   hipStream_t s) {
  const int64_t n_items = (int64_t)(sh.T / sh.r) * (dim / 8);   // rows <= T / r
  if (n_items == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_items + 255) / 256)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(k_compress_learned<float>, grid, block, 0, s, (const float*)x,
                       (const float*)score, bias, dim, sh.cu, sh.cu_cmp, sh.B, sh.r, overlap,
                       (float*)x_cmp, n_items);
  else
    hipLaunchKernelGGL(k_compress_learned<uint16_t>, grid, block, 0, s, (const uint16_t*)x,
                       (const uint16_t*)score, bias, dim, sh.cu, sh.cu_cmp, sh.B, sh.r, overlap,
                       (uint16_t*)x_cmp, n_items);
  return hipGetLastError();
}

hipError_t launch_compress_learned_bwd(const Shape& sh, int dtype, const void* x,
                                       const void* score, const float* bias,
                                       const float* d_x_cmp, int dim, int overlap, float* dx,
                                       float* dscore, float* dbias, hipStream_t s) {
  const int64_t rows = sh.T / sh.r;
  if (rows == 0) return hipSuccess;
  const int span = (overlap ? 2 : 1) * sh.r;
  // channel slice: the largest multiple-of-8 divisor of dim whose tile fits, at most 256
  // chunks; groups per thread so that the launch has a few hundred workgroups or more
  int cw = dim;
  while (cw > 8 && (span * cw > kBiasTile || cw / 8 > 256 || dim % cw != 0)) cw -= 8;
  if (span * cw > kBiasTile) return hipErrorInvalidValue;   // span > kBiasTile / 8
  const int gr = 256 / (cw / 8);
  const int64_t slices = dim / cw;
  int per = 16;
  while (per > 1 && ((rows + (int64_t)gr * per - 1) / ((int64_t)gr * per)) * slices < 512) per /= 2;
  const dim3 grid((unsigned)((rows + (int64_t)gr * per - 1) / ((int64_t)gr * per)),
                  (unsigned)slices),
      block(256);
  for (int part = 0; part < (overlap ? 2 : 1); ++part) {
    if (dtype == 0)
      hipLaunchKernelGGL(k_compress_learned_bwd<float>, grid, block, 0, s, (const float*)x,
                         (const float*)score, bias, d_x_cmp, dim, sh.cu, sh.cu_cmp, sh.B, sh.r,
                         overlap, part, cw, per, dx, dscore, dbias);
    else
      hipLaunchKernelGGL(k_compress_learned_bwd<uint16_t>, grid, block, 0, s,
                         (const uint16_t*)x, (const uint16_t*)score, bias, d_x_cmp, dim, sh.cu,
                         sh.cu_cmp, sh.B, sh.r, overlap, part, cw, per, dx, dscore, dbias);
  }
  return hipGetLastError();
}

}  // namespace csa
