// Metadata, compressor (forward and adjoint) and per-row e4m3 quantization.
//
// Compressor: sample b of a packed batch yields floor(L_b / r) compressed rows, row j
// being the mean of raw rows s_b + j*r .. s_b + j*r + r - 1; the incomplete tail yields
// none ("DeepSeek-V4 Attention Training Systems", section 4, the n_b^cmp equation; the
// mean-pool reading of the compressor).  All three kernels are pure HBM streams: every
// input byte is read once with 16-byte vector loads, consecutive lanes on consecutive
// addresses.
#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

// ------------------------------------------------------------------ metadata
__global__ void k_cmp_seqlens(const int32_t* __restrict__ cu, int B, int r,
                              int32_t* __restrict__ cu_cmp) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int acc = 0;
  cu_cmp[0] = 0;
  for (int b = 0; b < B; ++b) {
    acc += (cu[b + 1] - cu[b]) / r;
    cu_cmp[b + 1] = acc;
  }
}

hipError_t launch_cmp_seqlens(const int32_t* cu, int B, int r, int32_t* cu_cmp, hipStream_t s) {
  hipLaunchKernelGGL(k_cmp_seqlens, dim3(1), dim3(64), 0, s, cu, B, r, cu_cmp);
  return hipGetLastError();
}

__global__ void k_validate(const int32_t* __restrict__ cu, int B, int T, int max_seqlen,
                           int32_t* __restrict__ status) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int st = 0;
  if (cu[0] != 0) st = 1;
  for (int b = 0; b < B && st == 0; ++b) {
    const int L = cu[b + 1] - cu[b];
    if (L < 0) st = 2;
    else if (L > max_seqlen) st = 4;
  }
  if (st == 0 && cu[B] > T) st = 3;
  *status = st;
}

hipError_t launch_validate_metadata(const int32_t* cu, int B, int T, int max_seqlen,
                                    int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_validate, dim3(1), dim3(64), 0, s, cu, B, T, max_seqlen, status);
  return hipGetLastError();
}

// Offsets of the packed samples copied to LDS once per workgroup (the per-row sample
// lookups then cost LDS reads instead of a chain of dependent global loads); more samples
// than kLdsSamples keep the lookups in global memory.
constexpr int kLdsSamples = 255;

struct SampleTables {
  const int32_t* cu;
  const int32_t* cu_cmp;
};

__device__ __forceinline__ SampleTables stage_samples(const int32_t* __restrict__ cu,
                                                      const int32_t* __restrict__ cu_cmp, int B,
                                                      int32_t* s_cu, int32_t* s_cmp) {
  if (B > kLdsSamples) return {cu, cu_cmp};
  for (int i = threadIdx.x; i <= B; i += blockDim.x) {
    s_cu[i] = cu[i];
    s_cmp[i] = cu_cmp[i];
  }
  __syncthreads();
  return {s_cu, s_cmp};
}

// ------------------------------------------------------------------ compressor forward
// A workgroup of 256 lanes covers `rows_per_wg` compressed rows; each row is split into
// dim/8 chunks of 8 elements and the r source rows of a chunk into `rsplit` strided
// parts whose fp32 partial sums are added in part order through LDS.  RU > 0 fixes r = RU
// (rsplit 1) so that all RU loads of a lane are issued before the first add.
template <typename T, int RU>
__global__ __launch_bounds__(256) void k_compress(const T* __restrict__ x, int dim,
                                                  const int32_t* __restrict__ cu,
                                                  const int32_t* __restrict__ cu_cmp, int B,
                                                  int r, T* __restrict__ out, int rows_per_wg,
                                                  int rsplit) {
  __shared__ float red[256 * 9];
  __shared__ int32_t s_cu[kLdsSamples + 1], s_cmp[kLdsSamples + 1];
  const SampleTables st = stage_samples(cu, cu_cmp, B, s_cu, s_cmp);
  const int chunks = dim >> 3;
  const int per_row = chunks * rsplit;
  const int tid = threadIdx.x;
  const int lrow = tid / per_row;
  const int rem = tid - lrow * per_row;
  const int part = rem / chunks;
  const int chunk = rem - part * chunks;
  const int64_t j = (int64_t)blockIdx.x * rows_per_wg + lrow;
  const int Tc = st.cu_cmp[B];
  const bool active = lrow < rows_per_wg && j < Tc;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (active) {
    const int b = upper_bound_i32(st.cu_cmp, B + 1, (int)j) - 1;
    const int64_t src = (int64_t)st.cu[b] + (j - st.cu_cmp[b]) * (int64_t)r;
    const T* base = x + src * dim + chunk * 8;
    if constexpr (RU > 0) {
      float v[RU][8];
#pragma unroll
      for (int u = 0; u < RU; ++u) load8(base + (int64_t)u * dim, v[u]);
#pragma unroll
      for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[u][i];
    } else {
      for (int u = part; u < r; u += rsplit) {
        float v[8];
        load8(base + (int64_t)u * dim, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    }
  }
  if (rsplit > 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[tid * 9 + i] = acc[i];
    __syncthreads();
    if (part == 0) {
      for (int q = 1; q < rsplit; ++q) {
        const int o = (tid + q * chunks) * 9;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += red[o + i];
      }
    }
  }
  if (active && part == 0) {
    const float rf = (float)r;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] / rf;
    store8(out + j * dim + chunk * 8, acc);
  }
}

hipError_t launch_compress(const Shape& sh, int dtype, const void* x, int dim, void* x_cmp,
                           hipStream_t s) {
  const int chunks = dim / 8;
  int rsplit = 1;
  while (rsplit * 2 <= sh.r && chunks * rsplit * 2 <= 256 && rsplit < 16 &&
         (int64_t)sh.r / (rsplit * 2) >= 4)
    rsplit *= 2;
  if (sh.r < 16) rsplit = 1;
  const int rows_per_wg = 256 / (chunks * rsplit);
  const int64_t rows_cap = sh.r > 0 ? (int64_t)sh.T / sh.r : 0;
  const int64_t grid = (rows_cap + rows_per_wg - 1) / rows_per_wg;
  if (grid == 0) return hipSuccess;
  const bool r4 = sh.r == 4 && rsplit == 1;
  if (dtype == 0) {
    auto k = r4 ? k_compress<float, 4> : k_compress<float, 0>;
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(256), 0, s, (const float*)x, dim, sh.cu,
                       sh.cu_cmp, sh.B, sh.r, (float*)x_cmp, rows_per_wg, rsplit);
  } else {
    auto k = r4 ? k_compress<uint16_t, 4> : k_compress<uint16_t, 0>;
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(256), 0, s, (const uint16_t*)x, dim,
                       sh.cu, sh.cu_cmp, sh.B, sh.r, (uint16_t*)x_cmp, rows_per_wg, rsplit);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ compressor adjoint
// One lane per (raw row, 8-element chunk): dx[t] += d_cmp[row of t's group] / r.
// Each raw row belongs to at most one group, so no atomics are needed.
__global__ __launch_bounds__(256) void k_compress_bwd(const float* __restrict__ d_cmp, int dim,
                                                      const int32_t* __restrict__ cu,
                                                      const int32_t* __restrict__ cu_cmp,
                                                      int B, int r, float* __restrict__ dx,
                                                      int rows_per_wg) {
  __shared__ int32_t s_cu[kLdsSamples + 1], s_cmp[kLdsSamples + 1];
  const SampleTables st = stage_samples(cu, cu_cmp, B, s_cu, s_cmp);
  const int chunks = dim >> 3;
  const int lrow = threadIdx.x / chunks;
  const int chunk = threadIdx.x - lrow * chunks;
  const int64_t t = (int64_t)blockIdx.x * rows_per_wg + lrow;
  if (lrow >= rows_per_wg) return;
  TokenInfo ti;
  if (!token_info(st.cu, B, (int)t, ti)) return;
  const int j = ti.p / r;
  if (j >= ti.len / r) return;
  float g[8], a[8];
  load8(d_cmp + (int64_t)(st.cu_cmp[ti.b] + j) * dim + chunk * 8, g);
  float* dst = dx + t * dim + chunk * 8;
  load8(dst, a);
  const float rf = (float)r;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] += g[i] / rf;
  store8(dst, a);
}

hipError_t launch_compress_bwd(const Shape& sh, const float* d_cmp, int dim, float* dx,
                               hipStream_t s) {
  const int chunks = dim / 8;
  const int rows_per_wg = 256 / chunks;
  const int64_t grid = ((int64_t)sh.T + rows_per_wg - 1) / rows_per_wg;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_compress_bwd, dim3((unsigned)grid), dim3(256), 0, s, d_cmp, dim, sh.cu,
                     sh.cu_cmp, sh.B, sh.r, dx, rows_per_wg);
  return hipGetLastError();
}

// ------------------------------------------------------------------ e4m3 quantization
// fp32 -> OCP e4m3 code, round to nearest even, saturating at 448.  Written from the
// format's definition: subnormals are multiples of 2^-9 below 2^-6, normals keep 3
// mantissa bits.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a < 448.f)) return sign | 0x7eu;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid 2^-9
    const float m = rintf(a * 512.f);        // exact scaling, ties to even
    return sign | (uint32_t)m;               // m == 8 is the smallest normal, code 0x08
  }
  int e = (int)((bits >> 23) & 0xffu) - 127;  // -6 .. 8
  uint32_t keep = (bits >> 20) & 7u;
  const uint32_t rest = bits & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) { keep = 0u; ++e; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// A group of G lanes per row (G: the power of two, 8 .. 64, that covers the row's 8-element
// chunks, so a wave quantizes 64 / G rows; rows of up to 1024 elements, two chunks per lane
// at G = 64).  The row maximum is reduced within the group, then every lane encodes its
// chunks and stores them as 8 bytes.
template <typename T, int G>
__global__ __launch_bounds__(256) void k_quantize_fp8(const T* __restrict__ x, int64_t rows,
                                                      int row_len, uint8_t* __restrict__ codes,
                                                      float* __restrict__ scale) {
  const int lane = threadIdx.x & 63, li = lane & (G - 1);
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G) + lane / G;
  const bool ok = row < rows;   // no early exit: the group maximum is formed with shuffles
  const T* src = x + row * row_len;
  float v[2][8];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int off = (li + c * G) * 8;
    if (ok && off < row_len) {
      load8(src + off, v[c]);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    }
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int off = (li + c * G) * 8;
    if (ok && off < row_len) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(v[c][i] / sc) << (8 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(v[c][4 + i] / sc) << (8 * i);
      *reinterpret_cast<uint2*>(codes + row * row_len + off) = make_uint2(lo, hi);
    }
  }
  if (ok && li == 0) scale[row] = sc;
}

template <typename T>
static void launch_quantize_rows(const T* x, int64_t rows, int row_len, uint8_t* codes,
                                 float* scale, hipStream_t s) {
  const int chunks = row_len / 8;
  const int g = chunks <= 8 ? 8 : chunks <= 16 ? 16 : chunks <= 32 ? 32 : 64;
  const int64_t rows_per_wg = 4 * (64 / g);
  const dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg)), block(256);
  if (g == 8) hipLaunchKernelGGL((k_quantize_fp8<T, 8>), grid, block, 0, s, x, rows, row_len, codes, scale);
  else if (g == 16) hipLaunchKernelGGL((k_quantize_fp8<T, 16>), grid, block, 0, s, x, rows, row_len, codes, scale);
  else if (g == 32) hipLaunchKernelGGL((k_quantize_fp8<T, 32>), grid, block, 0, s, x, rows, row_len, codes, scale);
  else hipLaunchKernelGGL((k_quantize_fp8<T, 64>), grid, block, 0, s, x, rows, row_len, codes, scale);
}

hipError_t launch_quantize_fp8(const void* x, int dtype, int64_t rows, int row_len,
                               uint8_t* codes, float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dtype == 0)
    launch_quantize_rows((const float*)x, rows, row_len, codes, scale, s);
  else
    launch_quantize_rows((const uint16_t*)x, rows, row_len, codes, scale, s);
  return hipGetLastError();
}

}  // namespace csa
