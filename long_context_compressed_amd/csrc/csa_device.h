// Device-side helpers shared by the gfx950 kernels of the CSA/HCA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- element types
// bf16 is carried as its 16 raw bits; fp32 <-> bf16 uses round-to-nearest-even.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (low half = a), hardware round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Loads / stores of 8 consecutive elements as fp32.
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store1(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }

// OCP e4m3 code -> fp32 (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = (e == 0) ? (float)m * 0.001953125f                      // m * 2^-9
                       : __uint_as_float(((e + 120u) << 23) | (m << 20));  // 2^(e-7) (1 + m/8)
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------- rotary embedding
// cos and sin of pair i of the rotary band at position pos: angle pos * theta^(-2i / rope_dim)
// (its opposite when inverse), formed and reduced in fp64 so that the positions of long
// samples keep fp32 accuracy; l2t = log2(theta).
__device__ __forceinline__ void rope_cs(int pos, int i, int rope_dim, double l2t, bool inverse,
                                        float& c, float& s) {
  const double ang = (double)pos * exp2(-(double)(2 * i) / (double)rope_dim * l2t);
  double sd, cd;
  sincos(ang, &sd, &cd);
  c = (float)cd;
  s = inverse ? -(float)sd : (float)sd;
}

// (a, b) -> (a c - b s, a s + b c), in one fixed operation order wherever it is applied.
__device__ __forceinline__ void rotate_pair(float& a, float& b, float c, float s) {
  const float x = a, y = b;
  a = fmaf(x, c, -(y * s));
  b = fmaf(x, s, y * c);
}

// ---------------------------------------------------------------- metadata
// First index i in [0, n) with a[i] > v (n if none): with a = cu_seqlens it returns b+1
// for the sample b containing row v; empty samples are skipped correctly.
__device__ __forceinline__ int upper_bound_i32(const int32_t* __restrict__ a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

struct TokenInfo {
  int b;       // sample
  int start;   // first packed row of the sample
  int len;     // L_b
  int p;       // local position
  int c0;      // first compressed row of the sample (set by attn::token_info_wave when it is
               // given the compressed offsets)
};

// Sample of packed row t; returns false for capacity padding (t >= cu[B]).
__device__ __forceinline__ bool token_info(const int32_t* __restrict__ cu, int B, int t,
                                           TokenInfo& ti) {
  if (B <= 0 || t >= cu[B]) return false;
  const int b = upper_bound_i32(cu, B + 1, t) - 1;
  ti.b = b;
  ti.start = cu[b];
  ti.len = cu[b + 1] - cu[b];
  ti.p = t - ti.start;
  return true;
}

// ---------------------------------------------------------------- wave / block reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

}  // namespace csa
