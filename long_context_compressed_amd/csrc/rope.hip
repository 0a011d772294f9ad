// Rotary position embedding on the packed layout ("DeepSeek-V4 Attention Training Systems":
// positions restart at every packed sample for the main and the indexer operands (section 4);
// the positional mode is per layer and per compressed coordinate system, and the inverse
// rotation of the attention output must leave the saved unrotated output intact (section 12,
// invariants 2 and 5; section 10 on the inverse-rotation aliasing contract)).
//
// Row `row` of sample b (offsets[b] <= row < offsets[b + 1]) has position row - offsets[b]:
// with cu_seqlens that is the local token position, with the compressed-row offsets the
// compressed index.  The interleaved channel pairs (2i, 2i + 1) of the last rope_dim channels
// of every head are rotated by pos * theta^(-2i / rope_dim), by the opposite angle when
// inverse; rows of no sample are copied (or, in place, left alone).
//
// An HBM stream: one thread per (row, 8-channel chunk), looping over the heads so that the
// four angles of its chunk are formed once per row (fp64, then fp32 rotation); 16-byte loads
// and stores.  In place only the rotary chunks are visited.
#include <math.h>

#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

template <typename T>
__global__ __launch_bounds__(256) void k_rope(const T* __restrict__ x, T* __restrict__ y,
                                              int heads, int dim, int rope_dim, double l2t,
                                              int inverse, int B,
                                              const int32_t* __restrict__ offs, int c_lo,
                                              int n_ch, int64_t n_items) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_items) return;
  const int64_t row = e / n_ch;
  const int c = c_lo + (int)(e % n_ch);
  const int band0 = (dim - rope_dim) / 8;
  int pos = -1;
  if (B > 0 && row < offs[B]) {
    const int ub = upper_bound_i32(offs, B + 1, (int)row);
    if (ub > 0) pos = (int)row - offs[ub - 1];
  }
  const bool rot = pos >= 0 && c >= band0;
  if (!rot && x == y) return;
  float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
  if (rot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) rope_cs(pos, 4 * (c - band0) + j, rope_dim, l2t, inverse != 0, cs[j], sn[j]);
  }
  const int64_t base = row * heads * dim + 8 * c;
  int h = 0;
  for (; h + 4 <= heads; h += 4) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8(x + base + (int64_t)(h + u) * dim, v[u]);
    if (rot) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) rotate_pair(v[u][2 * j], v[u][2 * j + 1], cs[j], sn[j]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) store8(y + base + (int64_t)(h + u) * dim, v[u]);
  }
  for (; h < heads; ++h) {
    float v[8];
    load8(x + base + (int64_t)h * dim, v);
    if (rot) {
#pragma unroll
      for (int j = 0; j < 4; ++j) rotate_pair(v[2 * j], v[2 * j + 1], cs[j], sn[j]);
    }
    store8(y + base + (int64_t)h * dim, v);
  }
}

hipError_t launch_rope(int dtype, const void* x, void* y, int64_t rows, int heads, int dim,
                       int rope_dim, float theta, int inverse, int B, const int32_t* offs,
                       hipStream_t s) {
  const int c_lo = x == y ? (dim - rope_dim) / 8 : 0;
  const int n_ch = dim / 8 - c_lo;
  const int64_t n_items = rows * n_ch;
  if (n_items == 0) return hipSuccess;
  const double l2t = log2((double)theta);
  const dim3 grid((unsigned)((n_items + 255) / 256)), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(k_rope<float>, grid, block, 0, s, (const float*)x, (float*)y, heads, dim,
                       rope_dim, l2t, inverse, B, offs, c_lo, n_ch, n_items);
  else
    hipLaunchKernelGGL(k_rope<uint16_t>, grid, block, 0, s, (const uint16_t*)x, (uint16_t*)y,
                       heads, dim, rope_dim, l2t, inverse, B, offs, c_lo, n_ch, n_items);
  return hipGetLastError();
}

}  // namespace csa
