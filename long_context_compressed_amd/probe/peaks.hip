// Peak-rate probes for the roofline denominators measured on the device itself (not part
// of the layer library): a loop of independent matrix-core operations per wave, bf16
// (v_mfma_f32_16x16x32_bf16, 16384 FLOP each) and fp8 (v_mfma_scale_f32_16x16x128_f8f6f4
// with unit block scales, 65536 FLOP each), with enough waves to occupy every SIMD.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kChains = 8;   // independent accumulators per wave (covers the MFMA latency)

__global__ __launch_bounds__(256) void k_mfma_bf16_loop(float* out, int iters, float seed) {
  bf16x8 a, b0, b1, b2, b3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
    b0[i] = (__bf16)(seed * (float)((int)threadIdx.x - i));
    b1[i] = (__bf16)(seed * (float)((int)threadIdx.x - i + 3));
    b2[i] = (__bf16)(seed * (float)((int)threadIdx.x - i + 6));
    b3[i] = (__bf16)(seed * (float)((int)threadIdx.x - i + 9));
  }
  // eight accumulation chains written out in one asm block: the compiler's own loop moved
  // the loop-carried accumulators between registers and chained them
  f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %10, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %11, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %12, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %10, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %11, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %12, %7"
        : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
        : "v"(a), "v"(b0), "v"(b1), "v"(b2), "v"(b3));
  }
  const f32x4 s = c0 + 2.f * c1 + 3.f * c2 + 4.f * c3 + 5.f * c4 + 6.f * c5 + 7.f * c6 + 8.f * c7;
  out[blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

__global__ __launch_bounds__(256) void k_mfma_fp8_loop(float* out, int iters, int seed) {
  i32x8 a, b[kChains];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ ((seed + (int)threadIdx.x + i) & 0x03030303);
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      b[j][i] = 0x30303030 ^ ((seed - (int)threadIdx.x + i + 5 * j) & 0x03030303);
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], acc[j], 0, 0, 0, 127, 0,
                                                                 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += (float)(j + 1) * (acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3]);
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Enqueue `blocks` workgroups of 4 waves, each wave issuing iters * 8 matrix-core operations
// (bf16: 16384 FLOP each; fp8: 65536 FLOP each); out: fp32 [blocks * 256].  Returns the
// hipError_t of the launch.
int csa_probe_mfma_loop(int fp8, float* out, int blocks, int iters, hipStream_t s) {
  if (fp8)
    hipLaunchKernelGGL(k_mfma_fp8_loop, dim3(blocks), dim3(256), 0, s, out, iters, 7);
  else
    hipLaunchKernelGGL(k_mfma_bf16_loop, dim3(blocks), dim3(256), 0, s, out, iters, 1e-3f);
  return (int)hipGetLastError();
}

}  // extern "C"

namespace {
__global__ void k_trace_marker(int* p) {
  if (threadIdx.x == 0 && p) p[0] = 1;
}
}  // namespace

extern "C" {

// A one-thread kernel whose dispatch separates the sections of a benchmark run in a kernel
// trace (the layer steps before it, the stand-alone measurements after it).
int csa_probe_marker(int* p, hipStream_t s) {
  hipLaunchKernelGGL(k_trace_marker, dim3(1), dim3(64), 0, s, p);
  return (int)hipGetLastError();
}

}  // extern "C"
