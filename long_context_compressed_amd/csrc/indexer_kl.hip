// Indexer KL auxiliary loss and its eager backward.
//
// "DeepSeek-V4 Attention Training Systems", section 3: the indexer is trained by
// L_I = sum_t KL(Softmax(a_{t,C_t}) || Softmax(i_{t,C_t})) with C_t the full visible
// compressed history (dense-loss warm-up) or the selected set (sparse loss); the teacher
// (main query and compressed KV) and the indexer inputs are detached, so the gradient
// reaches only the indexer query, head weights and indexer keys.  Section 8.2: the fused
// stack recomputes teacher scores rather than keeping them, and runs the indexer-loss
// backward eagerly in the forward with the loss scale applied later (grad_scale here).
//
// Teacher reading: P_t = mean over heads of the per-head softmax over C_t of the main
// logits scale * q[t,h] . kv_cmp[j] (window and sink excluded).
//
// Scalar-fp32 kernel: one workgroup per query, two passes over C_t (per-head teacher
// log-sum-exp and the student log-sum-exp, then P, Q, KL and the gradients).
#include <math.h>

#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

struct KlK {
  const void* q;
  const void* kv_cmp;
  const float* scores;
  int64_t ld;
  const int32_t* idx;
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
  int B, H, D, r, n_cap, k_cap, teacher, HI, dI;
  float scale;
  int grads;
};

constexpr int kKB = 8;     // candidates per block
constexpr int kMaxQ = 32;  // dqI accumulators per lane: H_I * d_I <= 8192

template <typename TI>
__device__ __forceinline__ float ld_ix(const TI* p);
template <>
__device__ __forceinline__ float ld_ix<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_ix<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }
template <>
__device__ __forceinline__ float ld_ix<uint8_t>(const uint8_t* p) { return e4m3_to_f32(*p); }

template <typename T, typename TI>
__global__ __launch_bounds__(256) void k_kl_generic(KlK a) {
  extern __shared__ float sm[];
  const int H = a.H, D = a.D, HI = a.HI, dI = a.dI, Dp = D + 1;
  float* rs = sm;                       // [kKB][Dp]
  float* lg = rs + kKB * Dp;            // [H][kKB]
  float* mT = lg + H * kKB;             // [H]
  float* lT = mT + H;                   // [H]
  float* qIs = lT + H;                  // [HI*dI]
  float* kIs = qIs + HI * dI;           // [kKB][dI+1]
  float* Es = kIs + kKB * (dI + 1);     // [HI][kKB]
  float* Zs = Es + HI * kKB;            // [HI][kKB]
  float* gc = Zs + HI * kKB;            // [kKB]
  float* Ic = gc + kKB;                 // [kKB]
  float* klp = Ic + kKB;                // [kKB]
  int* rowid = (int*)(klp + kKB);       // [kKB]
  __shared__ int s_n;
  __shared__ float s_mS, s_lS;
  __shared__ float Pc[64];       // teacher probabilities of the block's candidates

  const int tid = threadIdx.x;
  const int t = blockIdx.x;
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
  float dq_acc[kMaxQ];
#pragma unroll
  for (int i = 0; i < kMaxQ; ++i) dq_acc[i] = 0.f;
  // KL terms and the teacher's mass Z = sum_j P_j in fp64: the loss is A / Z - log Z with
  // A = sum_j P_j (log P_j - log Q_j), the KL of P / Z, unbiased by the fp32 rounding of the
  // normalizers when P and Q are near-uniform
  float dw_acc = 0.f;
  double kl_acc = 0.0, z_acc = 0.0;

  if (n_c > 0) {
    const T* qt = (const T*)a.q + (int64_t)t * H * D;
    const bool fp8 = a.qI_scale != nullptr;
    for (int e = tid; e < HI * dI; e += 256) {
      float v = ld_ix<TI>((const TI*)a.qI + (int64_t)t * HI * dI + e);
      if (fp8) v *= a.qI_scale[(int64_t)t * HI + e / dI];
      qIs[e] = v;
    }
    if (tid < H) { mT[tid] = -INFINITY; lT[tid] = 0.f; }
    if (tid == 0) { s_mS = -INFINITY; s_lS = 0.f; }
    for (int pass = 0; pass < 2; ++pass) {
      for (int c0 = 0; c0 < n_c; c0 += kKB) {
        if (tid < kKB) {
          const int c = c0 + tid;
          int id = -1;
          if (c < n_c) {
            const int g = a.teacher == 2 ? row0 + c : a.idx[(int64_t)t * a.k_cap + c];
            if (g >= row0 && g < row0 + nv) id = g;
          }
          rowid[tid] = id;
          Ic[tid] = id >= 0 ? a.scores[(int64_t)t * a.ld + (id - row0)] : -INFINITY;
        }
        __syncthreads();
        for (int e = tid; e < kKB * D; e += 256) {
          const int cc = e / D, d = e - cc * D;
          const int id = rowid[cc];
          rs[cc * Dp + d] = id >= 0 ? load1((const T*)a.kv_cmp + (int64_t)id * D + d) : 0.f;
        }
        __syncthreads();
        for (int pr = tid; pr < H * kKB; pr += 256) {
          const int h = pr / kKB, cc = pr - h * kKB;
          float s = -INFINITY;
          if (rowid[cc] >= 0) {
            const T* qh = qt + h * D;
            const float* x = rs + cc * Dp;
            float z = 0.f;
            for (int d = 0; d < D; ++d) z = fmaf(load1(qh + d), x[d], z);
            s = z * a.scale;
          }
          lg[pr] = s;
        }
        __syncthreads();
        if (pass == 0) {
          if (tid < H) {
            const float* row = lg + tid * kKB;
            float mx = -INFINITY;
            for (int cc = 0; cc < kKB; ++cc) mx = fmaxf(mx, row[cc]);
            const float mnew = fmaxf(mT[tid], mx);
            if (mnew != -INFINITY) {
              float sum = 0.f;
              for (int cc = 0; cc < kKB; ++cc) sum += expf(row[cc] - mnew);
              lT[tid] = lT[tid] * expf(mT[tid] - mnew) + sum;
              mT[tid] = mnew;
            }
          }
          if (tid == 255) {  // the student's online log-sum-exp (H <= 128 < 255)
            float mx = -INFINITY;
            for (int cc = 0; cc < kKB; ++cc) mx = fmaxf(mx, Ic[cc]);
            const float mnew = fmaxf(s_mS, mx);
            if (mnew != -INFINITY) {
              float sum = 0.f;
              for (int cc = 0; cc < kKB; ++cc) sum += expf(Ic[cc] - mnew);
              s_lS = s_lS * expf(s_mS - mnew) + sum;
              s_mS = mnew;
            }
          }
          __syncthreads();
          continue;
        }
        // pass 1: teacher / student probabilities, KL and logit gradient
        if (tid < kKB) {
          float g = 0.f, klv = 0.f, pv = 0.f;
          if (rowid[tid] >= 0) {
            float P = 0.f;
            for (int h = 0; h < H; ++h) P += expf(lg[h * kKB + tid] - (mT[h] + logf(lT[h])));
            P /= (float)H;
            const float logQ = Ic[tid] - (s_mS + logf(s_lS));
            const float Q = expf(logQ);
            // log P - log Q = log(P * l_S) - (I - m_S): no cancellation of two logs of
            // the candidate count when both distributions are close to uniform
            if (P > 0.f) {
              klv = P * (logf(P * s_lS) - (Ic[tid] - s_mS));
              pv = P;
            }
            g = a.gs * (Q - P);
          }
          gc[tid] = g;
          klp[tid] = klv;
          Pc[tid] = pv;
        }
        __syncthreads();
        if (tid == 0) {
          for (int cc = 0; cc < kKB; ++cc) {
            kl_acc += (double)klp[cc];
            z_acc += (double)Pc[cc];
          }
        }
        if (a.grads) {
          for (int e = tid; e < kKB * dI; e += 256) {
            const int cc = e / dI, d = e - cc * dI;
            const int id = rowid[cc];
            float v = 0.f;
            if (id >= 0) {
              v = ld_ix<TI>((const TI*)a.kI + (int64_t)id * dI + d);
              if (fp8) v *= a.kI_scale[id];
            }
            kIs[cc * (dI + 1) + d] = v;
          }
          __syncthreads();
          for (int pr = tid; pr < HI * kKB; pr += 256) {
            const int h = pr / kKB, cc = pr - h * kKB;
            const float* qh = qIs + h * dI;
            const float* kr = kIs + cc * (dI + 1);
            float z = 0.f;
            for (int d = 0; d < dI; ++d) z = fmaf(qh[d], kr[d], z);
            const float wv = a.w[(int64_t)t * HI + h];
            Es[pr] = z > 0.f ? gc[cc] * wv : 0.f;
            Zs[pr] = gc[cc] * fmaxf(z, 0.f);
          }
          __syncthreads();
          if (tid < HI)
            for (int cc = 0; cc < kKB; ++cc) dw_acc += Zs[tid * kKB + cc];
#pragma unroll
          for (int i = 0; i < kMaxQ; ++i) {
            const int e = tid + i * 256;
            if (e < HI * dI) {
              const int h = e / dI, d = e - h * dI;
              float v = dq_acc[i];
              for (int cc = 0; cc < kKB; ++cc) v = fmaf(Es[h * kKB + cc], kIs[cc * (dI + 1) + d], v);
              dq_acc[i] = v;
            }
          }
          for (int e = tid; e < kKB * dI; e += 256) {
            const int cc = e / dI, d = e - cc * dI;
            const int id = rowid[cc];
            if (id < 0) continue;
            float v = 0.f;
            for (int h = 0; h < HI; ++h) v = fmaf(Es[h * kKB + cc], qIs[h * dI + d], v);
            atomicAdd(a.dkI + (int64_t)id * dI + d, v);
          }
        }
        __syncthreads();
      }
    }
  }
  if (tid == 0) a.kl[t] = z_acc > 0.0 ? (float)(kl_acc / z_acc - log1p(z_acc - 1.0)) : 0.f;
  if (a.grads) {
    if (tid < HI) a.dw[(int64_t)t * HI + tid] = dw_acc;
#pragma unroll
    for (int i = 0; i < kMaxQ; ++i) {
      const int e = tid + i * 256;
      if (e < HI * dI) a.dqI[(int64_t)t * HI * dI + e] = dq_acc[i];
    }
  }
}

// Deterministic sum of the per-query KL values: fixed strided partial sums, fixed tree.  The
// strided loads are issued 16 at a time and added in the same order as one by one.
__global__ __launch_bounds__(256) void k_sum(const float* __restrict__ x, int n,
                                             float* __restrict__ out) {
  __shared__ float red[256];
  constexpr int kU = 16;
  float s = 0.f;
  int i = threadIdx.x;
  for (; i + 256 * (kU - 1) < n; i += 256 * kU) {
    float v[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) v[j] = x[i + 256 * j];
#pragma unroll
    for (int j = 0; j < kU; ++j) s += v[j];
  }
  for (; i < n; i += 256) s += x[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

hipError_t launch_indexer_kl_mfma(const Shape& sh, const KlIO& io, hipStream_t s, bool* handled);
hipError_t launch_indexer_kl_cached(const Shape& sh, const KlIO& io, hipStream_t s, bool* handled);
hipError_t launch_indexer_kl_dense(const Shape& sh, const KlIO& io, hipStream_t s, bool* handled);
size_t indexer_kl_dense_workspace(const Shape& sh);

size_t indexer_kl_workspace(const Shape& sh) { return indexer_kl_dense_workspace(sh); }

hipError_t launch_indexer_kl(const Shape& sh, const KlIO& io, hipStream_t s) {
  if (sh.T == 0) {
    hipLaunchKernelGGL(k_sum, dim3(1), dim3(256), 0, s, io.kl, 0, io.loss);
    return hipGetLastError();
  }
  bool handled = false;
  hipError_t e = launch_indexer_kl_cached(sh, io, s, &handled);
  if (!handled && !io.t_logits) e = launch_indexer_kl_dense(sh, io, s, &handled);
  if (!handled) e = launch_indexer_kl_mfma(sh, io, s, &handled);
  if (!handled) {
    KlK a;
    a.q = io.q; a.kv_cmp = io.kv_cmp; a.scores = io.scores; a.ld = io.ld; a.idx = io.idx;
    a.qI = io.qI; a.qI_scale = io.qI_scale; a.w = io.w; a.kI = io.kI; a.kI_scale = io.kI_scale;
    a.cu = sh.cu; a.cu_cmp = sh.cu_cmp; a.gs = io.grad_scale; a.kl = io.kl; a.dqI = io.dqI;
    a.dw = io.dw; a.dkI = io.dkI; a.B = sh.B; a.H = sh.H; a.D = sh.D; a.r = sh.r;
    a.n_cap = sh.max_seqlen / sh.r; a.k_cap = sh.k_cap; a.teacher = sh.teacher; a.HI = sh.HI;
    a.dI = sh.dI; a.scale = sh.scale; a.grads = io.dqI != nullptr;
    const size_t lds = sizeof(float) * (kKB * (sh.D + 1) + sh.H * kKB + 2 * sh.H + sh.HI * sh.dI +
                                        kKB * (sh.dI + 1) + 2 * sh.HI * kKB + 3 * kKB) +
                       sizeof(int) * kKB;
    const dim3 grid(sh.T), block(256);
    if (sh.dtype == 0) {
      if (sh.idx_dtype == 0) hipLaunchKernelGGL((k_kl_generic<float, float>), grid, block, lds, s, a);
      else if (sh.idx_dtype == 1) hipLaunchKernelGGL((k_kl_generic<float, uint16_t>), grid, block, lds, s, a);
      else hipLaunchKernelGGL((k_kl_generic<float, uint8_t>), grid, block, lds, s, a);
    } else {
      if (sh.idx_dtype == 0) hipLaunchKernelGGL((k_kl_generic<uint16_t, float>), grid, block, lds, s, a);
      else if (sh.idx_dtype == 1) hipLaunchKernelGGL((k_kl_generic<uint16_t, uint16_t>), grid, block, lds, s, a);
      else hipLaunchKernelGGL((k_kl_generic<uint16_t, uint8_t>), grid, block, lds, s, a);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sum, dim3(1), dim3(256), 0, s, io.kl, sh.T, io.loss);
  return hipGetLastError();
}

}  // namespace csa
