// Sparse attention over compressed candidates + local window: forward and backward.
//
// "DeepSeek-V4 Attention Training Systems": the main attention of a CSA layer reads the
// top-k selected compressed entries plus a local sliding window (sparse phases), every
// completed compressed entry plus the window (dense mode, HCA), or the window alone
// (ratio-0 layer) (section 2 phase table); the forward returns the output and its
// log-sum-exp and the backward consumes the saved output, LSE and dO to produce query,
// KV and sink gradients without forming a dense attention matrix (section 8.2).  One
// 512-wide row is both key and value, shared by all heads (MQA).
//
// This file holds the scalar-fp32 kernels (fp32 operands, small head counts, and every
// shape without a matrix-core kernel) and the dispatch; the bf16 MFMA kernels for
// H = 64, D = 512 are in attn_mfma.hip.
#include <math.h>

#include "csa_device.h"
#include "csa_launch.h"

namespace csa {

struct AttnK {
  const void* q;
  const void* kv_cmp;
  const void* kv;
  const int32_t* idx;
  const float* sink;
  const int32_t* cu;
  const int32_t* cu_cmp;
  void* out;
  float* lse;
  float* lse_cmp;
  float* t_logits;
  int64_t ld_t;
  const void* o;
  const void* dout;
  void* dq;
  float* dkv_cmp;
  float* dkv;
  float* dsink;
  int B, H, D, r, n_cap, W, k_cap, mode, HG;
  float scale;
};

constexpr int kNB = 16;  // candidates per block

// Candidate bookkeeping of one query: compressed slots [0, n_c), masked padding
// [n_c, n_cs), then window rows.
struct Cands {
  int n_c, n_cs, n_w, row0, nv, win0;
};

// First -1 of an idx row (the number of leading selected entries); every lane returns it.
__device__ int leading_entries(const int32_t* __restrict__ row, int k_cap, int* s_tmp) {
  if (threadIdx.x == 0) *s_tmp = k_cap;
  __syncthreads();
  for (int c = threadIdx.x; c < k_cap; c += blockDim.x)
    if (row[c] < 0) atomicMin(s_tmp, c);
  __syncthreads();
  const int n = *s_tmp;
  __syncthreads();
  return n;
}

__device__ Cands make_cands(const AttnK& a, int t, const TokenInfo& ti, int* s_tmp) {
  Cands c;
  c.row0 = a.cu_cmp[ti.b];
  c.nv = min((ti.p + 1) / a.r, a.n_cap);
  c.n_w = min(a.W, ti.p + 1);
  c.win0 = t - c.n_w + 1;
  if (a.mode == 1) c.n_c = c.nv;
  else if (a.mode == 2) c.n_c = 0;
  else c.n_c = leading_entries(a.idx + (int64_t)t * a.k_cap, a.k_cap, s_tmp);
  c.n_cs = ((c.n_c + kNB - 1) / kNB) * kNB;   // whole blocks of compressed slots
  return c;
}

// Row id of candidate slot c: >= 0 compressed row, <= -2 window row -(id+2), -1 masked.
__device__ __forceinline__ int cand_row(const AttnK& a, int t, const Cands& cd, int c) {
  const int n = cd.n_cs + cd.n_w;
  if (c >= n) return -1;
  if (c < cd.n_c) {
    const int g = a.mode == 1 ? cd.row0 + c : a.idx[(int64_t)t * a.k_cap + c];
    return (g >= cd.row0 && g < cd.row0 + cd.nv) ? g : -1;
  }
  if (c < cd.n_cs) return -1;
  return -2 - (cd.win0 + (c - cd.n_cs));
}

template <typename T>
__device__ __forceinline__ void load_rows(const AttnK& a, const int* rowid, float* rs, int D) {
  const int Dp = D + 1;
  for (int e = threadIdx.x; e < kNB * D; e += 256) {
    const int cc = e / D, d = e - cc * D;
    const int id = rowid[cc];
    float v = 0.f;
    if (id >= 0) v = load1((const T*)a.kv_cmp + (int64_t)id * D + d);
    else if (id <= -2) v = load1((const T*)a.kv + (int64_t)(-2 - id) * D + d);
    rs[cc * Dp + d] = v;
  }
}

// ------------------------------------------------------------------ forward (scalar)
// Workgroup = (query t, group of HG heads).  Online softmax over blocks of 16 candidates.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_fwd_generic(AttnK a) {
  extern __shared__ float sm[];
  const int D = a.D, HG = a.HG, Dp = D + 1;
  float* qs = sm;                  // [HG*D]
  float* rs = qs + HG * D;         // [kNB*Dp]
  float* sl = rs + kNB * Dp;       // [HG*kNB]
  float* mh = sl + HG * kNB;       // [HG]
  float* lh = mh + HG;             // [HG]
  float* al = lh + HG;             // [HG]
  int* rowid = (int*)(al + HG);    // [kNB]
  __shared__ int s_tmp;
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int h0 = blockIdx.y * HG;
  T* outp = (T*)a.out + ((int64_t)t * a.H + h0) * D;
  TokenInfo ti;
  if (!token_info(a.cu, a.B, t, ti)) {
    for (int e = tid; e < HG * D; e += 256) store1(outp + e, 0.f);
    if (tid < HG) a.lse[(int64_t)t * a.H + h0 + tid] = 0.f;
    if (a.lse_cmp && tid < HG) a.lse_cmp[(int64_t)t * a.H + h0 + tid] = -INFINITY;
    return;
  }
  const Cands cd = make_cands(a, t, ti, &s_tmp);
  const T* qp = (const T*)a.q + ((int64_t)t * a.H + h0) * D;
  for (int e = tid; e < HG * D; e += 256) qs[e] = load1(qp + e);
  if (tid < HG) { mh[tid] = -INFINITY; lh[tid] = 0.f; }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float lse_c = -INFINITY;
  const int n = cd.n_cs + cd.n_w;
  for (int c0 = 0; c0 < n; c0 += kNB) {
    if (tid < kNB) rowid[tid] = cand_row(a, t, cd, c0 + tid);
    __syncthreads();
    load_rows<T>(a, rowid, rs, D);
    __syncthreads();
    for (int pr = tid; pr < HG * kNB; pr += 256) {
      const int h = pr / kNB, cc = pr - h * kNB;
      float s = -INFINITY;
      if (rowid[cc] != -1) {
        const float* qh = qs + h * D;
        const float* x = rs + cc * Dp;
        float z = 0.f;
        for (int d = 0; d < D; ++d) z = fmaf(qh[d], x[d], z);
        s = z * a.scale;
      }
      sl[pr] = s;
      if (a.t_logits && c0 + cc < cd.n_c)
        a.t_logits[((int64_t)t * a.H + h0 + h) * a.ld_t + c0 + cc] = s;
    }
    __syncthreads();
    if (tid < HG) {
      float* row = sl + tid * kNB;
      float mx = -INFINITY;
      for (int cc = 0; cc < kNB; ++cc) mx = fmaxf(mx, row[cc]);
      const float mold = mh[tid];
      const float mnew = fmaxf(mold, mx);
      float alpha = 1.f, sum = 0.f;
      if (mnew == -INFINITY) {
        for (int cc = 0; cc < kNB; ++cc) row[cc] = 0.f;
      } else {
        alpha = expf(mold - mnew);
        for (int cc = 0; cc < kNB; ++cc) {
          const float pv = expf(row[cc] - mnew);
          row[cc] = pv;
          sum += pv;
        }
      }
      lh[tid] = lh[tid] * alpha + sum;
      mh[tid] = mnew;
      al[tid] = alpha;
      if (c0 + kNB == cd.n_cs && lh[tid] > 0.f) lse_c = mnew + logf(lh[tid]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + i * 256;
      if (e < HG * D) {
        const int h = e / D, d = e - h * D;
        float v = acc[i] * al[h];
        const float* pr = sl + h * kNB;
        for (int cc = 0; cc < kNB; ++cc) v = fmaf(pr[cc], rs[cc * Dp + d], v);
        acc[i] = v;
      }
    }
    __syncthreads();
  }
  if (tid < HG) {
    const float m = mh[tid], l = lh[tid];
    float lse, f;
    if (a.sink) {
      const float sv = a.sink[h0 + tid];
      const float mf = fmaxf(m, sv);
      const float lf = l * expf(m - mf) + expf(sv - mf);
      lse = mf + logf(lf);
      f = expf(m - mf) / lf;
    } else {
      lse = m + logf(l);
      f = 1.f / l;
    }
    a.lse[(int64_t)t * a.H + h0 + tid] = lse;
    if (a.lse_cmp) a.lse_cmp[(int64_t)t * a.H + h0 + tid] = lse_c;
    al[tid] = f;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = tid + i * 256;
    if (e < HG * D) store1(outp + e, acc[i] * al[e / D]);
  }
}

// ------------------------------------------------------------------ backward (scalar)
template <typename T>
__global__ __launch_bounds__(256) void k_attn_bwd_generic(AttnK a) {
  extern __shared__ float sm[];
  const int D = a.D, HG = a.HG, Dp = D + 1;
  float* qs = sm;                  // [HG*D]
  float* dos = qs + HG * D;        // [HG*D]
  float* rs = dos + HG * D;        // [kNB*Dp]
  float* Ps = rs + kNB * Dp;       // [HG*kNB]
  float* dSs = Ps + HG * kNB;      // [HG*kNB]
  float* lse_s = dSs + HG * kNB;   // [HG]
  float* Dt_s = lse_s + HG;        // [HG]
  int* rowid = (int*)(Dt_s + HG);  // [kNB]
  __shared__ int s_tmp;
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int h0 = blockIdx.y * HG;
  T* dqp = (T*)a.dq + ((int64_t)t * a.H + h0) * D;
  TokenInfo ti;
  if (!token_info(a.cu, a.B, t, ti)) {
    for (int e = tid; e < HG * D; e += 256) store1(dqp + e, 0.f);
    return;
  }
  const Cands cd = make_cands(a, t, ti, &s_tmp);
  const int64_t off = ((int64_t)t * a.H + h0) * D;
  for (int e = tid; e < HG * D; e += 256) {
    qs[e] = load1((const T*)a.q + off + e);
    dos[e] = load1((const T*)a.dout + off + e);
  }
  __syncthreads();
  if (tid < HG) {
    const T* op = (const T*)a.o + off + tid * D;
    float s = 0.f;
    for (int d = 0; d < D; ++d) s = fmaf(dos[tid * D + d], load1(op + d), s);
    Dt_s[tid] = s;
    lse_s[tid] = a.lse[(int64_t)t * a.H + h0 + tid];
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const int n = cd.n_cs + cd.n_w;
  for (int c0 = 0; c0 < n; c0 += kNB) {
    if (tid < kNB) rowid[tid] = cand_row(a, t, cd, c0 + tid);
    __syncthreads();
    load_rows<T>(a, rowid, rs, D);
    __syncthreads();
    for (int pr = tid; pr < HG * kNB; pr += 256) {
      const int h = pr / kNB, cc = pr - h * kNB;
      float P = 0.f, dS = 0.f;
      if (rowid[cc] != -1) {
        const float* qh = qs + h * D;
        const float* gh = dos + h * D;
        const float* x = rs + cc * Dp;
        float z = 0.f, g = 0.f;
        for (int d = 0; d < D; ++d) {
          z = fmaf(qh[d], x[d], z);
          g = fmaf(gh[d], x[d], g);
        }
        P = expf(z * a.scale - lse_s[h]);
        dS = P * (g - Dt_s[h]);
      }
      Ps[pr] = P;
      dSs[pr] = dS;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + i * 256;
      if (e < HG * D) {
        const int h = e / D, d = e - h * D;
        float v = acc[i];
        const float* ds = dSs + h * kNB;
        for (int cc = 0; cc < kNB; ++cc) v = fmaf(ds[cc], rs[cc * Dp + d], v);
        acc[i] = v;
      }
    }
    for (int e = tid; e < kNB * D; e += 256) {
      const int cc = e / D, d = e - cc * D;
      const int id = rowid[cc];
      if (id == -1) continue;
      float v = 0.f;
      for (int h = 0; h < HG; ++h)
        v += a.scale * dSs[h * kNB + cc] * qs[h * D + d] + Ps[h * kNB + cc] * dos[h * D + d];
      float* dst = id >= 0 ? a.dkv_cmp + (int64_t)id * D + d : a.dkv + (int64_t)(-2 - id) * D + d;
      atomicAdd(dst, v);
    }
    __syncthreads();
  }
  if (tid < HG && a.sink && a.dsink)
    atomicAdd(a.dsink + h0 + tid, -expf(a.sink[h0 + tid] - lse_s[tid]) * Dt_s[tid]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = tid + i * 256;
    if (e < HG * D) store1(dqp + e, acc[i] * a.scale);
  }
}

// ------------------------------------------------------------------ dispatch
hipError_t launch_attn_fwd_mfma(const Shape& sh, const AttnIO& io, hipStream_t s, bool* handled);
hipError_t launch_attn_bwd_mfma(const Shape& sh, const AttnIO& io, hipStream_t s, bool* handled);

static int head_group(int H, int D) {
  int best = 1;
  for (int g = 1; g <= H; ++g)
    if (H % g == 0 && g * D <= 2048) best = g;
  return best;
}

static AttnK make_k(const Shape& sh, const AttnIO& io) {
  AttnK a;
  a.q = io.q; a.kv_cmp = io.kv_cmp; a.kv = io.kv; a.idx = io.idx; a.sink = io.sink;
  a.cu = sh.cu; a.cu_cmp = sh.cu_cmp; a.out = io.out; a.lse = io.lse; a.lse_cmp = io.lse_cmp;
  a.t_logits = io.t_logits; a.ld_t = teacher_logits_ld(sh);
  a.o = io.o;
  a.dout = io.dout; a.dq = io.dq; a.dkv_cmp = io.dkv_cmp; a.dkv = io.dkv; a.dsink = io.dsink;
  a.B = sh.B; a.H = sh.H; a.D = sh.D; a.r = sh.r; a.n_cap = sh.r > 0 ? sh.max_seqlen / sh.r : 0;
  a.W = sh.W; a.k_cap = sh.k_cap; a.mode = sh.mode; a.HG = head_group(sh.H, sh.D);
  a.scale = sh.scale;
  return a;
}

size_t attn_fwd_workspace(const Shape& sh) { (void)sh; return 0; }
size_t attn_bwd_workspace_mfma(const Shape& sh);
size_t attn_bwd_workspace_min_mfma(const Shape& sh);
size_t attn_bwd_workspace(const Shape& sh) { return attn_bwd_workspace_mfma(sh); }
size_t attn_bwd_workspace_min(const Shape& sh) { return attn_bwd_workspace_min_mfma(sh); }

hipError_t launch_attn_fwd(const Shape& sh, const AttnIO& io, hipStream_t s) {
  if (sh.T == 0) return hipSuccess;
  bool handled = false;
  hipError_t e = launch_attn_fwd_mfma(sh, io, s, &handled);
  if (handled) return e;
  const AttnK a = make_k(sh, io);
  const dim3 grid(sh.T, sh.H / a.HG);
  const size_t lds = sizeof(float) * (a.HG * sh.D + kNB * (sh.D + 1) + a.HG * kNB + 3 * a.HG) +
                     sizeof(int) * kNB;
  if (sh.dtype == 0) hipLaunchKernelGGL(k_attn_fwd_generic<float>, grid, dim3(256), lds, s, a);
  else hipLaunchKernelGGL(k_attn_fwd_generic<uint16_t>, grid, dim3(256), lds, s, a);
  e = hipGetLastError();
  // the generic kernel has no rotating epilogue: the inverse rotation reads the output back
  if (e == hipSuccess && io.out_rot)
    e = launch_rope(sh.dtype, io.out, io.out_rot, sh.T, sh.H, sh.D, sh.rope_dim, sh.rope_theta,
                    1, sh.B, sh.cu, s);
  return e;
}

hipError_t launch_attn_bwd(const Shape& sh, const AttnIO& io, hipStream_t s) {
  if (sh.T == 0) return hipSuccess;
  bool handled = false;
  hipError_t e = launch_attn_bwd_mfma(sh, io, s, &handled);
  if (handled) return e;
  const AttnK a = make_k(sh, io);
  const dim3 grid(sh.T, sh.H / a.HG);
  const size_t lds = sizeof(float) * (2 * a.HG * sh.D + kNB * (sh.D + 1) + 2 * a.HG * kNB +
                                      2 * a.HG) + sizeof(int) * kNB;
  if (sh.dtype == 0) hipLaunchKernelGGL(k_attn_bwd_generic<float>, grid, dim3(256), lds, s, a);
  else hipLaunchKernelGGL(k_attn_bwd_generic<uint16_t>, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace csa
