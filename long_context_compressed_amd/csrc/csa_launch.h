// Internal launcher interface between the C ABI (csa_api.cpp) and the kernels (*.hip).
// Every launcher assumes its arguments were validated on the host.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

// Shape and metadata common to the per-token kernels.
struct Shape {
  int B;          // samples
  int T;          // capacity rows
  int max_seqlen; // host bound on L_b
  int r;          // ratio
  int W;          // window
  int k;          // top-k
  int k_cap;      // idx row width
  int H, D;       // heads, head dim
  int HI, dI;     // indexer heads, indexer dim
  float scale;
  int mode;       // csa_mode_t
  int teacher;    // csa_teacher_t
  int dtype;      // csa_dtype_t main operands
  int idx_dtype;  // csa_dtype_t indexer operands
  int rope_dim;   // rotary band width (0: none)
  float rope_theta;
  const int32_t* cu;      // cu_seqlens [B+1]
  const int32_t* cu_cmp;  // cu_cmp [B+1]
};

hipError_t launch_cmp_seqlens(const int32_t* cu, int B, int r, int32_t* cu_cmp, hipStream_t s);
hipError_t launch_validate_metadata(const int32_t* cu, int B, int T, int max_seqlen,
                                    int32_t* status, hipStream_t s);
hipError_t launch_compress(const Shape& sh, int dtype, const void* x, int dim, void* x_cmp,
                           hipStream_t s);
hipError_t launch_compress_bwd(const Shape& sh, const float* d_cmp, int dim, float* dx,
                               hipStream_t s);
hipError_t launch_compress_learned(const Shape& sh, int dtype, const void* x, const void* score,
                                   const float* bias, int dim, int overlap, void* x_cmp,
                                   hipStream_t s);
hipError_t launch_compress_learned_bwd(const Shape& sh, int dtype, const void* x,
                                       const void* score, const float* bias,
                                       const float* d_x_cmp, int dim, int overlap, float* dx,
                                       float* dscore, float* dbias, hipStream_t s);
// Rotary embedding of rows [rows, heads, dim] at positions row - offs[b] (sample b);
// y == x rotates in place (rotary channels only), else y receives every channel.
hipError_t launch_rope(int dtype, const void* x, void* y, int64_t rows, int heads, int dim,
                       int rope_dim, float theta, int inverse, int B, const int32_t* offs,
                       hipStream_t s);
hipError_t launch_quantize_fp8(const void* x, int dtype, int64_t rows, int row_len,
                               uint8_t* codes, float* scale, hipStream_t s);
hipError_t launch_index_scores(const Shape& sh, const void* qI, const float* qI_scale,
                               const float* w, const void* kI, const float* kI_scale,
                               float* scores, int64_t ld, hipStream_t s);
hipError_t launch_topk(const Shape& sh, const float* scores, int64_t ld, int32_t* idx,
                       hipStream_t s);
// fused scores + top-k; *handled = false when the shape has no fused kernel
hipError_t launch_index_topk(const Shape& sh, const void* qI, const float* qI_scale,
                             const float* w, const void* kI, const float* kI_scale,
                             int scores_mode, float* scores, int64_t ld, int32_t* idx,
                             hipStream_t s, bool* handled);

struct AttnIO {
  const void* q;
  const void* kv_cmp;
  const void* kv;
  const int32_t* idx;
  const float* sink;
  void* out;
  void* out_rot;     // optional: out inverse-rotated at the query position (rope_dim > 0)
  float* lse;
  float* lse_cmp;    // optional: log-sum-exp over the compressed candidates only
  float* t_logits;   // optional: compressed-candidate logits [T, H, ld_t]
  // backward only
  const void* o;
  const void* dout;
  void* dq;
  float* dkv_cmp;
  float* dkv;
  float* dsink;
  void* ws;
  size_t ws_bytes;
};

size_t attn_fwd_workspace(const Shape& sh);
size_t attn_bwd_workspace(const Shape& sh);       // preferred size
size_t attn_bwd_workspace_min(const Shape& sh);   // smallest size the call accepts
hipError_t launch_attn_fwd(const Shape& sh, const AttnIO& io, hipStream_t s);
hipError_t launch_attn_bwd(const Shape& sh, const AttnIO& io, hipStream_t s);
// The backward with its workspace in the library's static per-device array (io.ws ignored).
size_t attn_bwd_scratch_bytes();
hipError_t launch_attn_bwd_noalloc(const Shape& sh, AttnIO io, hipStream_t s);

struct KlIO {
  const void* q;
  const void* kv_cmp;
  const float* scores;
  int64_t ld;
  const int32_t* idx;
  const float* teacher_lse;   // optional per-head teacher normalizer (selected teacher)
  const float* t_logits;      // optional teacher logits cache [T, H, ld_t]
  const void* qI;
  const float* qI_scale;
  const float* w;
  const void* kI;
  const float* kI_scale;
  float grad_scale;
  float* kl;
  float* loss;
  float* dqI;
  float* dw;
  float* dkI;
  void* ws;
  size_t ws_bytes;
};

// Matrix-core scores of tokens t_lo .. t_hi - 1 (t_hi < 0: through T) into rows t - t_lo of
// scores; handled = false for shapes without a matrix-core kernel.
hipError_t launch_index_scores_mfma(const Shape& sh, const void* qI, const float* qI_scale,
                                    const float* w, const void* kI, const float* kI_scale,
                                    float* scores, int64_t ld, hipStream_t s, bool* handled,
                                    int t_lo = 0, int t_hi = -1);
// Whether csa_indexer_kl can form the student scores itself (scores == NULL).
bool indexer_kl_recomputes_scores(const Shape& sh);
size_t indexer_kl_workspace(const Shape& sh);
size_t indexer_kl_cached_workspace(const Shape& sh);

// Row stride of the teacher-logit cache: compressed-slot capacity rounded up to 64.
inline int64_t teacher_logits_ld(const Shape& sh) {
  const int64_t n = sh.mode == 0 ? sh.k_cap : (sh.mode == 1 ? sh.max_seqlen / sh.r : 0);
  return ((n + 63) / 64) * 64;
}
hipError_t launch_indexer_kl(const Shape& sh, const KlIO& io, hipStream_t s);

}  // namespace csa
