// C ABI entry points: host-side argument validation, then one or more kernel launches.
// Validation never touches the device; an invalid call returns with nothing enqueued.
#include <math.h>

#include "../../include/csa.h"
#include "csa_launch.h"

namespace {

using csa::Shape;

bool dtype_main_ok(int d) { return d == CSA_F32 || d == CSA_BF16; }
bool dtype_idx_ok(int d) { return d == CSA_F32 || d == CSA_BF16 || d == CSA_FP8_E4M3; }

// Checks shared by every per-token call.
csa_status_t check_common(const csa_params_t* p) {
  if (!p) return CSA_ERR_NULL;
  if (p->batch < 0 || p->total_tokens < 0 || p->max_seqlen < 0) return CSA_ERR_ARG;
  if (p->ratio < 1 || p->ratio > 4096) return CSA_ERR_ARG;
  return CSA_OK;
}

int n_cap_of(const csa_params_t* p) { return p->max_seqlen / p->ratio; }

csa_status_t check_attn(const csa_params_t* p) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (p->window < 1) return CSA_ERR_ARG;
  if (p->mode < CSA_SPARSE || p->mode > CSA_WINDOW) return CSA_ERR_ARG;
  if (p->mode == CSA_SPARSE && (p->topk < 1 || p->topk_cap < p->topk || p->topk_cap % 64 != 0))
    return CSA_ERR_ARG;
  if (!(p->scale > 0.f) || !isfinite(p->scale)) return CSA_ERR_ARG;
  if (p->heads < 1 || p->head_dim < 8) return CSA_ERR_ARG;
  if (!dtype_main_ok(p->dtype)) return CSA_ERR_UNSUPPORTED;
  if (p->heads > 128 || p->head_dim > 512 || p->head_dim % 8 != 0) return CSA_ERR_UNSUPPORTED;
  if (p->rope_dim < 0 || p->rope_dim > p->head_dim || p->rope_dim % 8 != 0) return CSA_ERR_ARG;
  if (p->rope_dim > 0 && !(p->rope_theta > 0.f && isfinite(p->rope_theta))) return CSA_ERR_ARG;
  return CSA_OK;
}

csa_status_t check_indexer(const csa_params_t* p) {
  if (p->idx_heads < 1 || p->idx_dim < 8) return CSA_ERR_ARG;
  if (!dtype_idx_ok(p->idx_dtype)) return CSA_ERR_UNSUPPORTED;
  if (p->idx_heads > 64 || p->idx_dim > 128 || p->idx_dim % 8 != 0) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

Shape make_shape(const csa_params_t* p, const int32_t* cu, const int32_t* cu_cmp) {
  Shape s;
  s.B = p->batch; s.T = p->total_tokens; s.max_seqlen = p->max_seqlen; s.r = p->ratio;
  s.W = p->window; s.k = p->topk; s.k_cap = p->topk_cap; s.H = p->heads; s.D = p->head_dim;
  s.HI = p->idx_heads; s.dI = p->idx_dim; s.scale = p->scale; s.mode = p->mode;
  s.teacher = p->teacher; s.dtype = p->dtype; s.idx_dtype = p->idx_dtype; s.cu = cu;
  s.cu_cmp = cu_cmp; s.rope_dim = p->rope_dim; s.rope_theta = p->rope_theta;
  return s;
}

csa_status_t launched(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH; }

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(csa_status_t s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL: return "a required pointer is NULL";
    case CSA_ERR_ARG: return "an argument is out of range";
    case CSA_ERR_UNSUPPORTED: return "dtype or shape combination not supported";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

csa_status_t csa_workspace_size(const csa_params_t* p, int32_t op, size_t* bytes) {
  if (!p || !bytes) return CSA_ERR_NULL;
  csa_status_t st = check_common(p);
  if (st) return st;
  const Shape sh = make_shape(p, nullptr, nullptr);
  switch (op) {
    case CSA_OP_ATTN_FWD: *bytes = csa::attn_fwd_workspace(sh); return CSA_OK;
    case CSA_OP_ATTN_BWD: *bytes = csa::attn_bwd_workspace(sh); return CSA_OK;
    case CSA_OP_INDEXER_KL: *bytes = csa::indexer_kl_workspace(sh); return CSA_OK;
    case CSA_OP_INDEXER_KL_CACHED: *bytes = csa::indexer_kl_cached_workspace(sh); return CSA_OK;
    default: return CSA_ERR_ARG;
  }
}

csa_status_t csa_workspace_size_min(const csa_params_t* p, int32_t op, size_t* bytes) {
  if (!p || !bytes) return CSA_ERR_NULL;
  if (op == CSA_OP_ATTN_BWD) {
    csa_status_t st = check_common(p);
    if (st) return st;
    *bytes = csa::attn_bwd_workspace_min(make_shape(p, nullptr, nullptr));
    return CSA_OK;
  }
  return csa_workspace_size(p, op, bytes);
}

csa_status_t csa_cmp_seqlens(const int32_t* cu_seqlens, int32_t batch, int32_t ratio,
                             int32_t* cu_cmp, hipStream_t stream) {
  if (!cu_seqlens || !cu_cmp) return CSA_ERR_NULL;
  if (batch < 0 || ratio < 1 || ratio > 4096) return CSA_ERR_ARG;
  return launched(csa::launch_cmp_seqlens(cu_seqlens, batch, ratio, cu_cmp, stream));
}

csa_status_t csa_validate_metadata(const csa_params_t* p, const int32_t* cu_seqlens,
                                   int32_t* status_dev, hipStream_t stream) {
  if (!p || !cu_seqlens || !status_dev) return CSA_ERR_NULL;
  if (p->batch < 0 || p->total_tokens < 0 || p->max_seqlen < 0) return CSA_ERR_ARG;
  return launched(csa::launch_validate_metadata(cu_seqlens, p->batch, p->total_tokens,
                                                p->max_seqlen, status_dev, stream));
}

csa_status_t csa_compress(const csa_params_t* p, int32_t dtype, const void* x, int32_t dim,
                          const int32_t* cu_seqlens, const int32_t* cu_cmp, void* x_cmp,
                          hipStream_t stream) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (!x || !cu_seqlens || !cu_cmp || !x_cmp) return CSA_ERR_NULL;
  if (dim < 8) return CSA_ERR_ARG;
  if (!dtype_main_ok(dtype) || dim % 8 != 0 || dim > 2048) return CSA_ERR_UNSUPPORTED;
  return launched(csa::launch_compress(make_shape(p, cu_seqlens, cu_cmp), dtype, x, dim, x_cmp,
                                       stream));
}

csa_status_t csa_compress_bwd(const csa_params_t* p, const float* d_x_cmp, int32_t dim,
                              const int32_t* cu_seqlens, const int32_t* cu_cmp, float* dx,
                              hipStream_t stream) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (!d_x_cmp || !cu_seqlens || !cu_cmp || !dx) return CSA_ERR_NULL;
  if (dim < 8) return CSA_ERR_ARG;
  if (dim % 8 != 0 || dim > 2048) return CSA_ERR_UNSUPPORTED;
  return launched(csa::launch_compress_bwd(make_shape(p, cu_seqlens, cu_cmp), d_x_cmp, dim, dx,
                                           stream));
}

static csa_status_t check_learned(const csa_params_t* p, int32_t dtype, int32_t dim,
                                  int32_t overlap) {
  if (dim < 8 || (overlap != 0 && overlap != 1)) return CSA_ERR_ARG;
  if (!dtype_main_ok(dtype) || dim % 8 != 0 || dim > 2048) return CSA_ERR_UNSUPPORTED;
  (void)p;
  return CSA_OK;
}

csa_status_t csa_compress_learned(const csa_params_t* p, int32_t dtype, const void* x,
                                  const void* score, const float* bias, int32_t dim,
                                  int32_t overlap, const int32_t* cu_seqlens,
                                  const int32_t* cu_cmp, void* x_cmp, hipStream_t stream) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (!x || !score || !bias || !cu_seqlens || !cu_cmp || !x_cmp) return CSA_ERR_NULL;
  st = check_learned(p, dtype, dim, overlap);
  if (st) return st;
  return launched(csa::launch_compress_learned(make_shape(p, cu_seqlens, cu_cmp), dtype, x, score,
                                               bias, dim, overlap, x_cmp, stream));
}

csa_status_t csa_compress_learned_bwd(const csa_params_t* p, int32_t dtype, const void* x,
                                      const void* score, const float* bias,
                                      const float* d_x_cmp, int32_t dim, int32_t overlap,
                                      const int32_t* cu_seqlens, const int32_t* cu_cmp,
                                      float* dx, float* dscore, float* dbias,
                                      hipStream_t stream) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (!x || !score || !bias || !d_x_cmp || !cu_seqlens || !cu_cmp || !dx || !dscore || !dbias)
    return CSA_ERR_NULL;
  st = check_learned(p, dtype, dim, overlap);
  if (st) return st;
  return launched(csa::launch_compress_learned_bwd(make_shape(p, cu_seqlens, cu_cmp), dtype, x,
                                                   score, bias, d_x_cmp, dim, overlap, dx, dscore,
                                                   dbias, stream));
}

csa_status_t csa_quantize_fp8(const void* x, int32_t x_dtype, int64_t rows, int32_t row_len,
                              uint8_t* codes, float* row_scale, hipStream_t stream) {
  if (!x || !codes || !row_scale) return CSA_ERR_NULL;
  if (rows < 0 || row_len < 8) return CSA_ERR_ARG;
  if (!dtype_main_ok(x_dtype) || row_len % 8 != 0 || row_len > 1024) return CSA_ERR_UNSUPPORTED;
  return launched(csa::launch_quantize_fp8(x, x_dtype, rows, row_len, codes, row_scale, stream));
}

csa_status_t csa_index_scores(const csa_params_t* p, const void* qI, const float* qI_scale,
                              const float* w, const void* kI_cmp, const float* kI_scale,
                              const int32_t* cu_seqlens, const int32_t* cu_cmp, float* scores,
                              int64_t ld_scores, hipStream_t stream) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (!qI || !w || !kI_cmp || !cu_seqlens || !cu_cmp || !scores) return CSA_ERR_NULL;
  st = check_indexer(p);
  if (st) return st;
  const bool fp8 = p->idx_dtype == CSA_FP8_E4M3;
  if (fp8 && (!qI_scale || !kI_scale)) return CSA_ERR_NULL;
  if (ld_scores < n_cap_of(p)) return CSA_ERR_ARG;
  return launched(csa::launch_index_scores(make_shape(p, cu_seqlens, cu_cmp), qI,
                                           fp8 ? qI_scale : nullptr, w, kI_cmp,
                                           fp8 ? kI_scale : nullptr, scores, ld_scores, stream));
}

csa_status_t csa_topk_select(const csa_params_t* p, const float* scores, int64_t ld_scores,
                             const int32_t* cu_seqlens, const int32_t* cu_cmp, int32_t* idx,
                             hipStream_t stream) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (!scores || !cu_seqlens || !cu_cmp || !idx) return CSA_ERR_NULL;
  if (p->topk < 1 || p->topk_cap < p->topk || p->topk_cap % 64 != 0) return CSA_ERR_ARG;
  if (ld_scores < n_cap_of(p)) return CSA_ERR_ARG;
  if (n_cap_of(p) > 64 * 512) return CSA_ERR_UNSUPPORTED;
  return launched(csa::launch_topk(make_shape(p, cu_seqlens, cu_cmp), scores, ld_scores, idx,
                                   stream));
}

csa_status_t csa_index_topk(const csa_params_t* p, const void* qI, const float* qI_scale,
                            const float* w, const void* kI_cmp, const float* kI_scale,
                            const int32_t* cu_seqlens, const int32_t* cu_cmp, int32_t scores_mode,
                            float* scores, int64_t ld_scores, int32_t* idx, hipStream_t stream) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (!qI || !w || !kI_cmp || !cu_seqlens || !cu_cmp || !idx) return CSA_ERR_NULL;
  if (scores_mode < 0 || scores_mode > 2) return CSA_ERR_ARG;
  if (scores_mode != 0 && !scores) return CSA_ERR_NULL;
  if (scores_mode != 0 && ld_scores < n_cap_of(p)) return CSA_ERR_ARG;
  st = check_indexer(p);
  if (st) return st;
  const bool fp8 = p->idx_dtype == CSA_FP8_E4M3;
  if (fp8 && (!qI_scale || !kI_scale)) return CSA_ERR_NULL;
  if (p->topk < 1 || p->topk_cap < p->topk || p->topk_cap % 64 != 0) return CSA_ERR_ARG;
  if (p->idx_heads != 64 || p->idx_dim != 128 || p->idx_dtype == CSA_F32 || n_cap_of(p) > 64 * 512)
    return CSA_ERR_UNSUPPORTED;
  bool handled = false;
  const hipError_t e = csa::launch_index_topk(make_shape(p, cu_seqlens, cu_cmp), qI,
                                              fp8 ? qI_scale : nullptr, w, kI_cmp,
                                              fp8 ? kI_scale : nullptr, scores_mode, scores,
                                              ld_scores, idx, stream, &handled);
  if (!handled) return CSA_ERR_UNSUPPORTED;
  return launched(e);
}

csa_status_t csa_sparse_attn_fwd(const csa_params_t* p, const void* q, const void* kv_cmp,
                                 const void* kv, const int32_t* idx, const float* sink,
                                 const int32_t* cu_seqlens, const int32_t* cu_cmp, void* out,
                                 void* out_rot, float* lse, float* lse_cmp, float* t_logits,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  csa_status_t st = check_attn(p);
  if (st) return st;
  if (!q || !kv || !cu_seqlens || !cu_cmp || !out || !lse) return CSA_ERR_NULL;
  if (out_rot && (p->rope_dim == 0 || out_rot == out)) return CSA_ERR_ARG;
  if (p->mode != CSA_WINDOW && !kv_cmp) return CSA_ERR_NULL;
  if (p->mode == CSA_SPARSE && !idx) return CSA_ERR_NULL;
  const Shape sh = make_shape(p, cu_seqlens, cu_cmp);
  const size_t need = csa::attn_fwd_workspace(sh);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  csa::AttnIO io = {};
  io.q = q; io.kv_cmp = kv_cmp; io.kv = kv; io.idx = p->mode == CSA_SPARSE ? idx : nullptr;
  io.sink = sink; io.out = out; io.out_rot = out_rot; io.lse = lse; io.lse_cmp = lse_cmp;
  io.t_logits = p->mode == CSA_WINDOW ? nullptr : t_logits; io.ws = ws; io.ws_bytes = ws_bytes;
  return launched(csa::launch_attn_fwd(sh, io, stream));
}

csa_status_t csa_rope(int32_t dtype, const void* x, void* y, int64_t rows, int32_t heads,
                      int32_t dim, int32_t rope_dim, float theta, int32_t inverse,
                      int32_t batch, const int32_t* row_offsets, hipStream_t stream) {
  if (!row_offsets || (rows > 0 && (!x || !y))) return CSA_ERR_NULL;
  if (rows < 0 || rows > INT32_MAX || heads < 1 || dim < 8 || batch < 0) return CSA_ERR_ARG;
  if (inverse != 0 && inverse != 1) return CSA_ERR_ARG;
  if (dim % 8 != 0 || rope_dim < 8 || rope_dim > dim || rope_dim % 8 != 0) return CSA_ERR_ARG;
  if (!(theta > 0.f) || !isfinite(theta)) return CSA_ERR_ARG;
  if (dtype != CSA_F32 && dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  return launched(csa::launch_rope(dtype, x, y, rows, heads, dim, rope_dim, theta, inverse, batch,
                                   row_offsets, stream));
}

int64_t csa_teacher_logits_stride(const csa_params_t* p) {
  if (check_attn(p) != CSA_OK) return 0;
  return csa::teacher_logits_ld(make_shape(p, nullptr, nullptr));
}

csa_status_t csa_sparse_attn_bwd(const csa_params_t* p, const void* q, const void* kv_cmp,
                                 const void* kv, const int32_t* idx, const float* sink,
                                 const int32_t* cu_seqlens, const int32_t* cu_cmp,
                                 const void* out, const float* lse, const void* d_out, void* dq,
                                 float* dkv_cmp, float* dkv, float* dsink, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  csa_status_t st = check_attn(p);
  if (st) return st;
  if (!q || !kv || !cu_seqlens || !cu_cmp || !out || !lse || !d_out || !dq || !dkv)
    return CSA_ERR_NULL;
  if (p->mode != CSA_WINDOW && (!kv_cmp || !dkv_cmp)) return CSA_ERR_NULL;
  if (p->mode == CSA_SPARSE && !idx) return CSA_ERR_NULL;
  const Shape sh = make_shape(p, cu_seqlens, cu_cmp);
  const size_t need = csa::attn_bwd_workspace_min(sh);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  csa::AttnIO io = {};
  io.q = q; io.kv_cmp = kv_cmp; io.kv = kv; io.idx = p->mode == CSA_SPARSE ? idx : nullptr;
  io.sink = sink; io.o = out; io.lse = const_cast<float*>(lse); io.dout = d_out; io.dq = dq;
  io.dkv_cmp = dkv_cmp; io.dkv = dkv; io.dsink = sink ? dsink : nullptr; io.ws = ws;
  io.ws_bytes = ws_bytes;
  return launched(csa::launch_attn_bwd(sh, io, stream));
}

csa_status_t csa_sparse_attn_bwd_noalloc(const csa_params_t* p, const void* q,
                                         const void* kv_cmp, const void* kv, const int32_t* idx,
                                         const float* sink, const int32_t* cu_seqlens,
                                         const int32_t* cu_cmp, const void* out, const float* lse,
                                         const void* d_out, void* dq, float* dkv_cmp, float* dkv,
                                         float* dsink, hipStream_t stream) {
  csa_status_t st = check_attn(p);
  if (st) return st;
  if (!q || !kv || !cu_seqlens || !cu_cmp || !out || !lse || !d_out || !dq || !dkv)
    return CSA_ERR_NULL;
  if (p->mode != CSA_WINDOW && (!kv_cmp || !dkv_cmp)) return CSA_ERR_NULL;
  if (p->mode == CSA_SPARSE && !idx) return CSA_ERR_NULL;
  const Shape sh = make_shape(p, cu_seqlens, cu_cmp);
  if (csa::attn_bwd_workspace_min(sh) > csa::attn_bwd_scratch_bytes()) return CSA_ERR_WORKSPACE;
  csa::AttnIO io = {};
  io.q = q; io.kv_cmp = kv_cmp; io.kv = kv; io.idx = p->mode == CSA_SPARSE ? idx : nullptr;
  io.sink = sink; io.o = out; io.lse = const_cast<float*>(lse); io.dout = d_out; io.dq = dq;
  io.dkv_cmp = dkv_cmp; io.dkv = dkv; io.dsink = sink ? dsink : nullptr;
  return launched(csa::launch_attn_bwd_noalloc(sh, io, stream));
}

csa_status_t csa_indexer_kl(const csa_params_t* p, const void* q, const void* kv_cmp,
                            const float* scores, int64_t ld_scores, const int32_t* idx,
                            const float* teacher_lse, const float* teacher_logits,
                            const void* qI, const float* qI_scale,
                            const float* w, const void* kI_cmp, const float* kI_scale,
                            const int32_t* cu_seqlens, const int32_t* cu_cmp, float grad_scale,
                            float* kl, float* loss, float* dqI, float* dw, float* dkI_cmp,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  csa_status_t st = check_common(p);
  if (st) return st;
  if (!q || !kv_cmp || !qI || !w || !kI_cmp || !cu_seqlens || !cu_cmp || !kl || !loss)
    return CSA_ERR_NULL;
  if (p->teacher != CSA_TEACHER_SELECTED && p->teacher != CSA_TEACHER_DENSE) return CSA_ERR_ARG;
  if (p->teacher == CSA_TEACHER_SELECTED) {
    if (!idx) return CSA_ERR_NULL;
    if (p->topk_cap < 1 || p->topk_cap % 64 != 0) return CSA_ERR_ARG;
  }
  const int ngrad = (dqI != nullptr) + (dw != nullptr) + (dkI_cmp != nullptr);
  if (ngrad != 0 && ngrad != 3) return CSA_ERR_NULL;
  if (!(p->scale > 0.f) || !isfinite(p->scale) || !isfinite(grad_scale)) return CSA_ERR_ARG;
  if (p->heads < 1 || p->head_dim < 8) return CSA_ERR_ARG;
  if (!dtype_main_ok(p->dtype)) return CSA_ERR_UNSUPPORTED;
  if (p->heads > 64 || p->head_dim > 512 || p->head_dim % 8 != 0) return CSA_ERR_UNSUPPORTED;
  st = check_indexer(p);
  if (st) return st;
  const bool fp8 = p->idx_dtype == CSA_FP8_E4M3;
  if (fp8 && (!qI_scale || !kI_scale)) return CSA_ERR_NULL;
  if (scores && ld_scores < n_cap_of(p)) return CSA_ERR_ARG;
  if (!scores && (teacher_logits ||
                  !csa::indexer_kl_recomputes_scores(make_shape(p, cu_seqlens, cu_cmp))))
    return CSA_ERR_NULL;
  if (teacher_logits) {
    const bool same_set = (p->teacher == CSA_TEACHER_SELECTED && p->mode == CSA_SPARSE) ||
                          (p->teacher == CSA_TEACHER_DENSE && p->mode == CSA_DENSE);
    if (!same_set || check_attn(p) != CSA_OK) return CSA_ERR_ARG;
  }
  const Shape sh = make_shape(p, cu_seqlens, cu_cmp);
  const size_t need = teacher_logits ? csa::indexer_kl_cached_workspace(sh)
                                     : csa::indexer_kl_workspace(sh);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  csa::KlIO io = {};
  io.t_logits = teacher_logits;
  io.q = q; io.kv_cmp = kv_cmp; io.scores = scores; io.ld = ld_scores;
  io.idx = p->teacher == CSA_TEACHER_SELECTED ? idx : nullptr; io.qI = qI;
  io.teacher_lse = p->teacher == CSA_TEACHER_SELECTED ? teacher_lse : nullptr;
  io.qI_scale = fp8 ? qI_scale : nullptr; io.w = w; io.kI = kI_cmp;
  io.kI_scale = fp8 ? kI_scale : nullptr; io.grad_scale = grad_scale; io.kl = kl; io.loss = loss;
  io.dqI = dqI; io.dw = dw; io.dkI = dkI_cmp; io.ws = ws; io.ws_bytes = ws_bytes;
  return launched(csa::launch_indexer_kl(sh, io, stream));
}

}  // extern "C"
