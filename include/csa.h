/*
 * csa.h -- C ABI of the compressed-sparse-attention (CSA / HCA) layer library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the DeepSeek-V4 hybrid attention as described on the page
 * "DeepSeek-V4 Attention Training Systems" (v4-attn-notes, training-systems
 * chapter).  One layer step on a packed variable-length (THD) batch is:
 *
 *   csa_cmp_seqlens      compressed-row offsets from cu_seqlens           (section 4)
 *   csa_compress         ratio-r compressor, main KV and indexer key      (section 4)
 *   csa_quantize_fp8     optional e4m3 operands of an FP8 indexer         (section 9)
 *   csa_index_scores     lightning-indexer logits over visible entries   (section 3)
 *   csa_topk_select      per-query top-k + lowering to global rows        (sections 3, 8.1, 8.2)
 *   csa_index_topk       the two above fused: logits never leave the chip  (sections 3, 8.2)
 *   csa_sparse_attn_fwd  selected (or all) compressed rows + local window (sections 2, 8.2)
 *   csa_indexer_kl       KL auxiliary loss and its eager indexer backward (sections 3, 8.2)
 *   csa_sparse_attn_bwd  dq, dkv, dsink from saved O, LSE and dO          (section 8.2)
 *   csa_compress_bwd     adjoint of the compressor                        (section 3 ownership)
 *   csa_compress_learned      learned-score compressor, overlapping groups (sections 4, 5.1, 8.2, 9)
 *   csa_compress_learned_bwd  its adjoint
 *   csa_rope             rotary embedding / its inverse at per-sample positions (sections 4, 12)
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers, row-major, densely packed unless a
 *   leading dimension is given.  Every call is asynchronous on the given stream,
 *   never synchronizes the host, never allocates or frees memory and keeps no
 *   state between calls; the caller owns every buffer, including workspaces
 *   (sizes from csa_workspace_size).  Nothing depends on device values on the
 *   host side, so the packed lengths may change between calls within the same
 *   capacity (the static-capacity contract of section 4.1).
 * - Packed layout (section 4): sample b of B occupies rows cu_seqlens[b] ..
 *   cu_seqlens[b+1]-1 of a capacity of total_tokens rows; rows at or beyond
 *   cu_seqlens[B] are capacity padding: never read as keys or queries.  Owned
 *   per-query outputs of padding rows are zero-filled (idx rows: -1).
 * - Compressed rows (section 4): sample b owns n_b = floor(L_b / ratio) rows
 *   starting at cu_cmp[b]; the incomplete tail of L_b mod ratio tokens owns
 *   none.  Query at local position p sees compressed rows j < floor((p+1)/ratio)
 *   of its own sample (a group is visible once its last token is) and the raw
 *   window rows max(0, p-window+1) .. p of its own sample.
 * - Overwrite vs accumulate: per-query outputs overwrite (x_cmp, scores, idx,
 *   out, lse, dq, kl, loss, dqI, dw).  Gradients of shared rows ACCUMULATE (+=,
 *   caller zeroes): dx, dkv_cmp, dkv, dsink, dkI_cmp.
 * - Errors: argument validation runs on the host before anything is enqueued
 *   and returns a negative csa_status_t with nothing launched.  Device metadata
 *   (cu_seqlens non-decreasing, cu_seqlens[B] <= total_tokens, every L_b <=
 *   max_seqlen) is the caller's contract, checkable on request with
 *   csa_validate_metadata; cu_cmp, wherever a call takes it, must hold what
 *   csa_cmp_seqlens wrote for the same cu_seqlens (its values index the
 *   compressed buffers unchecked).  A failed launch returns CSA_ERR_LAUNCH.
 * - Calls that share an output buffer must not overlap in time.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 7

typedef int32_t csa_status_t;
enum {
  CSA_OK = 0,
  CSA_ERR_NULL = -1,        /* a required pointer is NULL */
  CSA_ERR_ARG = -2,         /* an argument is out of range */
  CSA_ERR_UNSUPPORTED = -3, /* dtype / shape combination not built */
  CSA_ERR_WORKSPACE = -4,   /* workspace missing or too small */
  CSA_ERR_LAUNCH = -5       /* a kernel launch failed (hipGetLastError) */
};

typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2 } csa_dtype_t;

/* Candidate sets of the main attention (section 2 phase table). */
typedef enum {
  CSA_SPARSE = 0, /* top-k selected compressed rows (idx) + window           */
  CSA_DENSE = 1,  /* every visible compressed row + window: HCA, dense mode  */
  CSA_WINDOW = 2  /* window only (the ratio-0 layer); kv_cmp unused          */
} csa_mode_t;

/* Candidate set C_t of the indexer KL teacher (section 2 phase table, section 3). */
typedef enum {
  CSA_TEACHER_NONE = 0,
  CSA_TEACHER_SELECTED = 1, /* C_t = selected set (sparse-loss phase)            */
  CSA_TEACHER_DENSE = 2     /* C_t = all visible compressed rows (warm-up phase) */
} csa_teacher_t;

typedef struct csa_params {
  int32_t batch;        /* B, number of packed samples (>= 0)                        */
  int32_t total_tokens; /* T, capacity rows of every per-token tensor (>= 0)          */
  int32_t max_seqlen;   /* host upper bound on every L_b; n_cap = max_seqlen / ratio  */
  int32_t ratio;        /* r, tokens per compressed row (1 .. 4096; 4 CSA, 128 HCA)   */
  int32_t window;       /* W >= 1, raw rows in the local window (query included)      */
  int32_t topk;         /* k >= 1, selected compressed rows per query (CSA_SPARSE)    */
  int32_t topk_cap;     /* k_cap >= k, multiple of 64: row width of idx               */
  int32_t heads;        /* H query heads sharing one KV row                           */
  int32_t head_dim;     /* D, width of q and of the shared K=V row                    */
  int32_t idx_heads;    /* H_I indexer heads                                          */
  int32_t idx_dim;      /* d_I indexer query / key width                              */
  float scale;          /* softmax scale of the main logits (usually 1/sqrt(D))       */
  int32_t mode;         /* csa_mode_t                                                 */
  int32_t teacher;      /* csa_teacher_t                                              */
  int32_t dtype;        /* csa_dtype_t of q, kv, kv_cmp, out, dO, dq: F32 or BF16     */
  int32_t idx_dtype;    /* csa_dtype_t of qI and kI_cmp: F32, BF16 or FP8_E4M3        */
  int32_t rope_dim;     /* rotary band of the output rotation (csa_sparse_attn_fwd      */
                        /* out_rot): 0 none, else a multiple of 8 <= head_dim          */
  float rope_theta;     /* rotary base (> 0) when rope_dim > 0                         */
} csa_params_t;

/* Workspace-using operations, for csa_workspace_size. */
enum { CSA_OP_ATTN_FWD = 1, CSA_OP_ATTN_BWD = 2, CSA_OP_INDEXER_KL = 3,
       CSA_OP_INDEXER_KL_CACHED = 4 /* csa_indexer_kl with teacher_logits */ };

int csa_abi_version(void);
const char* csa_status_string(csa_status_t status);

/* Bytes of device workspace `op` needs for these params (0 is possible).  For
 * CSA_OP_ATTN_BWD this is the preferred size; the call also accepts any smaller
 * workspace down to csa_workspace_size_min (it then processes the queries in more chunks:
 * the same results up to the order of floating-point sums, more launches). */
csa_status_t csa_workspace_size(const csa_params_t* p, int32_t op, size_t* bytes);

/* The smallest workspace `op` accepts for these params (equal to csa_workspace_size for
 * every op but CSA_OP_ATTN_BWD). */
csa_status_t csa_workspace_size_min(const csa_params_t* p, int32_t op, size_t* bytes);

/* cu_cmp[0] = 0, cu_cmp[b+1] = cu_cmp[b] + floor((cu_seqlens[b+1]-cu_seqlens[b]) / ratio).
 * (section 4, the n_b^cmp equation).  cu_seqlens, cu_cmp: int32 [batch+1]. */
csa_status_t csa_cmp_seqlens(const int32_t* cu_seqlens, int32_t batch, int32_t ratio,
                             int32_t* cu_cmp, hipStream_t stream);

/* Optional device-side check of the metadata contract.  Writes one int32 to
 * status_dev: 0 = valid, 1 = cu_seqlens[0] != 0, 2 = decreasing, 3 = cu_seqlens[B] >
 * total_tokens, 4 = a sample longer than max_seqlen. */
csa_status_t csa_validate_metadata(const csa_params_t* p, const int32_t* cu_seqlens,
                                   int32_t* status_dev, hipStream_t stream);

/* Ratio-r compressor (section 4; mean-pool reading of the compressor):
 *   x_cmp[cu_cmp[b] + j, :] = (1/r) sum_{u<r} x[cu_seqlens[b] + j*r + u, :],  j < n_b.
 * x: [total_tokens, dim] of `dtype` (CSA_F32 or CSA_BF16); x_cmp: [>= total_tokens/r, dim]
 * same dtype, fp32 accumulation, rows beyond cu_cmp[B] untouched.  dim % 8 == 0. */
csa_status_t csa_compress(const csa_params_t* p, int32_t dtype, const void* x, int32_t dim,
                          const int32_t* cu_seqlens, const int32_t* cu_cmp, void* x_cmp,
                          hipStream_t stream);

/* Adjoint of csa_compress: dx[cu_seqlens[b] + j*r + u, :] += d_x_cmp[cu_cmp[b] + j, :] / r.
 * d_x_cmp, dx: fp32.  Tail and padding rows of dx are untouched. */
csa_status_t csa_compress_bwd(const csa_params_t* p, const float* d_x_cmp, int32_t dim,
                              const int32_t* cu_seqlens, const int32_t* cu_cmp, float* dx,
                              hipStream_t stream);

/* Learned-score compressor (sections 4, 5.1, 8.2, 9).  For group j of sample b (complete
 * groups only, as csa_compress), per channel d:
 *   x_cmp[cu_cmp[b] + j, d] = sum_u w_u[d] x[t_u, d],  w[d] = softmax_u(score[t_u, d] + bias[p_u, d]),
 * over the source tokens t_u: the group's own r tokens at positions r .. 2r-1 and, when
 * overlap != 0 and j > 0, its left neighbour's r tokens at positions 0 .. r-1 (compression
 * restarts at each sample, so group 0 has no left neighbour); overlap == 0: the own tokens at
 * positions 0 .. r-1.  x, score: [total_tokens, dim] of dtype (CSA_F32 / CSA_BF16); bias:
 * fp32 [(overlap ? 2 : 1) * ratio, dim]; x_cmp: [Tc, dim] of dtype, overwritten.  dim % 8 ==
 * 0, dim <= 2048; overlap is 0 or 1 (CSA_ERR_ARG otherwise).  Reads p->batch,
 * total_tokens, ratio. */
csa_status_t csa_compress_learned(const csa_params_t* p, int32_t dtype, const void* x,
                                  const void* score, const float* bias, int32_t dim,
                                  int32_t overlap, const int32_t* cu_seqlens,
                                  const int32_t* cu_cmp, void* x_cmp, hipStream_t stream);

/* Adjoint of csa_compress_learned for d_x_cmp (fp32 [Tc, dim]): with c the compressed row,
 *   dx[t_u] += w_u d,  dscore[t_u] += w_u (x[t_u] - c) d,  dbias[p_u] += w_u (x[t_u] - c) d
 * (per channel, d = d_x_cmp of the group), summed over every group that reads the token.
 * dx, dscore: fp32 [total_tokens, dim]; dbias: fp32 like bias; all ACCUMULATE (caller
 * zeroes).  Tail and padding rows are untouched.  Same operands and limits as the forward. */
csa_status_t csa_compress_learned_bwd(const csa_params_t* p, int32_t dtype, const void* x,
                                      const void* score, const float* bias,
                                      const float* d_x_cmp, int32_t dim, int32_t overlap,
                                      const int32_t* cu_seqlens, const int32_t* cu_cmp,
                                      float* dx, float* dscore, float* dbias,
                                      hipStream_t stream);

/* Per-row OCP e4m3 quantization (FP8 indexer, section 9): scale = max|row| / 448 in
 * fp32 (1 for an all-zero row); code = e4m3(x / scale), fp32 division, round to nearest
 * even, saturating at +-448.  x: [rows, row_len] of x_dtype (CSA_F32 / CSA_BF16);
 * codes: uint8 [rows, row_len]; row_scale: fp32 [rows].  row_len % 8 == 0, <= 1024. */
csa_status_t csa_quantize_fp8(const void* x, int32_t x_dtype, int64_t rows, int32_t row_len,
                              uint8_t* codes, float* row_scale, hipStream_t stream);

/* Lightning-indexer logits (section 3 logits i_{t,j}):
 *   scores[t, j] = sum_h w[t,h] * max(0, qI[t,h,:] . kI_cmp[cu_cmp[b]+j, :]),
 * for j < n_vis(p) = floor((p+1)/r).  Entries j >= n_vis(p) and rows of padding are NOT
 * written.  qI: [T, H_I, d_I], kI_cmp: [Tc, d_I] of idx_dtype; for CSA_FP8_E4M3 they are
 * e4m3 codes with fp32 scales qI_scale [T, H_I] and kI_scale [Tc] (else both NULL).
 * w: fp32 [T, H_I].  scores: fp32 [T, ld_scores], ld_scores >= max_seqlen / r.
 * A -0 result is stored as +0. */
csa_status_t csa_index_scores(const csa_params_t* p, const void* qI, const float* qI_scale,
                              const float* w, const void* kI_cmp, const float* kI_scale,
                              const int32_t* cu_seqlens, const int32_t* cu_cmp, float* scores,
                              int64_t ld_scores, hipStream_t stream);

/* Top-k selection + local-to-global lowering (sections 3, 8.1, 8.2): row t gets the
 * n_sel = min(k, n_vis(p)) visible j with the largest scores[t, j] (ties: smaller j
 * wins; -0 == +0), written as the global compressed rows cu_cmp[b] + j in ascending
 * order in idx[t, 0 .. n_sel), then -1 up to topk_cap.  scores: fp32 [T, ld_scores]
 * (only the visible prefix of each row is read); idx: int32 [T, topk_cap]. */
csa_status_t csa_topk_select(const csa_params_t* p, const float* scores, int64_t ld_scores,
                             const int32_t* cu_seqlens, const int32_t* cu_cmp, int32_t* idx,
                             hipStream_t stream);

/* Indexer scores and top-k selection in one pass (section 3 logits and selection; section
 * 8.2 names score/top-k fusion as open work): the same idx as csa_index_scores followed by
 * csa_topk_select on the same operands, without the full [T, ld_scores] score matrix
 * making a round trip through HBM.  scores_mode: 0 = scores not written (scores may be
 * NULL); 1 = scores[t, j] written for the selected j only (what a selected-set indexer loss
 * reads); 2 = written for every visible j.  Other entries of scores are untouched.
 * Supported for idx_heads = 64, idx_dim = 128 (bf16 or fp8 indexer) and max_seqlen / ratio
 * <= 32768 (the row limit of csa_topk_select); else CSA_ERR_UNSUPPORTED (use the two calls).
 * idx: int32 [T, topk_cap]. */
csa_status_t csa_index_topk(const csa_params_t* p, const void* qI, const float* qI_scale,
                            const float* w, const void* kI_cmp, const float* kI_scale,
                            const int32_t* cu_seqlens, const int32_t* cu_cmp, int32_t scores_mode,
                            float* scores, int64_t ld_scores, int32_t* idx, hipStream_t stream);

/* Sparse attention forward (sections 2 and 8.2).  Candidates of query t: the compressed
 * rows idx[t, 0 .. first -1) (CSA_SPARSE; entries outside the query's visible range are
 * ignored), or all visible compressed rows (CSA_DENSE), or none (CSA_WINDOW); plus the
 * window rows of kv.  One row is both key and value (MQA).  For each head h:
 *   l_x = scale q[t,h].row_x,  lse[t,h] = log([e^{sink_h}] + sum_x e^{l_x}),
 *   out[t,h] = sum_x e^{l_x - lse[t,h]} row_x.
 * Optionally also lse_cmp[t,h] = log(sum over the compressed candidates only of e^{l_x})
 * (no window, no sink; -inf for a query without compressed candidates): with a
 * selected-set teacher this is the teacher's per-head normalizer, which csa_indexer_kl
 * then need not recompute (section 8.2, teacher score recomputation).
 * Optionally also the compressed-candidate logits themselves, t_logits[t, h, c] = l_x of
 * compressed slot c (slot order of the idx row for CSA_SPARSE, visible order for
 * CSA_DENSE) for c < the query's compressed count; other entries are unspecified.  They
 * are the teacher logits csa_indexer_kl needs when its candidate set equals the
 * attention's (selected teacher with CSA_SPARSE, dense teacher with CSA_DENSE).
 * q, out: [T, H, D]; kv_cmp: [Tc, D]; kv: [T, D] (dtype); idx: int32 [T, topk_cap] or NULL
 * unless CSA_SPARSE; sink: fp32 [H] or NULL; lse, lse_cmp: fp32 [T, H] (natural log);
 * t_logits: fp32 [T, H, csa_teacher_logits_stride(p)].  lse_cmp and t_logits may be NULL.
 * out_rot: NULL, or [T, H, D] (dtype) receiving out inverse-rotated at the query's local
 * position (csa_rope with inverse = 1 on out, p->rope_dim and p->rope_theta; zero rows for
 * padding), written by the same pass where the kernel has a rotating epilogue.  out itself
 * stays unrotated: it is the saved output the backward consumes (section 10, the
 * inverse-rotation aliasing contract; section 12, invariant 5), so out_rot must not alias it
 * (CSA_ERR_ARG, as is out_rot with rope_dim 0). */
csa_status_t csa_sparse_attn_fwd(const csa_params_t* p, const void* q, const void* kv_cmp,
                                 const void* kv, const int32_t* idx, const float* sink,
                                 const int32_t* cu_seqlens, const int32_t* cu_cmp, void* out,
                                 void* out_rot, float* lse, float* lse_cmp, float* t_logits,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Rotary position embedding (section 4: positions restart at every packed sample, for the
 * main and the indexer operands; section 12, invariant 2: the positional mode is per layer
 * and per compressed coordinate system).  Row `row` of sample b, row_offsets[b] <= row <
 * row_offsets[b+1], has position pos = row - row_offsets[b]: pass cu_seqlens for token rows
 * (q, kv, qI, the output) and cu_cmp for compressed rows (kv_cmp, kI_cmp).  In every head
 * the interleaved channel pairs (2i, 2i+1) of the last rope_dim channels are rotated by
 * pos * theta^(-2i / rope_dim) radians (angle formed in fp64), by minus that when inverse = 1;
 * rows at or beyond row_offsets[batch] are copied unchanged.  A rotation's adjoint is its
 * inverse, so the same call maps gradients back (inverse = 1 on the gradient of a rotated
 * operand; inverse = 0 on the gradient of an inverse-rotated output).
 * x, y: [rows, heads, dim] of dtype F32 or BF16.  y == x rotates in place and touches only
 * the rotary channels; otherwise y receives every channel and must not overlap x.
 * dim and rope_dim: multiples of 8, 8 <= rope_dim <= dim; theta > 0; rows < 2^31 (x and y
 * may be NULL when rows is 0). */
csa_status_t csa_rope(int32_t dtype, const void* x, void* y, int64_t rows, int32_t heads,
                      int32_t dim, int32_t rope_dim, float theta, int32_t inverse,
                      int32_t batch, const int32_t* row_offsets, hipStream_t stream);

/* Row stride (in elements) of the t_logits cache: the compressed-slot capacity (topk_cap
 * for CSA_SPARSE, max_seqlen / ratio for CSA_DENSE) rounded up to a multiple of 64; 0 for
 * CSA_WINDOW or invalid parameters. */
int64_t csa_teacher_logits_stride(const csa_params_t* p);

/* Sparse attention backward (section 8.2: consumes saved O, LSE, dO; no dense matrix).
 * With P = e^{l_x - lse}, dP = dO.row_x, Dt = dO.O, dS = P (dP - Dt):
 *   dq[t,h] = scale sum_x dS row_x                       (overwrite, dtype)
 *   d row_x += scale dS q[t,h] + P dO[t,h]               (dkv_cmp / dkv, fp32, +=)
 *   dsink[h] += -e^{sink_h - lse[t,h]} Dt                (fp32, +=; NULL if no sink)
 * Same candidate sets and layouts as the forward; dkv receives window-row gradients only
 * (add the compressor's share with csa_compress_bwd).  ws: ws_bytes bytes, at least
 * csa_workspace_size_min and best csa_workspace_size (CSA_ERR_WORKSPACE below the minimum). */
csa_status_t csa_sparse_attn_bwd(const csa_params_t* p, const void* q, const void* kv_cmp,
                                 const void* kv, const int32_t* idx, const float* sink,
                                 const int32_t* cu_seqlens, const int32_t* cu_cmp,
                                 const void* out, const float* lse, const void* d_out, void* dq,
                                 float* dkv_cmp, float* dkv, float* dsink, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* csa_sparse_attn_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same operands, results and errors as csa_sparse_attn_bwd; its workspace is a static
 * 256 MiB array of the library on each GPU (held from the library's first use on that GPU
 * until the process ends), so the queries are processed in as many chunks as that needs.
 * CSA_ERR_WORKSPACE when even the smallest chunk (csa_workspace_size_min) exceeds 256 MiB.
 * The call allocates nothing.  All calls on one GPU share that GPU's array: calls that
 * overlap in time on one GPU (two streams, two host threads) race and must be serialized
 * by the caller.  Nothing carries over from one call to the next. */
csa_status_t csa_sparse_attn_bwd_noalloc(const csa_params_t* p, const void* q,
                                         const void* kv_cmp, const void* kv, const int32_t* idx,
                                         const float* sink, const int32_t* cu_seqlens,
                                         const int32_t* cu_cmp, const void* out, const float* lse,
                                         const void* d_out, void* dq, float* dkv_cmp, float* dkv,
                                         float* dsink, hipStream_t stream);

/* Indexer KL auxiliary loss with its eager backward (section 3 loss equation; section
 * 8.2: the indexer-loss backward runs inside the forward, the loss scale is applied by
 * the caller through grad_scale).  C_t = idx row (CSA_TEACHER_SELECTED) or all visible
 * rows (CSA_TEACHER_DENSE).  Teacher (detached): P_t = mean_h softmax_{C_t}(scale q[t,h] .
 * kv_cmp[j]); student: Q_t = softmax_{C_t}(scores[t, j]).
 *   kl[t] = sum_{j in C_t} P_t (log P_t - log Q_t)  (0 if C_t is empty);  loss[0] = sum_t kl[t]
 *   g = grad_scale (Q_t - P_t), z = qI[t,h] . kI[j]:
 *   dw[t,h] = sum_j g relu(z); dqI[t,h,:] = sum_j g w[t,h] 1[z>0] kI[j,:]     (overwrite)
 *   dkI_cmp[j,:] += sum_{t,h} g w[t,h] 1[z>0] qI[t,h,:]                        (+=)
 * For CSA_FP8_E4M3 the gradients are taken with respect to the dequantized operands.
 * teacher_lse: NULL, or (CSA_TEACHER_SELECTED only) the lse_cmp [T, H] that
 * csa_sparse_attn_fwd returned for the same q, kv_cmp and idx; it is then used as the
 * teacher's per-head log-normalizer instead of being recomputed.
 * teacher_logits: NULL, or the t_logits cache csa_sparse_attn_fwd wrote for the same
 * q, kv_cmp, idx and params (allowed for CSA_TEACHER_SELECTED with CSA_SPARSE and for
 * CSA_TEACHER_DENSE with CSA_DENSE; else CSA_ERR_ARG).  Teacher logits may then be read
 * from it instead of recomputed; results agree up to floating-point rounding.  With a
 * cache the workspace must be csa_workspace_size(p, CSA_OP_INDEXER_KL_CACHED) bytes.
 * scores: fp32 [T, ld_scores] as csa_index_scores writes them (only the entries of C_t are
 * read), or NULL for CSA_TEACHER_DENSE with a bf16 main path (H = 64, D = 512) and a 64 x 128
 * bf16 / fp8 indexer: the student scores are then formed inside the call, a chunk of queries
 * at a time, in the workspace (the same values csa_index_scores would write), so no
 * [T, max_seqlen / ratio] score matrix need exist (CSA_ERR_NULL for other shapes).
 * kl: fp32 [T]; loss: fp32 [1]; dqI: fp32 [T, H_I, d_I]; dw: fp32 [T, H_I];
 * dkI_cmp: fp32 [Tc, d_I].  dqI, dw and dkI_cmp all NULL => loss only.
 * Supported for heads <= 64 teacher heads (CSA_ERR_UNSUPPORTED beyond). */
csa_status_t csa_indexer_kl(const csa_params_t* p, const void* q, const void* kv_cmp,
                            const float* scores, int64_t ld_scores, const int32_t* idx,
                            const float* teacher_lse, const float* teacher_logits,
                            const void* qI, const float* qI_scale, const float* w,
                            const void* kI_cmp, const float* kI_scale,
                            const int32_t* cu_seqlens, const int32_t* cu_cmp, float grad_scale,
                            float* kl, float* loss, float* dqI, float* dw, float* dkI_cmp,
                            void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
