"""Plain, slow, fp64 CPU oracle for the CSA/HCA attention layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; it is used by tests/, by the smoke check and by the benchmark's CPU
baseline leg.  It shares no code, tables or helpers with the HIP library.

Every function restates, in numpy float64, what one step of the method
computes, following the page "DeepSeek-V4 Attention Training Systems"
(v4-attn-notes, training-systems chapter):

  * section 2 (phase table): dense mode attends every completed compressed
    entry plus the local window; the sparse phases attend the top-k selected
    compressed entries plus the window; HCA (ratio 128) has no indexer.
  * section 3 (the indexer loss equation): L_I is the sum over queries of the
    KL divergence from the softmax of teacher logits to the softmax of indexer
    logits, both restricted to a candidate set C_t (all visible compressed
    entries for the dense-loss warm-up, the selected set for sparse loss); the
    teacher side is detached.
  * section 4 (varlen, the n_b^cmp equation): sample b of a packed batch yields
    floor(L_b / r) compressed entries; the incomplete tail yields none; every
    step restarts at a sample boundary.
  * section 8.2 (training kernel map): attention returns its output and
    log-sum-exp; the backward consumes the saved output, LSE and dO and returns
    query, KV and sink gradients.

Readings taken where the page leaves a step open (each restated where used):
  R1 compressor = mean of the r rows of each completed non-overlapping block;
  R3 compressed row j is visible to local position p once its last token
     j*r + r - 1 <= p, i.e. n_vis(p) = floor((p + 1) / r);
  R4 window = raw rows max(0, p - W + 1) .. p of the query's own sample,
     not de-duplicated against compressed rows;
  R5 one shared 512-wide row serves as key and value (MQA);
  R6 optional sink logit s_h adds e^{s_h} to the softmax denominator only;
  R7 indexer score I[t, j] = sum_h w[t, h] * relu(qI[t, h] . kI[j]);
  R8 top-k ties go to the lower j, and -0 equals +0;
  R9 teacher P_t = mean over heads of the per-head softmax over C_t of the
     main-attention logits (window and sink excluded);
  R11 loss = sum over real rows of KL_t, KL_t = 0 for an empty C_t;
  R13 fp8 = OCP e4m3 (max 448), one scale per row = max|row| / 448 computed in
     float32, codes = round-to-nearest-even(x / scale) saturated to +-448;
  R20 learned compressor = per channel, softmax over the group's source tokens of
     (score row + positional parameter) weighting the value rows; ratio-4 groups
     overlap their left neighbour (8 source tokens), ratio-128 groups do not; the
     normalization is the softmax's own (no further learned scaling);
  R22 RoPE = rotation of the interleaved channel pairs of the last rope_dim channels by
     position * theta^(-2i / rope_dim); positions restart per sample, token rows use the
     local token position, compressed rows their index within the sample; the inverse
     (on the attention output, at the query's position) rotates by the opposite angle;
  R23 a layer chain "with storage rounding" holds every intermediate a step hands to the
     next in the precision it is stored in: compressed main and indexer rows and rotated
     operands in the layer's main / indexer dtype (the section 5.5 storage estimate counts
     the compressed state in BF16), index scores and the log-sum-exp in FP32 (section 9:
     score, softmax and KL math in FP32), the saved output in the main dtype; each step
     itself is still evaluated in float64 on those rounded values.
"""
import numpy as np

F8_MAX = 448.0


# ---------------------------------------------------------------------------
# storage precision of intermediates (reading R23)
# ---------------------------------------------------------------------------
def round_bf16(x):
    """x rounded to bfloat16 (float32 first, then round-to-nearest-even on the upper 16
    bits of the float32 encoding), returned as float64.  Inputs are finite."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def store(x, dtype):
    """x as a buffer of `dtype` holds it: "f32" -> float32, "bf16" -> bfloat16; the fp8
    indexer path keeps its unquantized rows in bfloat16.  Infinities pass through."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype in ("bf16", "fp8"):
        fin = np.isfinite(x)
        out = x.copy()
        out[fin] = round_bf16(x[fin])
        return out
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# metadata (section 4)
# ---------------------------------------------------------------------------
def sample_table(cu_seqlens):
    """Starts and lengths of the packed samples delimited by cu_seqlens."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0:
        raise ValueError("cu_seqlens must be a 1-D prefix array starting at 0")
    lens = cu[1:] - cu[:-1]
    if np.any(lens < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    return cu[:-1].copy(), lens


def cmp_seqlens(cu_seqlens, ratio):
    """Prefix offsets of the compressed rows: sample b owns floor(L_b / r) rows."""
    if ratio < 1:
        raise ValueError("ratio must be >= 1")
    _, lens = sample_table(cu_seqlens)
    out = np.zeros(lens.size + 1, dtype=np.int64)
    out[1:] = np.cumsum(lens // ratio)
    return out


def token_positions(cu_seqlens, total_tokens):
    """Per packed row t: its sample b and local position p (-1 for padding rows)."""
    starts, lens = sample_table(cu_seqlens)
    if int(starts[-1] + lens[-1] if lens.size else 0) > total_tokens:
        raise ValueError("samples exceed the packed capacity")
    b = np.full(total_tokens, -1, dtype=np.int64)
    p = np.full(total_tokens, -1, dtype=np.int64)
    for i, (s, L) in enumerate(zip(starts, lens)):
        b[s:s + L] = i
        p[s:s + L] = np.arange(L)
    return b, p


def n_visible(p, ratio):
    """Number of completed compressed rows visible at local position p (R3)."""
    return (np.asarray(p) + 1) // ratio


def window_rows(start, p, window):
    """Global raw rows of the local window of the query at local position p (R4)."""
    lo = max(0, p - window + 1)
    return start + np.arange(lo, p + 1)


# ---------------------------------------------------------------------------
# compressor (section 4; reading R1)
# ---------------------------------------------------------------------------
def compress(x, cu_seqlens, ratio):
    """x_cmp[cu_cmp[b] + j] = mean of rows s_b + j*r .. s_b + j*r + r - 1, j < floor(L_b/r)."""
    x = np.asarray(x, dtype=np.float64)
    starts, lens = sample_table(cu_seqlens)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    out = np.zeros((int(cu_cmp[-1]),) + x.shape[1:], dtype=np.float64)
    for b, (s, L) in enumerate(zip(starts, lens)):
        for j in range(int(L) // ratio):
            block = x[s + j * ratio: s + (j + 1) * ratio]
            out[cu_cmp[b] + j] = block.sum(axis=0) / ratio
    return out


def compress_bwd(d_cmp, cu_seqlens, ratio, total_tokens):
    """Adjoint of compress: each of the r source rows receives d_cmp / r; tails get 0."""
    d_cmp = np.asarray(d_cmp, dtype=np.float64)
    starts, lens = sample_table(cu_seqlens)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    dx = np.zeros((total_tokens,) + d_cmp.shape[1:], dtype=np.float64)
    for b, (s, L) in enumerate(zip(starts, lens)):
        for j in range(int(L) // ratio):
            dx[s + j * ratio: s + (j + 1) * ratio] += d_cmp[cu_cmp[b] + j] / ratio
    return dx


# ---------------------------------------------------------------------------
# learned-score compressor (reading R20)
# ---------------------------------------------------------------------------
def _learned_groups(cu_seqlens, ratio, overlap):
    """(output row, source token rows, positions in the positional parameter) per group.

    Group j of sample b owns tokens s_b + j r .. s_b + j r + r - 1 (complete groups only,
    section 4).  Overlapping groups (ratio-4 CSA, section 5.1: 8 source tokens) also read
    the left neighbour's r tokens, at positions 0 .. r-1, their own at r .. 2r-1; group 0
    of a sample has no left neighbour (compression restarts at the sample boundary).
    Non-overlapping groups (HCA) read their own tokens at positions 0 .. r-1."""
    starts, lens = sample_table(cu_seqlens)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    out = []
    for b, (s, L) in enumerate(zip(starts, lens)):
        for j in range(int(L) // ratio):
            own = np.arange(s + j * ratio, s + (j + 1) * ratio)
            if overlap and j > 0:
                toks = np.arange(s + (j - 1) * ratio, s + (j + 1) * ratio)
                pos = np.arange(2 * ratio)
            elif overlap:
                toks, pos = own, np.arange(ratio, 2 * ratio)
            else:
                toks, pos = own, np.arange(ratio)
            out.append((int(cu_cmp[b]) + j, toks, pos))
    return out


def compress_learned(x, score, bias, cu_seqlens, ratio, overlap):
    """x_cmp[row, d] = sum_u w[u, d] x[t_u, d],  w[:, d] = softmax_u(score[t_u, d] + bias[p_u, d])
    over the group's source tokens t_u at positions p_u (see _learned_groups): a per-channel
    learned-score reduction with an fp32 positional parameter (sections 8.2 and 9), reset
    per sample.  bias: [2r, dim] if overlap else [r, dim].  Returns [Tc, dim]."""
    x = np.asarray(x, dtype=np.float64)
    score = np.asarray(score, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    groups = _learned_groups(cu_seqlens, ratio, overlap)
    Tc = int(cmp_seqlens(cu_seqlens, ratio)[-1])
    out = np.zeros((Tc, x.shape[1]))
    for row, toks, pos in groups:
        z = score[toks] + bias[pos]
        z = z - z.max(axis=0, keepdims=True)
        w = np.exp(z)
        w /= w.sum(axis=0, keepdims=True)
        out[row] = (w * x[toks]).sum(axis=0)
    return out


def compress_learned_bwd(x, score, bias, d_cmp, cu_seqlens, ratio, overlap, total_tokens):
    """Adjoint of compress_learned: with c = sum_u w_u x_u per channel,
      dx[t_u] += w_u dc,  dscore[t_u] += w_u (x_u - c) dc,  dbias[p_u] += w_u (x_u - c) dc
    summed over every group reading the token (two for overlapping groups).  Returns
    (dx [T, dim], dscore [T, dim], dbias like bias)."""
    x = np.asarray(x, dtype=np.float64)
    score = np.asarray(score, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    d_cmp = np.asarray(d_cmp, dtype=np.float64)
    dx = np.zeros((total_tokens, x.shape[1]))
    ds = np.zeros((total_tokens, x.shape[1]))
    db = np.zeros_like(bias)
    for row, toks, pos in _learned_groups(cu_seqlens, ratio, overlap):
        z = score[toks] + bias[pos]
        z = z - z.max(axis=0, keepdims=True)
        w = np.exp(z)
        w /= w.sum(axis=0, keepdims=True)
        c = (w * x[toks]).sum(axis=0)
        dz = w * (x[toks] - c) * d_cmp[row]
        dx[toks] += w * d_cmp[row]
        ds[toks] += dz
        db[pos] += dz
    return dx, ds, db


# ---------------------------------------------------------------------------
# rotary position embedding (reading R22)
# ---------------------------------------------------------------------------
def rope_positions(cu_seqlens, n_rows, ratio=None):
    """Position of each row, restarting at every packed sample (section 4): the local token
    position p for token rows (ratio None), or the compressed index j within the sample for
    compressed rows (ratio given: the compressed coordinate system, section 12).  -1 marks
    rows outside every sample."""
    if ratio is None:
        _, pp = token_positions(cu_seqlens, n_rows)
        return np.where(pp >= 0, pp, -1)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    pos = np.full(n_rows, -1, dtype=np.int64)
    for b in range(len(cu_cmp) - 1):
        pos[cu_cmp[b]:cu_cmp[b + 1]] = np.arange(cu_cmp[b + 1] - cu_cmp[b])
    return pos


def rope(x, pos, rope_dim, theta, inverse=False):
    """Rotate the interleaved channel pairs (2i, 2i+1) of the last rope_dim channels of each
    row by pos * theta^(-2i / rope_dim) (by minus that for the inverse); rows with pos < 0
    are returned unchanged.  x: [rows, ..., dim]; pos: [rows]."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    dim = x.shape[-1]
    i = np.arange(rope_dim // 2)
    inv_freq = float(theta) ** (-2.0 * i / rope_dim)
    for r, p in enumerate(np.asarray(pos)):
        if p < 0:
            continue
        ang = (-1.0 if inverse else 1.0) * p * inv_freq
        c, s = np.cos(ang), np.sin(ang)
        a = x[r, ..., dim - rope_dim::2]
        b_ = x[r, ..., dim - rope_dim + 1::2]
        out[r, ..., dim - rope_dim::2] = a * c - b_ * s
        out[r, ..., dim - rope_dim + 1::2] = a * s + b_ * c
    return out


# ---------------------------------------------------------------------------
# fp8 e4m3 encoding (reading R13)
# ---------------------------------------------------------------------------
def _e4m3_table():
    """All non-negative finite OCP e4m3 values, indexed by their 7-bit code."""
    vals = np.zeros(127, dtype=np.float64)
    for code in range(127):          # 0x7f is NaN
        e = code >> 3
        m = code & 7
        if e == 0:
            vals[code] = (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = _e4m3_table()


def e4m3_encode(v):
    """Round float values to the nearest e4m3 code (ties to the even code), saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    flat = v.reshape(-1)
    codes = np.zeros(flat.size, dtype=np.uint8)
    even = (np.arange(127) % 2 == 0)
    step = 1 << 15
    for lo in range(0, flat.size, step):
        x = flat[lo:lo + step]
        mag = np.minimum(np.abs(x), F8_MAX)
        # nearest representable magnitude by exhaustive comparison with the table
        diff = np.abs(mag[:, None] - _E4M3[None, :])
        cand = diff == diff.min(axis=1, keepdims=True)
        # among two equally near codes (a tie) keep the even one
        pick_even = cand & even
        choose = np.where(pick_even.any(axis=1, keepdims=True), pick_even, cand)
        code = np.argmax(choose, axis=1).astype(np.uint8)
        sign = np.signbit(x).astype(np.uint8)      # the sign is kept, also on zero
        codes[lo:lo + step] = code | (sign << 7)
    return codes.reshape(v.shape)


def e4m3_decode(code):
    code = np.asarray(code, dtype=np.uint8)
    mag = _E4M3[code & 0x7F]
    return np.where(code & 0x80, -mag, mag)


def quantize_fp8(x):
    """Per-row e4m3 quantization: scale = max|row| / 448 in float32 (1 for a zero row);
    code = e4m3(float32(x) / scale) with the division in float32."""
    x = np.asarray(x, dtype=np.float32)
    rows = x.reshape(-1, x.shape[-1])
    amax = np.abs(rows).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(F8_MAX), np.float32(1.0)).astype(np.float32)
    scaled = (rows / scale[:, None]).astype(np.float32)
    codes = e4m3_encode(scaled)
    return codes.reshape(x.shape), scale.reshape(x.shape[:-1])


def dequantize_fp8(codes, scale):
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


# ---------------------------------------------------------------------------
# lightning indexer scores (section 3 logits i_{t,j}; reading R7)
# ---------------------------------------------------------------------------
def index_scores(qI, w, kI_cmp, cu_seqlens, ratio, n_cap, rows=None):
    """I[t, j] = sum_h w[t,h] * max(0, qI[t,h] . kI_cmp[cu_cmp[b] + j]) for j < n_vis(p).

    Columns j >= n_vis(p) hold -inf (not visible).  Returns [len(rows), n_cap]."""
    qI = np.asarray(qI, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    kI_cmp = np.asarray(kI_cmp, dtype=np.float64)
    T = qI.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    bb, pp = token_positions(cu_seqlens, T)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    out = np.full((rows.size, n_cap), -np.inf)
    for i, t in enumerate(rows):
        if bb[t] < 0:
            continue
        nv = int(n_visible(pp[t], ratio))
        if nv == 0:
            continue
        c0 = cu_cmp[bb[t]]
        z = qI[t] @ kI_cmp[c0:c0 + nv].T          # [H_I, nv]
        out[i, :nv] = w[t] @ np.maximum(z, 0.0) + 0.0   # + 0.0 turns -0 into +0
    return out


# ---------------------------------------------------------------------------
# top-k selection + lowering to global compressed rows (reading R8)
# ---------------------------------------------------------------------------
def topk_select(scores, cu_seqlens, ratio, k, k_cap, total_tokens, rows=None):
    """Per query: the min(k, n_vis) visible j with the largest score, ties to smaller j,
    written as global rows cu_cmp[b] + j and padded with -1 to k_cap.

    `scores[i]` is the score row of query rows[i] (any float dtype; compared as given)."""
    rows = np.arange(total_tokens) if rows is None else np.asarray(rows)
    bb, pp = token_positions(cu_seqlens, total_tokens)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    idx = np.full((rows.size, k_cap), -1, dtype=np.int64)
    for i, t in enumerate(rows):
        if bb[t] < 0:
            continue
        nv = int(n_visible(pp[t], ratio))
        m = min(k, nv)
        if m == 0:
            continue
        s = np.asarray(scores[i][:nv], dtype=np.float64) + 0.0
        j = np.arange(nv)
        order = np.lexsort((j, -s))       # primary: score descending; then j ascending
        idx[i, :m] = cu_cmp[bb[t]] + order[:m]
    return idx


# ---------------------------------------------------------------------------
# sparse attention (section 2 candidate sets; section 8.2 outputs; R4-R6)
# ---------------------------------------------------------------------------
def attn_candidates(t, bb, pp, starts, cu_cmp, ratio, window, idx_row):
    """Compressed rows (global indices into kv_cmp) and window rows (into kv) of query t.

    idx_row None => dense mode / HCA: every visible compressed row."""
    b, p = bb[t], pp[t]
    if idx_row is None:
        cmp_rows = cu_cmp[b] + np.arange(int(n_visible(p, ratio)))
    else:
        r = np.asarray(idx_row)
        cmp_rows = r[r >= 0]
    return cmp_rows.astype(np.int64), window_rows(starts[b], p, window)


def sparse_attn_fwd(q, kv_cmp, kv, idx, sink, cu_seqlens, ratio, window, scale, rows=None):
    """O[t,h] = sum_x softmax_x(scale q[t,h].row_x) row_x over compressed + window candidates;
    LSE[t,h] = log([e^{sink_h}] + sum_x e^{scale q[t,h].row_x}).

    idx: [len(rows), k_cap] global compressed rows (-1 = padding) or None (all visible).
    Returns O [len(rows), H, D], LSE [len(rows), H]."""
    q = np.asarray(q, dtype=np.float64)
    kv_cmp = np.asarray(kv_cmp, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    T, H, D = q.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    bb, pp = token_positions(cu_seqlens, T)
    starts, _ = sample_table(cu_seqlens)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    O = np.zeros((rows.size, H, D))
    LSE = np.zeros((rows.size, H))
    for i, t in enumerate(rows):
        if bb[t] < 0:
            continue
        cr, wr = attn_candidates(t, bb, pp, starts, cu_cmp, ratio, window,
                                 None if idx is None else idx[i])
        X = np.concatenate([kv_cmp[cr], kv[wr]], axis=0)      # [N, D]
        logits = scale * (q[t] @ X.T)                          # [H, N]
        full = logits if sink is None else np.concatenate(
            [logits, np.asarray(sink, dtype=np.float64)[:, None]], axis=1)
        m = full.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(full - m).sum(axis=1))
        P = np.exp(logits - lse[:, None])
        O[i] = P @ X
        LSE[i] = lse
    return O, LSE


def compressed_logits(q, kv_cmp, idx, cu_seqlens, ratio, scale, rows=None):
    """Main-attention logits of the compressed candidates of each query, in the order the
    attention takes them: l[h, c] = scale q[t,h] . kv_cmp[row_c], row_c the c-th valid entry
    of the idx row (idx given) or the c-th visible compressed row (idx None).  With C_t equal
    to that set these are the indexer teacher's logits (section 3 with R9).
    Returns a list (one entry per row) of [H, n_c] arrays."""
    q = np.asarray(q, dtype=np.float64)
    kv_cmp = np.asarray(kv_cmp, dtype=np.float64)
    T = q.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    bb, pp = token_positions(cu_seqlens, T)
    starts, _ = sample_table(cu_seqlens)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    out = []
    for i, t in enumerate(rows):
        if bb[t] < 0:
            out.append(np.zeros((q.shape[1], 0)))
            continue
        cr, _ = attn_candidates(t, bb, pp, starts, cu_cmp, ratio, 0,
                                None if idx is None else idx[i])
        out.append(scale * (q[t] @ kv_cmp[cr].T))
    return out


def sparse_attn_bwd(q, kv_cmp, kv, idx, sink, cu_seqlens, ratio, window, scale, O, LSE, dO,
                    rows=None):
    """Gradients of the sparse attention given the saved O, LSE and the incoming dO.

    With P = e^{scale q.x - LSE}, dP = dO.x, Dt = dO.O and dS = P (dP - Dt):
      dq = scale sum_x dS x;  d x += scale dS q + P dO  (K = V, so key and value
      contributions add);  dsink_h = -sum_t e^{sink_h - LSE} Dt.
    O/LSE/dO are indexed like rows.  Returns dq [len(rows),H,D], dkv_cmp [Tc,D],
    dkv [T,D], dsink [H] (zeros if sink is None).  dkv_cmp/dkv/dsink sum over `rows`."""
    q = np.asarray(q, dtype=np.float64)
    kv_cmp = np.asarray(kv_cmp, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    LSE = np.asarray(LSE, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    T, H, D = q.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    bb, pp = token_positions(cu_seqlens, T)
    starts, _ = sample_table(cu_seqlens)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    dq = np.zeros((rows.size, H, D))
    dkv_cmp = np.zeros_like(kv_cmp)
    dkv = np.zeros((kv.shape[0], D))
    dsink = np.zeros(H)
    for i, t in enumerate(rows):
        if bb[t] < 0:
            continue
        cr, wr = attn_candidates(t, bb, pp, starts, cu_cmp, ratio, window,
                                 None if idx is None else idx[i])
        X = np.concatenate([kv_cmp[cr], kv[wr]], axis=0)       # [N, D]
        P = np.exp(scale * (q[t] @ X.T) - LSE[i][:, None])     # [H, N]
        dP = dO[i] @ X.T                                        # [H, N]
        Dt = (dO[i] * O[i]).sum(axis=1)                         # [H]
        dS = P * (dP - Dt[:, None])
        dq[i] = scale * (dS @ X)
        dX = scale * (dS.T @ q[t]) + P.T @ dO[i]                # [N, D]
        np.add.at(dkv_cmp, cr, dX[:cr.size])
        np.add.at(dkv, wr, dX[cr.size:])
        if sink is not None:
            dsink += -np.exp(np.asarray(sink, dtype=np.float64) - LSE[i]) * Dt
    return dq, dkv_cmp, dkv, dsink


# ---------------------------------------------------------------------------
# indexer KL auxiliary loss and its (eager) backward (section 3; section 8.2)
# ---------------------------------------------------------------------------
def _teacher_set(t, bb, pp, cu_cmp, ratio, teacher, idx_row):
    """Local compressed indices j of C_t: the selected set or every visible entry."""
    nv = int(n_visible(pp[t], ratio))
    if teacher == "dense" or idx_row is None:
        return np.arange(nv)
    r = np.asarray(idx_row)
    return (r[r >= 0] - cu_cmp[bb[t]]).astype(np.int64)


def indexer_kl(q, kv_cmp, scores, idx, qI, w, kI_cmp, cu_seqlens, ratio, scale, teacher,
               grad_scale=1.0, rows=None, relu_eps=None):
    """KL_t = sum_{j in C_t} P_t[j] (log P_t[j] - log Q_t[j]) with
      P_t = (1/H) sum_h softmax_{C_t}(scale q[t,h] . kv_cmp[j])   (detached teacher, R9)
      Q_t = softmax_{C_t}(I[t, j])                                 (student = indexer logits)
    and its gradients, scaled by grad_scale, into the indexer operands only:
      g_tj = grad_scale (Q_t[j] - P_t[j]),  z = qI[t,h] . kI[j]
      dw[t,h] = sum_j g relu(z);  dqI[t,h] = sum_j g w[t,h] 1[z>0] kI[j];
      dkI_cmp[j] += sum_{t,h} g w[t,h] 1[z>0] qI[t,h].
    scores[i] is the score row of query rows[i]; idx[i] its selected global rows
    (teacher "selected").  Returns kl [len(rows)], loss, dqI, dw, dkI_cmp [Tc, d_I].

    The ReLU mask 1[z>0] is a floating-point decision: with relu_eps given, every z with
    |z| <= relu_eps * sum_d |qI[t,h,d] kI[j,d]| counts as undecided, and a sixth value
    (dqI, dw, dkI_cmp bounds) gives, per output element, the sum of |change| that flipping
    the mask of all undecided z would cause."""
    q = np.asarray(q, dtype=np.float64)
    kv_cmp = np.asarray(kv_cmp, dtype=np.float64)
    qI = np.asarray(qI, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    kI_cmp = np.asarray(kI_cmp, dtype=np.float64)
    T, H, D = q.shape
    HI, dI = qI.shape[1], qI.shape[2]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    bb, pp = token_positions(cu_seqlens, T)
    cu_cmp = cmp_seqlens(cu_seqlens, ratio)
    kl = np.zeros(rows.size)
    dqI = np.zeros((rows.size, HI, dI))
    dw = np.zeros((rows.size, HI))
    dkI = np.zeros_like(kI_cmp)
    if relu_eps is not None:
        b_dqI, b_dw, b_dkI = np.zeros_like(dqI), np.zeros_like(dw), np.zeros_like(dkI)
    for i, t in enumerate(rows):
        if bb[t] < 0:
            continue
        C = _teacher_set(t, bb, pp, cu_cmp, ratio, teacher, None if idx is None else idx[i])
        if C.size == 0:
            continue
        g_rows = cu_cmp[bb[t]] + C
        a = scale * (q[t] @ kv_cmp[g_rows].T)                 # [H, |C|] teacher logits
        a = a - a.max(axis=1, keepdims=True)
        Ph = np.exp(a)
        Ph /= Ph.sum(axis=1, keepdims=True)
        P = Ph.mean(axis=0)                                   # head-averaged teacher
        s = np.asarray(scores[i], dtype=np.float64)[C]
        logQ = s - (s.max() + np.log(np.exp(s - s.max()).sum()))
        Q = np.exp(logQ)
        pos = P > 0
        kl[i] = float((P[pos] * (np.log(P[pos]) - logQ[pos])).sum())
        g = grad_scale * (Q - P)                              # dKL/dI scaled
        K = kI_cmp[g_rows]                                    # [|C|, d_I]
        z = qI[t] @ K.T                                       # [H_I, |C|]
        act = (z > 0).astype(np.float64)
        dw[i] = np.maximum(z, 0.0) @ g
        E = act * (w[t][:, None] * g[None, :])                # [H_I, |C|] = dI/dz * g
        dqI[i] = E @ K
        np.add.at(dkI, g_rows, E.T @ qI[t])
        if relu_eps is not None:
            open_ = np.abs(z) <= relu_eps * (np.abs(qI[t]) @ np.abs(K).T)
            if open_.any():
                flip = open_ * np.abs(w[t][:, None] * g[None, :])   # |E| a flip adds or removes
                b_dqI[i] = flip @ np.abs(K)
                b_dw[i] = (open_ * np.abs(z)) @ np.abs(g)
                np.add.at(b_dkI, g_rows, flip.T @ np.abs(qI[t]))
    if relu_eps is not None:
        return kl, float(kl.sum()), dqI, dw, dkI, (b_dqI, b_dw, b_dkI)
    return kl, float(kl.sum()), dqI, dw, dkI


# ---------------------------------------------------------------------------
# one whole layer step (all steps chained, as the HIP path chains them)
# ---------------------------------------------------------------------------
def layer_step(inp, cfg, rows=None, backward=None, grad_scale=1.0, stored=False):
    """Chain the steps on host arrays.  inp holds float64 arrays q, kv, [qI, kI_tok, w],
    [dO], [sink], cu_seqlens; cfg supplies ratio, window, topk, topk_cap, scale, mode,
    teacher, idx_dtype and optionally rope_dim / rope_theta.  Per-query outputs are returned
    for `rows`; the shared-row gradients (dkv, dkI_tok) are complete only when rows covers
    every query.

    With rope_dim > 0 (reading R22) the layer rotates q, qI and the window rows of kv at
    their token positions and the compressed rows of kv and kI at their compressed
    positions, all restarting per sample (section 4); O stays unrotated (it is what the
    attention backward consumes) and O_rot, the inverse rotation of O at the query's
    position, is the layer output, so dO is taken as the gradient of O_rot.  The gradients
    returned are those of the unrotated inputs (a rotation's adjoint is its inverse).

    stored=True (reading R23) rounds every intermediate handed from one step to the next
    to the precision it is stored in: compressed and rotated rows to the main / indexer
    dtype, scores and LSE to float32, the output saved for the backward to the main dtype.
    stored=False is the all-float64 chain."""
    cu = inp["cu_seqlens"]
    q = inp["q"]
    T = q.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    backward = cfg.backward if backward is None else backward
    r = cfg.ratio
    rd = int(getattr(cfg, "rope_dim", 0) or 0)
    theta = float(getattr(cfg, "rope_theta", 0.0) or 0.0)
    res = {}
    ident = lambda x: x                                                      # noqa: E731
    st_main = (lambda x: store(x, cfg.dtype)) if stored else ident          # noqa: E731
    st_idx = (lambda x: store(x, cfg.idx_dtype)) if stored else ident       # noqa: E731
    st_f32 = (lambda x: store(x, "f32")) if stored else ident               # noqa: E731
    kv = inp["kv"]
    kv_cmp = st_main(compress(kv, cu, r))
    res["kv_cmp"] = kv_cmp
    if rd:
        tpos = rope_positions(cu, T)
        cpos = rope_positions(cu, kv_cmp.shape[0], ratio=r)
        rot = lambda x, pos: rope(x, pos, rd, theta)                        # noqa: E731
        unrot = lambda x, pos: rope(x, pos, rd, theta, inverse=True)        # noqa: E731
        q_in = q
        q = np.zeros(q_in.shape)             # untouched pages stay unallocated
        q[rows] = st_main(rot(q_in[rows], tpos[rows]))
        kv = st_main(rot(kv, tpos))
        kv_cmp = st_main(rot(kv_cmp, cpos))
    idx = None
    if cfg.mode == "window":          # ratio-0 layer: no compressed candidates at all
        idx = np.full((rows.size, 1), -1, dtype=np.int64)
    if cfg.has_indexer and cfg.mode == "sparse":
        kI_cmp = st_idx(compress(inp["kI_tok"], cu, r))
        qI = inp["qI"]
        if rd:
            qI_in = qI
            qI = np.zeros(qI_in.shape)
            qI[rows] = st_idx(rot(qI_in[rows], tpos[rows]))
            kI_cmp = st_idx(rot(kI_cmp, cpos))
        if cfg.idx_dtype == "fp8":
            qI_full = qI
            qI = np.zeros(qI.shape)          # untouched pages stay unallocated
            qc, qs = quantize_fp8(qI_full[rows].astype(np.float32))
            qI[rows] = dequantize_fp8(qc, qs)
            kc, ks = quantize_fp8(kI_cmp.astype(np.float32))
            kI_cmp = dequantize_fp8(kc, ks)
        res["kI_cmp"] = kI_cmp
        n_cap = int(inp["max_seqlen"]) // r
        scores = st_f32(index_scores(qI, inp["w"], kI_cmp, cu, r, n_cap, rows=rows))
        res["scores"] = scores
        idx = topk_select(scores, cu, r, cfg.topk, cfg.topk_cap, T, rows=rows)
        res["idx"] = idx
    O, LSE = sparse_attn_fwd(q, kv_cmp, kv, idx, inp.get("sink"), cu, r, cfg.window,
                             cfg.scale, rows=rows)
    res["O"], res["LSE"] = O, LSE
    if rd:
        res["O_rot"] = unrot(O, tpos[rows])
    if cfg.has_indexer and cfg.mode == "sparse" and cfg.teacher != "none":
        kl, loss, dqI, dw, dkI = indexer_kl(q, kv_cmp, res["scores"], idx, qI, inp["w"], kI_cmp,
                                            cu, r, cfg.scale, cfg.teacher, grad_scale, rows=rows)
        if rd:
            dqI = unrot(dqI, tpos[rows])
            dkI = unrot(dkI, cpos)
        res.update(kl=kl, loss=loss, dqI=dqI, dw=dw, dkI_cmp=dkI)
        res["dkI_tok"] = compress_bwd(dkI, cu, r, T)
    if backward:
        dO = inp["dO"][rows]
        if rd:
            dO = st_main(rot(dO, tpos[rows]))   # gradient of O from that of O_rot
        dq, dkv_cmp, dkv_win, dsink = sparse_attn_bwd(
            q, kv_cmp, kv, idx, inp.get("sink"), cu, r, cfg.window, cfg.scale,
            st_main(O), st_f32(LSE), dO, rows=rows)
        if rd:
            dq = unrot(dq, tpos[rows])
            dkv_cmp = unrot(dkv_cmp, cpos)
            dkv_win = unrot(dkv_win, tpos)
        res.update(dq=dq, dkv_cmp=dkv_cmp, dkv_win=dkv_win, dsink=dsink)
        res["dkv"] = dkv_win + compress_bwd(dkv_cmp, cu, r, T)
    return res
