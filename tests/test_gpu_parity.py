"""GPU parity: every C-ABI call against the fp64 oracle on the same seeded inputs.

Step isolation: each GPU step is fed the ORACLE's upstream outputs (rounded once to the
device dtype), and the oracle step is evaluated on exactly those rounded values, so a
top-k near-tie cannot hide or fake an error downstream.  An end-to-end layer step is
compared as well.  Tolerances: fp32 max-abs 1e-5; bf16 max-abs / max|ref| <= 2e-2;
top-k sets bit-exact on identical fp32 score bytes; KL loss relative 1e-3.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synth import configs, inputs as synth_inputs
from tests import gpu_support as G

pytestmark = pytest.mark.gpu

# Reduced instances keep the layer shapes of the workloads (heads, widths, ratio, window,
# dtypes, phase) at sizes the oracle finishes in seconds, with several tiles, ragged
# tails and capacity padding.
CASES = {
    "tiny_f32_L256": ("tiny_csa_f32_L256", {}),
    "tiny_f32_packed_tails_pad": ("tiny_csa_f32_L256", dict(lengths=(37, 100, 3, 64),
                                                            total_tokens=220)),
    "tiny_f32_sink_selected": ("tiny_csa_f32_L256", dict(sink=True, teacher="selected",
                                                         lengths=(130, 90), total_tokens=224)),
    "tiny_f32_window_only": ("tiny_csa_f32_L256", dict(mode="window", teacher="none",
                                                       idx_heads=0, lengths=(70, 129),
                                                       total_tokens=200)),
    "tiny_f32_dense_mode": ("tiny_csa_f32_L256", dict(mode="dense", teacher="none",
                                                      idx_heads=0, lengths=(77, 150),
                                                      total_tokens=230)),
    "csa_bf16_thd_small": ("thd64k_csa_bf16", dict(lengths=(301, 515, 1027), total_tokens=1856,
                                                   topk=64, topk_cap=64, draw=None)),
    "hca_bf16_thd_small": ("thd64k_hca_bf16", dict(lengths=(1024, 700, 300),
                                                   total_tokens=2048)),
    "window_bf16_thd_small": ("thd64k_window_bf16", dict(lengths=(301, 515, 1027),
                                                         total_tokens=1856, draw=None)),
    "sink_bf16_thd_small": ("thd64k_csa_sink_bf16", dict(lengths=(301, 515, 1027),
                                                         total_tokens=1856, topk=64,
                                                         topk_cap=64, draw=None)),
    "fp8_warmup_small": ("csa128k_warmup_fp8", dict(lengths=(1500,), total_tokens=1536,
                                                    topk=64, topk_cap=64)),
    "rope_bf16_thd_small": ("thd64k_csa_rope_bf16", dict(lengths=(301, 515, 1027),
                                                         total_tokens=1856, topk=64,
                                                         topk_cap=64, draw=None)),
    "rope_f32_selected_pad": ("tiny_csa_f32_L256", dict(teacher="selected", lengths=(130, 90),
                                                        total_tokens=224, rope_dim=16,
                                                        rope_theta=500.0)),
    # the generic (non-MFMA) kernels at the widest rows and the most heads the ABI accepts
    "f32_wide_rows_generic": ("tiny_csa_f32_L256", dict(heads=64, head_dim=512, idx_heads=4,
                                                        idx_dim=64, lengths=(40, 25),
                                                        total_tokens=72, window=16, topk=8,
                                                        teacher="selected")),
    # (the indexer loss takes at most 64 teacher heads: selection only here)
    "bf16_128_heads_generic": ("thd64k_csa_bf16", dict(heads=128, head_dim=256,
                                                       lengths=(100, 77), total_tokens=192,
                                                       topk=64, topk_cap=64, draw=None,
                                                       teacher="none")),
    "rope_fp8_warmup_small": ("csa128k_warmup_fp8", dict(lengths=(1500,), total_tokens=1536,
                                                         topk=64, topk_cap=64, rope_dim=64)),
    # top-k well below the visible rows (2600 // 4 = 650 > 6 x 64): the backward stages one
    # row gradient per attended pair and sums them per row, instead of the key-major products
    "csa_bf16_thd_staged": ("thd64k_csa_bf16", dict(lengths=(301, 515, 2600),
                                                    total_tokens=3456, topk=32, topk_cap=64,
                                                    draw=None)),
    # dense mode at ratio 4 (every visible compressed row + the window, no indexer) on the
    # matrix-core kernels
    "dense_bf16_thd_small": ("thd64k_csa_bf16", dict(mode="dense", teacher="none", idx_heads=0,
                                                     lengths=(301, 515, 1027),
                                                     total_tokens=1856, draw=None)),
}

# Sharp-softmax variants of the matrix-core cases: every tensor at unit variance (logits of
# order 1 instead of 1e-3, so P depends on the logits), and "rescale" cases whose raw kv rows
# in the second half of each sample are scaled by 8 (exact in bf16): a query there meets
# logits in a later candidate block that exceed the first block's maximum by far more than
# 2^8, so the lazily moved running maximum of the attention forward and of the dense teacher
# normalizer is moved after the first block (checked below from the oracle's logits).
SHARP = {
    "csa_bf16_thd_unit": ("csa_bf16_thd_small", dict(strength=True)),
    "csa_bf16_thd_rescale": ("csa_bf16_thd_small", dict(strength=True, kv_boost=8.0)),
    "sink_bf16_thd_unit": ("sink_bf16_thd_small", dict(strength=True)),
    "hca_bf16_thd_rescale": ("hca_bf16_thd_small", dict(strength=True, kv_boost=8.0)),
    "window_bf16_thd_rescale": ("window_bf16_thd_small", dict(strength=True, kv_boost=8.0)),
    "dense_bf16_thd_rescale": ("dense_bf16_thd_small", dict(strength=True, kv_boost=8.0)),
    "fp8_warmup_unit": ("fp8_warmup_small", dict(strength=True)),
    "fp8_warmup_rescale": ("fp8_warmup_small", dict(strength=True, kv_boost=8.0)),
}
for _n, (_b, _x) in SHARP.items():
    CASES[_n] = CASES[_b] + (_x,)

# the one fp32 case held to the summed-terms bound (64 heads x 512-wide rows)
F32_SUM = {"f32_wide_rows_generic"}

_CACHE = {}


def _kind(name, kind):
    return "f32_sum" if (kind == "f32" and name in F32_SUM) else kind


def _boost_kv(host, factor):
    """Scale the raw kv rows of the second half of every sample by `factor` (in place)."""
    cu = host["cu_seqlens"]
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        host["kv"][s + (e - s) // 2:e] *= factor


def _case(name):
    if name in _CACHE:
        return _CACHE[name]
    base, over = CASES[name][:2]
    extra = CASES[name][2] if len(CASES[name]) > 2 else {}
    w = configs.workload(base, **over)
    host = synth_inputs.make_inputs(w, variant=0, strength=extra.get("strength", False))
    if extra.get("kv_boost"):
        _boost_kv(host, extra["kv_boost"])
    h64 = {k: synth_inputs.to_f64(v) for k, v in host.items() if isinstance(v, torch.Tensor)}
    h64["cu_seqlens"] = host["cu_seqlens"]
    h64["max_seqlen"] = host["max_seqlen"]
    _CACHE[name] = (w, host, h64)
    return _CACHE[name]


def _rescale_margin(w, q, kv_cmp, kv, idx, cu, rows, first_block=64):
    """Largest growth, in log2 units, of a (query, head)'s logit maximum past the maximum of
    its first `first_block` candidates, in the order the forward takes them (compressed
    rows in idx order, then the window)."""
    bb, pp = O.token_positions(cu, q.shape[0])
    starts, _ = O.sample_table(cu)
    cu_cmp = O.cmp_seqlens(cu, w.ratio)
    best = 0.0
    for i, t in enumerate(rows):
        cr, wr = O.attn_candidates(t, bb, pp, starts, cu_cmp, w.ratio, w.window,
                                   None if idx is None else idx[i])
        # compressed candidates padded to whole 64-row blocks before the window rows
        X = np.concatenate([kv_cmp[cr], kv[wr]], axis=0)
        if X.shape[0] == 0:
            continue
        lg = w.scale * (q[t] @ X.T) / np.log(2.0)
        n_first = min(first_block, cr.size) if cr.size else min(first_block, wr.size)
        best = max(best, float((lg.max(axis=1) - lg[:, :n_first].max(axis=1)).max()))
    return best


def _layer(w, host, backward=True):
    from long_context_compressed_amd.pipeline import CsaLayer, LayerConfig
    return CsaLayer(LayerConfig.of(w), len(host["lengths"]), w.total_tokens, host["max_seqlen"],
                    backward=backward)


def _cu(host):
    return torch.tensor(host["cu_seqlens"], dtype=torch.int32, device="cuda")


def _announce(name, step):
    print(f"[gpu] case={name} step={step}", flush=True)


def _wl(n):
    return configs.workload(CASES[n][0], **CASES[n][1])


def _idx_cases():
    return [n for n in CASES if _wl(n).has_indexer and _wl(n).mode == "sparse"]


def _kl_cases():
    return [n for n in _idx_cases() if _wl(n).teacher != "none"]


# ------------------------------------------------------------------------- metadata
@pytest.mark.parametrize("name", list(CASES))
def test_metadata_and_compress(name):
    from long_context_compressed_amd import binding as B
    w, host, h64 = _case(name)
    _announce(name, "compress")
    L = _layer(w, host, backward=False)
    cu = _cu(host)
    L.metadata(cu)
    ref_cmp = O.cmp_seqlens(host["cu_seqlens"], w.ratio)
    assert L.cu_cmp.cpu().numpy().tolist() == ref_cmp.tolist()
    Tc = int(ref_cmp[-1])
    L.kv_cmp.fill_(7.0)
    kv = host["kv"].cuda()
    B.csa_compress(L.p, kv, cu, L.cu_cmp, L.kv_cmp)
    torch.cuda.synchronize()
    G.check("kv_cmp", G.back(L.kv_cmp[:Tc]), O.compress(h64["kv"], host["cu_seqlens"], w.ratio),
            _kind(name, w.dtype))
    assert torch.all(L.kv_cmp[Tc:] == 7.0), "rows beyond cu_cmp[B] were written"
    # validate_metadata accepts the packed batch
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    B.csa_validate_metadata(L.p, cu, st)
    assert int(st.item()) == 0


@pytest.mark.parametrize("name", ["tiny_f32_packed_tails_pad", "hca_bf16_thd_small",
                                  "csa_bf16_thd_small"])
def test_compress_bwd(name):
    from long_context_compressed_amd import binding as B
    w, host, h64 = _case(name)
    _announce(name, "compress_bwd")
    L = _layer(w, host, backward=True)
    cu = _cu(host)
    L.metadata(cu)
    Tc = int(O.cmp_seqlens(host["cu_seqlens"], w.ratio)[-1])
    rng = np.random.default_rng(101)
    d = rng.standard_normal((Tc, w.head_dim))
    base = rng.standard_normal((w.total_tokens, w.head_dim))
    dx = G.dev(base, torch.float32)
    B.csa_compress_bwd(L.p, G.dev(d, torch.float32), cu, L.cu_cmp, dx)
    ref = base.astype(np.float32).astype(np.float64) + O.compress_bwd(
        G.rounded(d, torch.float32), host["cu_seqlens"], w.ratio, w.total_tokens)
    torch.cuda.synchronize()
    G.check("dx", G.back(dx), ref, "f32")


LEARNED_CASES = {
    # name: (lengths, capacity T, dim, ratio, overlap, dtype)
    "f32_overlap_tails_pad": ((13, 9, 4, 3, 20), 56, 64, 4, True, "f32"),
    "f32_nonoverlap": ((13, 9, 4, 3, 20), 56, 64, 4, False, "f32"),
    "bf16_csa_thd_kv": ((301, 515, 1027), 1856, 512, 4, True, "bf16"),
    "bf16_csa_thd_indexer_key": ((301, 515, 1027), 1856, 128, 4, True, "bf16"),
    "bf16_hca": ((1024, 700, 300), 2048, 512, 128, False, "bf16"),
    "bf16_csa_64k_full": (None, 65536, 512, 4, True, "bf16"),
}


@pytest.mark.parametrize("name", list(LEARNED_CASES))
def test_compress_learned_fwd_bwd(name):
    """Learned-score compressor and its adjoint against the oracle on every row; capacity
    padding rows hold NaN (never read)."""
    from long_context_compressed_amd import binding as B
    lens, T, dim, r, overlap, dt_name = LEARNED_CASES[name]
    _announce(name, "compress_learned")
    if lens is None:   # the 64K THD batch's lengths
        lens = tuple(synth_inputs.draw_lengths(configs.workload("thd64k_csa_bf16")))
    rng = np.random.default_rng(53)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = int(cu[-1])
    dt = G.torch_dtype(dt_name)
    x = G.rounded(rng.standard_normal((T, dim)), dt)
    sc = G.rounded(rng.standard_normal((T, dim)) * 2.0, dt)
    x[n:] = np.nan
    sc[n:] = np.nan
    span = (2 if overlap else 1) * r
    bias = rng.standard_normal((span, dim)).astype(np.float32).astype(np.float64)
    p = B.make_params(batch=len(lens), total_tokens=T, max_seqlen=max(lens), ratio=r, window=1,
                      topk=1, topk_cap=64, heads=1, head_dim=8, idx_heads=0, idx_dim=0,
                      scale=1.0, mode=B.CSA_DENSE, teacher=B.CSA_TEACHER_NONE,
                      dtype=B.CSA_BF16 if dt_name == "bf16" else B.CSA_F32, idx_dtype=B.CSA_BF16)
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    cmp_d = torch.empty(len(lens) + 1, dtype=torch.int32, device="cuda")
    B.csa_cmp_seqlens(cu_d, len(lens), r, cmp_d)
    xd, sd = G.dev(x, dt), G.dev(sc, dt)
    bd = torch.from_numpy(bias.astype(np.float32)).cuda()
    Tc = int(O.cmp_seqlens(cu, r)[-1])
    out = torch.full((max(Tc, 1), dim), float("nan"), dtype=dt, device="cuda")
    B.csa_compress_learned(p, xd, sd, bd, overlap, cu_d, cmp_d, out)
    ref = O.compress_learned(x[:n], sc[:n], bias, cu, r, overlap)
    torch.cuda.synchronize()
    G.check("x_cmp", G.back(out)[:Tc], ref, dt_name)
    # adjoint, accumulated onto nonzero starting values
    dc = rng.standard_normal((max(Tc, 1), dim)).astype(np.float32)
    dx0 = rng.standard_normal((T, dim)).astype(np.float32)
    dx = torch.from_numpy(dx0).cuda()
    ds = torch.from_numpy(dx0[::-1].copy()).cuda()
    db = torch.ones((span, dim), dtype=torch.float32, device="cuda")
    B.csa_compress_learned_bwd(p, xd, sd, bd, torch.from_numpy(dc).cuda(), overlap, cu_d, cmp_d,
                               dx, ds, db)
    rdx, rds, rdb = O.compress_learned_bwd(x[:n], sc[:n], bias, dc[:Tc], cu, r, overlap, n)
    torch.cuda.synchronize()
    G.check("dx", G.back(dx)[:n] - dx0[:n], rdx, dt_name)
    G.check("dscore", G.back(ds)[:n] - dx0[::-1][:n], rds, dt_name)
    G.check("dbias", G.back(db) - 1.0, rdb, dt_name)
    assert np.array_equal(G.back(dx)[n:], dx0[n:].astype(np.float64)), "padding rows of dx written"


@pytest.mark.parametrize("row_len,dtype", [(128, torch.bfloat16), (8, torch.bfloat16),
                                           (64, torch.float32), (200, torch.bfloat16),
                                           (512, torch.float32), (1024, torch.bfloat16)])
def test_quantize_fp8_bit_exact(row_len, dtype):
    # row lengths span every lane-group width of the kernel (8 .. 64 lanes per row, one or
    # two 8-element chunks per lane); 777 rows leave a ragged last workgroup
    from long_context_compressed_amd import binding as B
    rng = np.random.default_rng(5)
    x = rng.standard_normal((777, row_len)) * np.logspace(-4, 3, 777)[:, None]
    x[3] = 0.0
    x[4, :5] = [1e-30, -0.0, 0.0, 448.0, -1e-9]
    xb = torch.tensor(x).to(dtype)
    print(f"[gpu] case=quantize step=fp8 row_len={row_len} dtype={dtype}", flush=True)
    codes = torch.empty(777, row_len, dtype=torch.uint8, device="cuda")
    scale = torch.empty(777, dtype=torch.float32, device="cuda")
    B.csa_quantize_fp8(xb.cuda(), codes, scale)
    ref_codes, ref_scale = O.quantize_fp8(xb.to(torch.float32).numpy())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scale.cpu().numpy(), ref_scale)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)


# ------------------------------------------------------------------------- indexer
def _indexer_inputs(w, host, h64):
    """Oracle-side compressed indexer keys, rounded to the device's indexer dtype, and the
    values (dequantized for fp8) that the oracle evaluates on."""
    cu = host["cu_seqlens"]
    kI = O.compress(h64["kI_tok"], cu, w.ratio)
    if w.idx_dtype == "fp8":
        kI_b = G.rounded(kI, torch.bfloat16)
        kc, ks = O.quantize_fp8(kI_b.astype(np.float32))
        qc, qs = O.quantize_fp8(h64["qI"].astype(np.float32))
        dev = dict(qI=torch.from_numpy(qc).cuda(), qI_scale=torch.from_numpy(qs).cuda(),
                   kI=torch.from_numpy(kc).cuda(), kI_scale=torch.from_numpy(ks).cuda())
        return dev, O.dequantize_fp8(qc, qs), O.dequantize_fp8(kc, ks)
    dt = G.torch_dtype(w.idx_dtype)
    kI_r = G.rounded(kI, dt)
    dev = dict(qI=host["qI"].cuda(), qI_scale=None, kI=G.dev(kI_r, dt), kI_scale=None)
    return dev, h64["qI"], kI_r


@pytest.mark.parametrize("name", _idx_cases())
def test_index_scores(name):
    from long_context_compressed_amd import binding as B
    w, host, h64 = _case(name)
    _announce(name, "index_scores")
    L = _layer(w, host, backward=False)
    cu = _cu(host)
    L.metadata(cu)
    d, qI64, kI64 = _indexer_inputs(w, host, h64)
    L.scores.fill_(12345.0)
    B.csa_index_scores(L.p, d["qI"], d["qI_scale"], host["w"].cuda(), d["kI"], d["kI_scale"], cu,
                       L.cu_cmp, L.scores)
    ref = O.index_scores(qI64, h64["w"], kI64, host["cu_seqlens"], w.ratio, L.n_cap)
    torch.cuda.synchronize()
    got = G.back(L.scores)
    vis = np.isfinite(ref)
    assert np.all(got[~vis] == 12345.0), "non-visible score entries were written"
    G.check("scores(visible)", got[vis], ref[vis], "f32" if w.idx_dtype == "f32" else "bf16")
    assert not np.any(np.signbit(got[vis]) & (got[vis] == 0)), "-0 stored"


@pytest.mark.parametrize("name", _idx_cases())
def test_topk_bit_exact_on_same_fp32_scores(name):
    from long_context_compressed_amd import binding as B
    w, host, h64 = _case(name)
    _announce(name, "topk")
    L = _layer(w, host, backward=False)
    cu = _cu(host)
    L.metadata(cu)
    _, qI64, kI64 = _indexer_inputs(w, host, h64)
    ref_scores = O.index_scores(qI64, h64["w"], kI64, host["cu_seqlens"], w.ratio, L.n_cap)
    s32 = np.where(np.isfinite(ref_scores), ref_scores, 0.0).astype(np.float32)
    B.csa_topk_select(L.p, torch.from_numpy(s32).cuda(), cu, L.cu_cmp, L.idx)
    ref = O.topk_select(s32, host["cu_seqlens"], w.ratio, w.topk, w.topk_cap, w.total_tokens)
    torch.cuda.synchronize()
    got = L.idx.cpu().numpy()
    for t in range(w.total_tokens):
        g, r = got[t], ref[t]
        n = int((r >= 0).sum())
        assert np.all(g[n:] == -1), t
        assert np.array_equal(g[:n], np.sort(r[:n])), t     # sets equal; GPU rows ascending


def test_topk_ties_signed_zero_and_long_rows():
    """Heavy ties, -0/+0 and rows longer than one register pass of the kernel."""
    from long_context_compressed_amd import binding as B
    for L_len, k, kcap, seed in ((9000, 700, 704, 1), (40000, 2048, 2048, 2), (3000, 5, 64, 3)):
        print(f"[gpu] case=topk_ties L={L_len} k={k}", flush=True)
        rng = np.random.default_rng(seed)
        T = 256
        n_cap = L_len // 4
        # 256 query rows taken from the end of one long sample (large n_vis)
        cu = np.array([0, L_len], dtype=np.int64)
        rows = np.arange(L_len - T, L_len)
        s = (np.round(rng.standard_normal((T, n_cap)) * 3) / 4).astype(np.float32)
        s[s == 0] = -0.0
        s[::2, ::3] = 0.0
        p = B.make_params(batch=1, total_tokens=L_len, max_seqlen=L_len, ratio=4, window=1,
                          topk=k, topk_cap=kcap, heads=1, head_dim=8, idx_heads=1, idx_dim=8,
                          scale=1.0, mode=0, teacher=0, dtype=1, idx_dtype=1)
        full = torch.zeros(L_len, n_cap, dtype=torch.float32)
        full[rows] = torch.from_numpy(s)
        idx = torch.empty(L_len, kcap, dtype=torch.int32, device="cuda")
        cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
        cmp_d = torch.empty(2, dtype=torch.int32, device="cuda")
        B.csa_cmp_seqlens(cu_d, 1, 4, cmp_d)
        B.csa_topk_select(p, full.cuda(), cu_d, cmp_d, idx)
        ref = O.topk_select(s, cu, 4, k, kcap, L_len, rows=rows)
        got = idx.cpu().numpy()[rows]
        for i in range(T):
            n = int((ref[i] >= 0).sum())
            assert np.array_equal(got[i][:n], np.sort(ref[i][:n])), (L_len, i)
            assert np.all(got[i][n:] == -1)


def test_topk_mixed_rows_with_padding():
    """Rows of up to 4096 visible scores (the wave kernel's largest register footprint) over
    several samples and capacity padding: light rows (every visible row selected), heavy rows
    with and without ties, and padding rows (-1) in one launch, bit-exact against the oracle
    on every fifth row and on the rows around the end of the packed batch."""
    from long_context_compressed_amd import binding as B
    lengths, pad, k, kcap = (9001, 301, 11999, 7), 499, 1024, 1088
    print(f"[gpu] case=topk_mixed_rows lengths={lengths} pad={pad} k={k}", flush=True)
    rng = np.random.default_rng(11)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1]) + pad
    max_len = max(lengths)
    n_cap = max_len // 4
    s = rng.standard_normal((T, n_cap)).astype(np.float32)
    s[1::7, ::5] = 0.0                       # ties in some rows
    p = B.make_params(batch=len(lengths), total_tokens=T, max_seqlen=max_len, ratio=4,
                      window=1, topk=k, topk_cap=kcap, heads=1, head_dim=8, idx_heads=1,
                      idx_dim=8, scale=1.0, mode=0, teacher=0, dtype=1, idx_dtype=1)
    idx = torch.full((T, kcap), 7, dtype=torch.int32, device="cuda")
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    cmp_d = torch.empty(len(lengths) + 1, dtype=torch.int32, device="cuda")
    B.csa_cmp_seqlens(cu_d, len(lengths), 4, cmp_d)
    B.csa_topk_select(p, torch.from_numpy(s).cuda(), cu_d, cmp_d, idx)
    got = idx.cpu().numpy()
    assert np.all(got[int(cu[-1]):] == -1), "padding rows"
    rows = np.unique(np.concatenate([np.arange(0, T, 5), np.arange(int(cu[-1]) - 40, T)]))
    ref = O.topk_select(s[rows], cu, 4, k, kcap, T, rows=rows)
    for i, t in enumerate(rows):
        n = int((ref[i] >= 0).sum())
        assert np.array_equal(got[t][:n], np.sort(ref[i][:n])), t
        assert np.all(got[t][n:] == -1), t


def _check_selection(got, ref_scores, row0, k, rel_tol, tag):
    """`got` (one idx row) against fp64 oracle scores of the same query: the min(k, n_vis)
    selected rows ascending, -1 after them, and the set equal to the oracle's top-k except
    for swaps across the k-th score within rel_tol * max|score| (the device accumulates the
    same products in fp32, so entries that close may order either way)."""
    vis = np.isfinite(ref_scores)
    nv = int(vis.sum())
    m = min(k, nv)
    sel = got[:m].astype(np.int64) - row0
    assert np.all(got[m:] == -1), tag
    assert np.all(np.diff(sel) > 0) and (m == 0 or (sel[0] >= 0 and sel[-1] < nv)), tag
    if m == nv:
        return 0
    s = ref_scores[:nv]
    order = np.lexsort((np.arange(nv), -s))        # descending score, ties to smaller j
    ref = set(order[:m].tolist())
    thr = s[order[m - 1]]
    tol = rel_tol * float(np.abs(s).max())
    extra = set(sel.tolist()) - ref
    missing = ref - set(sel.tolist())
    assert len(extra) == len(missing), tag
    assert all(s[j] >= thr - tol for j in extra), (tag, "selected below the k-th score")
    assert all(s[j] <= thr + tol for j in missing), (tag, "skipped above the k-th score")
    return len(extra)


@pytest.mark.parametrize("name", _idx_cases())
def test_index_topk_fused(name):
    """Fused scores + top-k: idx against the oracle's top-k of its fp64 scores (near-tie
    swaps only), the score output of each mode, and agreement with the two separate calls."""
    from long_context_compressed_amd import binding as B
    w, host, h64 = _case(name)
    _announce(name, "index_topk")
    L = _layer(w, host, backward=False)
    cu = _cu(host)
    L.metadata(cu)
    d, qI64, kI64 = _indexer_inputs(w, host, h64)
    wd = host["w"].cuda()
    args = (L.p, d["qI"], d["qI_scale"], wd, d["kI"], d["kI_scale"], cu, L.cu_cmp)
    if w.idx_dtype == "f32" or w.idx_heads != 64 or w.idx_dim != 128:
        with pytest.raises(B.CsaError):
            B.csa_index_topk(*args, L.idx)
        return
    ref = O.index_scores(qI64, h64["w"], kI64, host["cu_seqlens"], w.ratio, L.n_cap)
    vis = np.isfinite(ref)
    out = {}
    for mode in (0, 1, 2):
        sc = torch.full_like(L.scores, 12345.0)
        idx = torch.full_like(L.idx, -7)
        B.csa_index_topk(*args, idx, scores=sc, scores_mode=mode)
        torch.cuda.synchronize()
        out[mode] = (G.back(sc), idx.cpu().numpy())
    s2, i2 = out[2]
    assert np.all(s2[~vis] == 12345.0), "non-visible score entries were written"
    G.check("fused scores(visible)", s2[vis], ref[vis], "bf16")
    assert np.array_equal(out[0][1], i2) and np.array_equal(out[1][1], i2)
    assert np.all(out[0][0] == 12345.0), "mode 0 wrote scores"
    s1 = out[1][0]
    chosen = np.zeros_like(vis)
    cu_cmp = O.cmp_seqlens(host["cu_seqlens"], w.ratio)
    bb, _ = O.token_positions(host["cu_seqlens"], w.total_tokens)
    swaps = 0
    for t_ in range(w.total_tokens):
        row0 = int(cu_cmp[bb[t_]]) if bb[t_] >= 0 else 0
        sel = i2[t_][i2[t_] >= 0] - row0
        chosen[t_, sel] = True
        swaps += _check_selection(i2[t_], ref[t_], row0, w.topk, 1e-4, (name, t_))
    assert np.array_equal(s1[chosen], s2[chosen]), "mode 1 selected scores differ from mode 2"
    assert np.all(s1[~chosen] == 12345.0), "mode 1 wrote unselected scores"
    print(f"[gpu] {name}: near-tie swaps {swaps}", flush=True)
    # the separate calls on the same operands give the same selection
    sc = torch.zeros_like(L.scores)
    B.csa_index_scores(*args, sc)
    idx = torch.empty_like(L.idx)
    B.csa_topk_select(L.p, sc, cu, L.cu_cmp, idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), i2)
    assert np.array_equal(G.back(sc)[vis], s2[vis])


def _random_e4m3(rng, shape):
    """Finite e4m3 codes with exponent fields 3..11 (magnitudes 2^-4 .. 2^4), random sign."""
    e = rng.integers(3, 12, size=shape)
    m = rng.integers(0, 8, size=shape)
    s = rng.integers(0, 2, size=shape)
    return ((s << 7) | (e << 3) | m).astype(np.uint8)


@pytest.mark.parametrize("idx_dtype,lengths,k", [
    ("bf16", (16384, 2500), 1000),     # rows up to 4096 keys: one wave per token
    ("fp8", (16384, 2500), 1000),
    ("bf16", (40000, 3000), 2000),     # up to 10000 keys: a workgroup per token, 32 per lane
    ("fp8", (70000, 5000), 2048),      # up to 17500 keys: 64 per lane
])
def test_index_topk_fused_long_rows(idx_dtype, lengths, k):
    """Fused scores + top-k on long rows in a two-sample batch, k not always a multiple of
    64: sampled rows against the oracle (selection and the selected scores), and the whole
    selection and score matrix equal to those of the two separate calls."""
    from long_context_compressed_amd import binding as B
    print(f"[gpu] case=index_topk_long dtype={idx_dtype} lengths={lengths} k={k}", flush=True)
    rng = np.random.default_rng(11)
    T = sum(lengths)
    cu = np.array([0, lengths[0], T], dtype=np.int64)
    r = 4
    kcap = -(-k // 64) * 64
    n_cap = max(lengths) // r
    cu_cmp = O.cmp_seqlens(cu, r)
    n_c = int(cu_cmp[-1])
    wts = (rng.standard_normal((T, 64)) / 8).astype(np.float32)
    if idx_dtype == "bf16":
        q = torch.from_numpy(rng.standard_normal((T, 64, 128), dtype=np.float32)).to(torch.bfloat16)
        kk = torch.from_numpy(rng.standard_normal((n_c, 128), dtype=np.float32)
                              / np.sqrt(128)).to(torch.bfloat16)
        dq, dk, dqs, dks = q.cuda(), kk.cuda(), None, None
        code = B.CSA_BF16
    else:
        qc, kc = _random_e4m3(rng, (T, 64, 128)), _random_e4m3(rng, (n_c, 128))
        qs = rng.uniform(0.5, 2.0, (T, 64)).astype(np.float32)
        ks = rng.uniform(0.01, 0.05, (n_c,)).astype(np.float32)
        dq, dk = torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda()
        dqs, dks = torch.from_numpy(qs).cuda(), torch.from_numpy(ks).cuda()
        code = B.CSA_FP8_E4M3
    p = B.make_params(batch=2, total_tokens=T, max_seqlen=max(lengths), ratio=r, window=128,
                      topk=k, topk_cap=kcap, heads=64, head_dim=512, idx_heads=64, idx_dim=128,
                      scale=1.0 / np.sqrt(512), mode=B.CSA_SPARSE, teacher=B.CSA_TEACHER_SELECTED,
                      dtype=B.CSA_BF16, idx_dtype=code)
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    cmp_d = torch.tensor(cu_cmp, dtype=torch.int32, device="cuda")
    args = (p, dq, dqs, torch.from_numpy(wts).cuda(), dk, dks, cu_d, cmp_d)
    idx = torch.full((T, kcap), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((T, n_cap), 12345.0, dtype=torch.float32, device="cuda")
    B.csa_index_topk(*args, idx, scores=sc, scores_mode=1)
    torch.cuda.synchronize()
    L0 = lengths[0]
    rows = [L0 - 8 + i for i in range(8)] + [L0 - 1 - 4 * 1500, 4 * k + 3, 4 * k - 1, 4 * k,
                                            4 * (k - 1) + 2, L0 // 2, L0 // 3 + 1]
    rows += [L0 + x for x in (0, 3, 4, lengths[1] // 2, lengths[1] - 1)]
    rows = np.array(sorted(set(x for x in rows if 0 <= x < T)), dtype=np.int64)
    if idx_dtype == "bf16":
        q64 = q[torch.as_tensor(rows)].double().numpy()
        k64 = kk.double().numpy()
    else:
        q64 = O.dequantize_fp8(qc[rows], qs[rows])
        k64 = O.dequantize_fp8(kc, ks)
    qv = np.zeros((T, 64, 128))
    qv[rows] = q64
    ref = O.index_scores(qv, wts.astype(np.float64), k64, cu, r, n_cap, rows=rows)
    got_i = idx.cpu().numpy()[rows]
    got_s = sc.cpu().numpy().astype(np.float64)[rows]
    for i, t_ in enumerate(rows):
        row0 = int(cu_cmp[0 if t_ < L0 else 1])
        _check_selection(got_i[i], ref[i], row0, k, 1e-4, (idx_dtype, int(t_)))
        sel = got_i[i][got_i[i] >= 0] - row0
        G.check(f"selected scores t={t_}", got_s[i][sel], ref[i][sel], "bf16")
        mask = np.ones(n_cap, bool)
        mask[sel] = False
        assert np.all(got_s[i][mask] == 12345.0), t_
    # the same operands through the two separate calls: the same selection, and the fused
    # call's every-visible-score mode writes the same score matrix
    sc2 = torch.full_like(sc, 12345.0)
    B.csa_index_scores(*args, sc2)
    idx2 = torch.empty_like(idx)
    B.csa_topk_select(p, sc2, cu_d, cmp_d, idx2)
    sc3 = torch.full_like(sc, 12345.0)
    idx3 = torch.empty_like(idx)
    B.csa_index_topk(*args, idx3, scores=sc3, scores_mode=2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(idx, idx3)
    assert torch.equal(sc2, sc3)


# ------------------------------------------------------------------------- attention
def _attn_inputs(w, host, h64):
    cu = host["cu_seqlens"]
    dt = G.torch_dtype(w.dtype)
    kv_cmp_r = G.rounded(O.compress(h64["kv"], cu, w.ratio), dt)
    idx = None
    if w.mode == "sparse" and w.has_indexer:
        _, qI64, kI64 = _indexer_inputs(w, host, h64)
        n_cap = host["max_seqlen"] // w.ratio
        sc = O.index_scores(qI64, h64["w"], kI64, cu, w.ratio, n_cap)
        idx = O.topk_select(sc, cu, w.ratio, w.topk, w.topk_cap, w.total_tokens)
    elif w.mode == "window":
        idx = np.full((w.total_tokens, 64), -1)
    return kv_cmp_r, idx


def _mode_idx(w, idx):
    return idx if w.mode in ("sparse", "window") else None


@pytest.mark.parametrize("name", list(CASES))
def test_attn_fwd(name):
    from long_context_compressed_amd import binding as B
    w, host, h64 = _case(name)
    _announce(name, "attn_fwd")
    L = _layer(w, host, backward=False)
    cu = _cu(host)
    L.metadata(cu)
    dt = G.torch_dtype(w.dtype)
    kv_cmp_r, idx = _attn_inputs(w, host, h64)
    kvc = G.dev(kv_cmp_r if kv_cmp_r.size else np.zeros((1, w.head_dim)), dt)
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda() if w.mode == "sparse" else None
    sink = host.get("sink")
    lse_cmp = torch.empty_like(L.lse)
    ld_t = B.csa_teacher_logits_stride(L.p)
    t_logits = (torch.full((w.total_tokens, w.heads, ld_t), float("nan"), device="cuda")
                if ld_t else None)
    B.csa_sparse_attn_fwd(L.p, host["q"].cuda(), kvc, host["kv"].cuda(), idx_d,
                          None if sink is None else sink.cuda(), cu, L.cu_cmp, L.out, L.lse,
                          lse_cmp, ws=L.ws_fwd, t_logits=t_logits)
    n = int(host["cu_seqlens"][-1])
    rows = np.arange(n)
    Oref, Lref = O.sparse_attn_fwd(h64["q"], kv_cmp_r, h64["kv"], _mode_idx(w, idx),
                                   h64.get("sink"), host["cu_seqlens"], w.ratio, w.window,
                                   w.scale, rows=rows)
    torch.cuda.synchronize()
    kind = _kind(name, w.dtype)
    if "rescale" in name:
        # the case reaches the lazy rescale: some (query, head) maximum grows past its first
        # block's by more than the 2^8 the forward tolerates before moving its running max
        mi = _mode_idx(w, idx)
        margin = _rescale_margin(w, h64["q"], kv_cmp_r, h64["kv"], mi, host["cu_seqlens"], rows)
        print(f"[gpu] {name}: largest growth past the first block {margin:.1f} log2 units",
              flush=True)
        assert margin > 12.0
    G.check("O", G.back(L.out)[:n], Oref, kind)
    G.check("LSE", G.back(L.lse)[:n], Lref, kind)
    # compressed-only normalizer: the same attention with an empty window and no sink
    bb, pp = O.token_positions(host["cu_seqlens"], w.total_tokens)
    if w.mode == "sparse":
        has_c = np.array([(idx[t] >= 0).any() for t in rows])
    elif w.mode == "dense":
        has_c = (pp[rows] + 1) // w.ratio > 0
    else:
        has_c = np.zeros(n, dtype=bool)
    got_c = G.back(lse_cmp)[:n]
    assert np.all(np.isneginf(got_c[~has_c])), "queries without compressed candidates"
    rc = rows[has_c]
    if rc.size:
        mi = None if _mode_idx(w, idx) is None else idx[rc]
        _, Lc = O.sparse_attn_fwd(h64["q"], kv_cmp_r, h64["kv"], mi, None, host["cu_seqlens"],
                                  w.ratio, 0, w.scale, rows=rc)
        G.check("LSE(compressed only)", got_c[has_c], Lc, kind)
    if t_logits is not None:
        # cached compressed-candidate logits, slot order of the attention call
        ref_l = O.compressed_logits(h64["q"], kv_cmp_r, None if _mode_idx(w, idx) is None
                                    else idx[rows], host["cu_seqlens"], w.ratio, w.scale,
                                    rows=rows)
        tl = G.back(t_logits)
        got_f = np.concatenate([tl[t, :, :r.shape[1]].ravel() for t, r in zip(rows, ref_l)])
        ref_f = np.concatenate([r.ravel() for r in ref_l])
        assert got_f.size > 0
        G.check("teacher logits cache", got_f, ref_f, kind)
    if n < w.total_tokens:
        assert torch.all(L.out[n:] == 0) and torch.all(L.lse[n:] == 0)


@pytest.mark.parametrize("name", list(CASES))
def test_attn_bwd(name):
    _attn_bwd_check(name)


def _repeat_rows(idx, cu, ratio):
    """Every query with at least four selected rows lists its first row again in slot 2 and
    its second row again in slot 3 (each listing is a candidate of its own)."""
    idx = idx.copy()
    n_rep = 0
    for t in range(idx.shape[0]):
        row = idx[t]
        nc = int(np.argmax(row < 0)) if np.any(row < 0) else row.shape[0]
        if nc >= 4:
            row[2], row[3] = row[0], row[1]
            n_rep += 1
    assert n_rep > 0
    return idx


@pytest.mark.parametrize("name", ["csa_bf16_thd_small", "csa_bf16_thd_staged"])
def test_attn_bwd_repeated_rows(name):
    """A row listed twice in one query's idx row is two candidates: forward and backward
    against the oracle on such idx rows (the key-major backward adds the later listings in
    a separate pass)."""
    _attn_bwd_check(name, lambda idx, host, w: _repeat_rows(idx, host["cu_seqlens"], w.ratio))


def _attn_bwd_check(name, edit_idx=None):
    from long_context_compressed_amd import binding as B
    w, host, h64 = _case(name)
    if "dO" not in host:
        pytest.skip("forward-only workload")
    _announce(name, "attn_bwd" if edit_idx is None else "attn_bwd repeated rows")
    L = _layer(w, host, backward=True)
    cu = _cu(host)
    L.metadata(cu)
    dt = G.torch_dtype(w.dtype)
    kv_cmp_r, idx = _attn_inputs(w, host, h64)
    if edit_idx is not None:
        idx = edit_idx(idx, host, w)
    n = int(host["cu_seqlens"][-1])
    rows = np.arange(n)
    Oref, Lref = O.sparse_attn_fwd(h64["q"], kv_cmp_r, h64["kv"], _mode_idx(w, idx),
                                   h64.get("sink"), host["cu_seqlens"], w.ratio, w.window,
                                   w.scale, rows=rows)
    O_r = np.zeros((w.total_tokens, w.heads, w.head_dim))
    O_r[:n] = G.rounded(Oref, dt)
    L_r = np.zeros((w.total_tokens, w.heads))
    L_r[:n] = G.rounded(Lref, torch.float32)
    dO = h64["dO"].copy()
    dO[n:] = 0
    kvc = G.dev(kv_cmp_r if kv_cmp_r.size else np.zeros((1, w.head_dim)), dt)
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda() if w.mode == "sparse" else None
    sink = host.get("sink")
    L.dkv_cmp.zero_()
    L.dkv.zero_()
    L.dsink.zero_()
    B.csa_sparse_attn_bwd(L.p, host["q"].cuda(), kvc, host["kv"].cuda(), idx_d,
                          None if sink is None else sink.cuda(), cu, L.cu_cmp, G.dev(O_r, dt),
                          G.dev(L_r, torch.float32), host["dO"].cuda(), L.dq, L.dkv_cmp, L.dkv,
                          L.dsink if sink is not None else None, L.ws_bwd)
    dq, dkc, dkv, dsink = O.sparse_attn_bwd(h64["q"], kv_cmp_r, h64["kv"], _mode_idx(w, idx),
                                            h64.get("sink"), host["cu_seqlens"], w.ratio, w.window,
                                            w.scale, O_r[:n], L_r[:n], dO[:n], rows=rows)
    torch.cuda.synchronize()
    kind = _kind(name, w.dtype)
    G.check("dq", G.back(L.dq)[:n], dq, kind)
    Tc = kv_cmp_r.shape[0]
    if w.mode != "window":
        G.check("dkv_cmp", G.back(L.dkv_cmp)[:Tc], dkc, kind)
    G.check("dkv(window)", G.back(L.dkv), dkv, kind)
    if sink is not None:
        G.check("dsink", G.back(L.dsink), dsink, kind)
    if n < w.total_tokens:
        assert torch.all(L.dq[n:] == 0)


# ------------------------------------------------------------------------- indexer KL
def _kl_variants():
    out = []
    for n in _kl_cases():
        w = configs.workload(CASES[n][0], **CASES[n][1])
        out += [(n, True, "none"), (n, False, "none")]
        if w.teacher == "selected":
            out += [(n, True, "lse"), (n, True, "cache"), (n, False, "cache")]
    return out


@pytest.mark.parametrize("name,grads,from_fwd", _kl_variants())
def test_indexer_kl(name, grads, from_fwd):
    """from_fwd: "none" (teacher recomputed), "lse" (teacher normalizer from the GPU
    forward), "cache" (normalizer and teacher logits from the GPU forward)."""
    _indexer_kl_check(name, grads, from_fwd)


@pytest.mark.parametrize("name", ["csa_bf16_thd_small", "csa_bf16_thd_staged"])
def test_indexer_kl_repeated_rows(name):
    """A row listed twice in one query's idx row is two members of C_t: loss and gradients
    from the cached teacher against the oracle on such idx rows (the key-major key gradient
    adds the later listings in a separate pass, from the same E records)."""
    _indexer_kl_check(name, True, "cache",
                      lambda idx, host, w: _repeat_rows(idx, host["cu_seqlens"], w.ratio))


def _indexer_kl_check(name, grads, from_fwd, edit_idx=None):
    from long_context_compressed_amd import binding as B
    w, host, h64 = _case(name)
    _announce(name, f"indexer_kl grads={grads} from_fwd={from_fwd}" +
              ("" if edit_idx is None else " repeated rows"))
    fwd_lse = from_fwd != "none"
    L = _layer(w, host, backward=True)
    cu = _cu(host)
    L.metadata(cu)
    dt = G.torch_dtype(w.dtype)
    kv_cmp_r, idx = _attn_inputs(w, host, h64)
    if edit_idx is not None:
        idx = edit_idx(idx, host, w)
    d, qI64, kI64 = _indexer_inputs(w, host, h64)
    sc = O.index_scores(qI64, h64["w"], kI64, host["cu_seqlens"], w.ratio, L.n_cap)
    s32 = np.where(np.isfinite(sc), sc, 0.0).astype(np.float32)
    gs = 0.5
    teacher_lse = t_logits = None
    ws = L.ws_kl
    if fwd_lse:
        # the selected-set teacher normalizer (and logits) from the GPU forward on the same inputs
        teacher_lse = torch.empty_like(L.lse)
        if from_fwd == "cache":
            ld_t = B.csa_teacher_logits_stride(L.p)
            t_logits = torch.full((w.total_tokens, w.heads, ld_t), float("nan"), device="cuda")
            n_ws = B.csa_workspace_size(L.p, B.CSA_OP_INDEXER_KL_CACHED)
            ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda") if n_ws else None
        B.csa_sparse_attn_fwd(L.p, host["q"].cuda(), G.dev(kv_cmp_r, dt), host["kv"].cuda(),
                              torch.from_numpy(idx.astype(np.int32)).cuda(), None, cu, L.cu_cmp,
                              L.out, L.lse, teacher_lse, ws=L.ws_fwd, t_logits=t_logits)
    L.dkI_cmp.zero_()
    B.csa_indexer_kl(L.p, host["q"].cuda(), G.dev(kv_cmp_r, dt), torch.from_numpy(s32).cuda(),
                     torch.from_numpy(idx.astype(np.int32)).cuda(), d["qI"], d["qI_scale"],
                     host["w"].cuda(), d["kI"], d["kI_scale"], cu, L.cu_cmp, gs, L.kl, L.loss,
                     L.dqI if grads else None, L.dw if grads else None,
                     L.dkI_cmp if grads else None, ws, teacher_lse, teacher_logits=t_logits)
    n = int(host["cu_seqlens"][-1])
    rows = np.arange(n)
    kl, loss, dqI, dw, dkI = O.indexer_kl(h64["q"], kv_cmp_r, s32[:n], idx[:n], qI64, h64["w"],
                                          kI64, host["cu_seqlens"], w.ratio, w.scale, w.teacher,
                                          gs, rows=rows)
    torch.cuda.synchronize()
    if "rescale" in name and w.teacher == "dense":
        # the dense teacher's per-head normalizer meets a key block whose logits exceed the
        # first block's maximum by more than the 2^8 its running maximum tolerates
        wd = dataclasses.replace(w, window=0)
        margin = _rescale_margin(wd, h64["q"], kv_cmp_r, h64["kv"], None, host["cu_seqlens"],
                                 rows)
        print(f"[gpu] {name}: teacher logit growth past the first key block {margin:.1f} "
              f"log2 units", flush=True)
        assert margin > 12.0
    got_loss = float(L.loss.item())
    print(f"loss gpu={got_loss:.8e} ref={loss:.8e}", flush=True)
    assert abs(got_loss - loss) <= G.TOL_LOSS_REL * abs(loss)
    G.check("kl", G.back(L.kl)[:n], kl, _kind(name, w.dtype) if w.dtype == "f32" else "bf16")
    if n < w.total_tokens:
        assert torch.all(L.kl[n:] == 0)
    if grads:
        kind = _kind(name, "f32") if (w.dtype == "f32" and w.idx_dtype == "f32") else "bf16"
        G.check("dqI", G.back(L.dqI)[:n], dqI, kind)
        G.check("dw", G.back(L.dw)[:n], dw, kind)
        Tc = kI64.shape[0]
        G.check("dkI_cmp", G.back(L.dkI_cmp)[:Tc], dkI, kind)


def _check_open(name, got, ref, bound):
    """bf16 tolerance plus, per element, the oracle's bound for ReLU masks left undecided by
    the fp32 accumulation (the device and the fp64 oracle may take either side)."""
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in the GPU result"
    tol = G.TOL_BF16_REL * float(np.abs(ref).max())
    excess = np.abs(got - ref) - tol - bound
    n_open = int((bound > 0).sum())
    print(f"[gpu] {name}: max|err| {np.abs(got - ref).max():.3e} tol {tol:.3e}, "
          f"{n_open} elements with an open-mask bound", flush=True)
    assert excess.max() <= 0, (name, float(excess.max()))


@pytest.mark.parametrize("idx_dtype,boost,given", [("bf16", None, True), ("fp8", None, True),
                                                   ("fp8", 8.0, True), ("bf16", None, False),
                                                   ("fp8", None, False)])
def test_indexer_kl_dense_teacher_chunked(idx_dtype, boost, given):
    """Dense-teacher loss on the tiled path across more than one 8192-query chunk: three
    samples starting at rows that are not multiples of 4, capacity padding, unit-variance
    inputs (peaked teacher), with and without gradients, against the oracle.  With `boost`
    the second half of every sample's kv rows is scaled so that the teacher normalizer's
    running maximum is moved after its first key block.  given = False: no score matrix is
    passed and the call forms the student scores itself."""
    from long_context_compressed_amd import binding as B
    w = configs.workload("csa128k_warmup_fp8", idx_dtype=idx_dtype, lengths=(4003, 2998, 2501),
                         total_tokens=9560, topk=64, topk_cap=64)
    host = synth_inputs.make_inputs(w, variant=0, strength=True)
    if boost:
        _boost_kv(host, boost)
    h64 = {k: synth_inputs.to_f64(v) for k, v in host.items() if isinstance(v, torch.Tensor)}
    h64["cu_seqlens"] = host["cu_seqlens"]
    h64["max_seqlen"] = host["max_seqlen"]
    name = f"dense_teacher_{idx_dtype}" + ("_rescale" if boost else "") + \
        ("" if given else "_recomputed_scores")
    L = _layer(w, host, backward=True)
    assert L.ws_kl is not None and B.csa_workspace_size(L.p, B.CSA_OP_INDEXER_KL) > 0
    cu = _cu(host)
    L.metadata(cu)
    dt = G.torch_dtype(w.dtype)
    kv_cmp_r, idx = _attn_inputs(w, host, h64)
    d, qI64, kI64 = _indexer_inputs(w, host, h64)
    sc = O.index_scores(qI64, h64["w"], kI64, host["cu_seqlens"], w.ratio, L.n_cap)
    s32 = np.where(np.isfinite(sc), sc, 0.0).astype(np.float32)
    gs = 0.25
    n = int(host["cu_seqlens"][-1])
    # fp32 accumulation of the exact products of the rounded operands: below 128 * 2^-24 of
    # sum |products|; 2^-16 leaves a margin for any summation order
    kl, loss, dqI, dw, dkI, open_bound = O.indexer_kl(
        h64["q"], kv_cmp_r, s32[:n], idx[:n], qI64, h64["w"], kI64, host["cu_seqlens"],
        w.ratio, w.scale, w.teacher, gs, rows=np.arange(n), relu_eps=2.0 ** -16)
    if boost:
        wd = dataclasses.replace(w, window=0)
        margin = _rescale_margin(wd, h64["q"], kv_cmp_r, h64["kv"], None, host["cu_seqlens"],
                                 np.arange(0, n, 7))
        print(f"[gpu] {name}: teacher logit growth past the first key block {margin:.1f}",
              flush=True)
        assert margin > 12.0
    for grads in (True, False):
        _announce(name, f"indexer_kl grads={grads}")
        L.kl.fill_(float("nan"))
        L.dkI_cmp.zero_()
        B.csa_indexer_kl(L.p, host["q"].cuda(), G.dev(kv_cmp_r, dt),
                         torch.from_numpy(s32).cuda() if given else None,
                         torch.from_numpy(idx.astype(np.int32)).cuda(), d["qI"], d["qI_scale"],
                         host["w"].cuda(), d["kI"], d["kI_scale"], cu, L.cu_cmp, gs, L.kl,
                         L.loss, L.dqI if grads else None, L.dw if grads else None,
                         L.dkI_cmp if grads else None, L.ws_kl)
        torch.cuda.synchronize()
        got_loss = float(L.loss.item())
        print(f"loss gpu={got_loss:.8e} ref={loss:.8e}", flush=True)
        assert abs(got_loss - loss) <= G.TOL_LOSS_REL * abs(loss)
        G.check("kl", G.back(L.kl)[:n], kl, "bf16")
        assert torch.all(L.kl[n:] == 0)
        if grads:
            _check_open("dqI", G.back(L.dqI)[:n], dqI, open_bound[0])
            _check_open("dw", G.back(L.dw)[:n], dw, open_bound[1])
            _check_open("dkI_cmp", G.back(L.dkI_cmp)[:kI64.shape[0]], dkI, open_bound[2])


def test_indexer_kl_dense_teacher_from_cache():
    """The cached-teacher loss with the dense teacher (CSA_DENSE attention: C_t = every visible
    compressed row): the forward keeps every visible row's logits in visible order, the loss
    reads them instead of recomputing the teacher, and the key-major key gradient runs over the
    dense kind of rows.  Unit-variance inputs (peaked teacher), capacity padding, against the
    oracle with its open-ReLU bound."""
    from long_context_compressed_amd import binding as B
    w = configs.workload("thd64k_csa_bf16", mode="dense", teacher="dense", lengths=(301, 515, 1027),
                         total_tokens=1856, draw=None)
    host = synth_inputs.make_inputs(w, variant=0, strength=True)
    h64 = {k: synth_inputs.to_f64(v) for k, v in host.items() if isinstance(v, torch.Tensor)}
    h64["cu_seqlens"] = host["cu_seqlens"]
    h64["max_seqlen"] = host["max_seqlen"]
    _announce("dense_teacher_bf16_cached", "attn_fwd + indexer_kl from the teacher cache")
    L = _layer(w, host, backward=True)
    cu = _cu(host)
    L.metadata(cu)
    dt = G.torch_dtype(w.dtype)
    kv_cmp_r, _ = _attn_inputs(w, host, h64)
    d, qI64, kI64 = _indexer_inputs(w, host, h64)
    sc = O.index_scores(qI64, h64["w"], kI64, host["cu_seqlens"], w.ratio, L.n_cap)
    s32 = np.where(np.isfinite(sc), sc, 0.0).astype(np.float32)
    ld_t = B.csa_teacher_logits_stride(L.p)
    assert ld_t >= L.n_cap and ld_t % 64 == 0
    t_logits = torch.full((w.total_tokens, w.heads, ld_t), float("nan"), device="cuda")
    kvc = G.dev(kv_cmp_r, dt)
    B.csa_sparse_attn_fwd(L.p, host["q"].cuda(), kvc, host["kv"].cuda(), None, None, cu,
                          L.cu_cmp, L.out, L.lse, None, ws=L.ws_fwd, t_logits=t_logits)
    n_ws = B.csa_workspace_size(L.p, B.CSA_OP_INDEXER_KL_CACHED)
    ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    gs = 0.5
    n = int(host["cu_seqlens"][-1])
    # (the layer object allocates the loss buffers only for the sparse phase)
    T, HI, dI = w.total_tokens, w.idx_heads, w.idx_dim
    kl_d = torch.empty(T, device="cuda")
    loss_d = torch.empty(1, device="cuda")
    dqI_d = torch.empty(T, HI, dI, device="cuda")
    dw_d = torch.empty(T, HI, device="cuda")
    dkI_d = torch.empty(L.tc_cap, dI, device="cuda")
    kl, loss, dqI, dw, dkI, open_bound = O.indexer_kl(
        h64["q"], kv_cmp_r, s32[:n], None, qI64, h64["w"], kI64, host["cu_seqlens"], w.ratio,
        w.scale, w.teacher, gs, rows=np.arange(n), relu_eps=2.0 ** -16)
    for grads in (True, False):
        kl_d.fill_(float("nan"))
        dkI_d.zero_()
        B.csa_indexer_kl(L.p, host["q"].cuda(), kvc, torch.from_numpy(s32).cuda(), None, d["qI"],
                         d["qI_scale"], host["w"].cuda(), d["kI"], d["kI_scale"], cu, L.cu_cmp,
                         gs, kl_d, loss_d, dqI_d if grads else None, dw_d if grads else None,
                         dkI_d if grads else None, ws, None, teacher_logits=t_logits)
        torch.cuda.synchronize()
        got_loss = float(loss_d.item())
        print(f"[gpu] grads={grads} loss gpu={got_loss:.8e} ref={loss:.8e}", flush=True)
        assert abs(got_loss - loss) <= G.TOL_LOSS_REL * abs(loss)
        G.check("kl", G.back(kl_d)[:n], kl, "bf16")
        assert torch.all(kl_d[n:] == 0)
        if grads:
            _check_open("dqI", G.back(dqI_d)[:n], dqI, open_bound[0])
            _check_open("dw", G.back(dw_d)[:n], dw, open_bound[1])
            _check_open("dkI_cmp", G.back(dkI_d)[:kI64.shape[0]], dkI, open_bound[2])


# ------------------------------------------------------------------------- whole layer
def _sets(a):
    return [set(r[r >= 0].tolist()) for r in np.asarray(a)]


@pytest.mark.parametrize("name", list(CASES))
def test_layer_end_to_end(name):
    """The whole layer step (every call chained on the device) against the oracle's layer
    chain with storage rounding (the chain holds compressed rows, rotated operands and the
    saved output in the device dtype and scores / LSE in fp32, as the device buffers do).
    Top-k sets then differ only where fp32 score sums meet an exact tie of the rounded
    values: each differing row is checked to be such a near-tie, every per-query output is
    compared on the rows whose sets agree, the loss over those rows to 1e-3, and the
    shared-row gradients (sums over all queries) when every set agrees."""
    from long_context_compressed_amd.pipeline import to_device
    w, host, h64 = _case(name)
    _announce(name, "layer")
    L = _layer(w, host, backward=w.backward)
    dev = to_device(host)
    L.step(dev, dev["cu_seqlens"])
    n = int(host["cu_seqlens"][-1])
    ref = O.layer_step(h64, w, rows=np.arange(n), stored=True)
    torch.cuda.synchronize()
    kind = _kind(name, w.dtype)
    k2 = _kind(name, "f32") if (w.dtype == "f32" and w.idx_dtype == "f32") else "bf16"
    ok = np.ones(n, dtype=bool)
    if "idx" in ref:
        got = L.idx.cpu().numpy()[:n]
        gs, rs = _sets(got), _sets(ref["idx"])
        ok = np.array([a == b for a, b in zip(gs, rs)], dtype=bool)
        cu_cmp = O.cmp_seqlens(host["cu_seqlens"], w.ratio)
        bb, _ = O.token_positions(host["cu_seqlens"], w.total_tokens)
        # a differing set: the swapped entries lie within fp32 accumulation error of the k-th
        # score (1e-5 of the row's largest |score|); with rotated indexer operands, whose
        # device rotation (fp32) and the oracle's (fp64) may round one element a bf16 step
        # apart, within the bf16 selection rule's 1e-3
        rel = 1e-3 if w.rope_dim else 1e-5
        for t in np.nonzero(~ok)[0]:
            _check_selection(got[t], ref["scores"][t], int(cu_cmp[bb[t]]), w.topk, rel,
                             (name, int(t)))
        print(f"[gpu] idx rows differing from the oracle chain: {int((~ok).sum())} / {n}",
              flush=True)
        assert (~ok).sum() <= max(2, n // 200)
    G.check("O", G.back(L.out)[:n][ok], ref["O"][ok], kind)
    G.check("LSE", G.back(L.lse)[:n][ok], ref["LSE"][ok], kind)
    if "O_rot" in ref:
        G.check("O_rot", G.back(L.out_rot)[:n][ok], ref["O_rot"][ok], kind)
    if "loss" in ref:
        kl_ok = ok if w.teacher == "selected" else np.ones(n, dtype=bool)
        got_kl = G.back(L.kl)[:n]
        G.check("kl", got_kl[kl_ok], ref["kl"][kl_ok], kind if w.dtype == "f32" else "bf16")
        lg, lr = float(got_kl[kl_ok].sum()), float(ref["kl"][kl_ok].sum())
        print(f"loss over {int(kl_ok.sum())} rows gpu={lg:.8e} ref={lr:.8e}", flush=True)
        assert abs(lg - lr) <= G.TOL_LOSS_REL * abs(lr)
        if kl_ok.all():
            assert abs(L.loss.item() - ref["loss"]) <= G.TOL_LOSS_REL * abs(ref["loss"])
        if w.backward:
            G.check("dqI", G.back(L.dqI)[:n][kl_ok], ref["dqI"][kl_ok], k2)
            G.check("dw", G.back(L.dw)[:n][kl_ok], ref["dw"][kl_ok], k2)
    if w.backward:
        G.check("dq", G.back(L.dq)[:n][ok], ref["dq"][ok], kind)
        if ok.all():
            G.check("dkv", G.back(L.dkv), ref["dkv"], kind)
            if "dkI_tok" in ref:
                G.check("dkI_tok", G.back(L.dkI_tok), ref["dkI_tok"], k2)


@pytest.mark.parametrize("name", ["tiny_f32_packed_tails_pad", "csa_bf16_thd_small"])
def test_forward_deterministic(name):
    from long_context_compressed_amd.pipeline import to_device
    w, host, h64 = _case(name)
    _announce(name, "determinism")
    L = _layer(w, host, backward=False)
    dev = to_device(host)
    outs = []
    for _ in range(2):
        L.step(dev, dev["cu_seqlens"])
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (L.kv_cmp, L.kI_cmp, L.scores, L.idx, L.out, L.lse)])
    for a, b in zip(*outs):
        # bitwise: unwritten capacity rows hold arbitrary bits (NaN included)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
