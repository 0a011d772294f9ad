"""GPU parity of the rotary embedding: csa_rope against the oracle's rotation, and the
attention forward's fused inverse rotation (out_rot) against both the oracle and the
stand-alone call.

Tolerances: f32 max-abs 1e-5 at any position (the angle is formed in fp64; an fp32 angle
would be off by ~4e-3 radians near position 131071); bf16 per element within one bf16
rounding of the reference (2^-8 relative, plus 1e-6 absolute).  Channels outside the rotary
band and rows outside every sample are compared bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests import gpu_support as G

pytestmark = pytest.mark.gpu


def _check_rot(name, got, ref, dtype):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    print(f"{name}: max_abs_err={err.max():.3e} max_ref={np.abs(ref).max():.3e}", flush=True)
    if dtype == "f32":
        assert err.max() <= 1e-5
    else:
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6), name


def _offsets(lens):
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    return cu


ROPE_CASES = {
    # name: (dtype, sample lengths, capacity rows, heads, dim, rope_dim, theta, compressed r)
    "f32_tokens_3heads_pad": ("f32", (37, 100, 3, 64), 220, 3, 64, 16, 10000.0, None),
    "bf16_tokens_64x512": ("bf16", (301, 515, 1027), 1856, 64, 512, 64, 10000.0, None),
    "bf16_compressed_rows": ("bf16", (301, 515, 1027), 1856, 1, 512, 64, 10000.0, 4),
    "f32_indexer_rows": ("f32", (301, 515, 1027), 1856, 64, 128, 64, 10000.0, None),
    "f32_full_band_one_head": ("f32", (50, 0, 77), 140, 1, 8, 8, 3.0, None),
    "f32_long_sample_positions": ("f32", (131072,), 131072, 1, 64, 64, 10000.0, None),
}


@pytest.mark.parametrize("inverse", [0, 1])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("name", list(ROPE_CASES))
def test_rope(name, in_place, inverse):
    from long_context_compressed_amd import binding as B
    dt, lens, T, H, D, rd, theta, r = ROPE_CASES[name]
    print(f"[gpu] rope case={name} in_place={in_place} inverse={inverse}", flush=True)
    cu = _offsets(lens)
    offs = O.cmp_seqlens(cu, r) if r else cu
    rows = int(offs[-1]) + (3 if r else T - int(cu[-1]))        # a few rows of no sample
    rng = np.random.default_rng(list(ROPE_CASES).index(name) * 10 + inverse)
    shape = (rows, H, D) if H > 1 else (rows, D)
    x = G.dev(rng.standard_normal(shape), G.torch_dtype(dt))
    x64 = G.back(x)
    pos = (O.rope_positions(cu, rows, ratio=r) if r else O.rope_positions(cu, rows))
    ref = O.rope(x64, pos, rd, theta, inverse=bool(inverse))
    y = x.clone() if in_place else torch.full_like(x, float("nan"))
    offs_d = torch.tensor(offs, dtype=torch.int32, device="cuda")
    B.csa_rope(y if in_place else x, y, rd, theta, inverse, len(lens), offs_d)
    torch.cuda.synchronize()
    got = G.back(y)
    _check_rot(name, got[..., D - rd:], ref[..., D - rd:], dt)
    # outside the band, and rows of no sample: the input's bits
    raw_x, raw_y = x.view(torch.int16 if dt == "bf16" else torch.int32), \
        y.view(torch.int16 if dt == "bf16" else torch.int32)
    assert torch.equal(raw_y[..., :D - rd], raw_x[..., :D - rd])
    n = int(offs[-1])
    assert torch.equal(raw_y[n:], raw_x[n:])
    if not in_place:
        assert torch.equal(raw_x, G.dev(x64, G.torch_dtype(dt)).view(raw_x.dtype))  # x untouched


def test_rope_roundtrip_and_empty():
    from long_context_compressed_amd import binding as B
    rng = np.random.default_rng(3)
    x = torch.tensor(rng.standard_normal((500, 4, 64)), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 200, 450], dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    B.csa_rope(x, y, 32, 500.0, 0, 2, cu)
    B.csa_rope(y, y, 32, 500.0, 1, 2, cu)
    torch.cuda.synchronize()
    assert float((y - x).abs().max()) <= 1e-5
    e = torch.empty(0, 4, 64, device="cuda")
    B.csa_rope(e, e, 32, 500.0, 0, 2, cu)            # zero rows: nothing launched
    torch.cuda.synchronize()


FUSED_CASES = {
    # bf16 64 x 512: the MFMA forward rotates in its epilogue; f32: the generic forward,
    # then the stand-alone rotation
    "bf16_mfma_epilogue": ("thd64k_csa_bf16", dict(lengths=(301, 515, 1027), total_tokens=1856,
                                                   topk=64, topk_cap=64, draw=None,
                                                   rope_dim=64)),
    "bf16_mfma_dense_hca": ("thd64k_hca_bf16", dict(lengths=(1024, 700, 300),
                                                    total_tokens=2048, rope_dim=64)),
    "f32_generic": ("tiny_csa_f32_L256", dict(lengths=(37, 100, 3, 64), total_tokens=220,
                                              rope_dim=16, rope_theta=777.0)),
}


@pytest.mark.parametrize("name", list(FUSED_CASES))
def test_attn_fwd_out_rot(name):
    """out_rot = inverse rotation of out at the query position: against the oracle's
    rotation of the GPU's own out (isolating the epilogue), against the oracle's whole
    attention, and bit for bit against csa_rope of out; out itself is left unchanged."""
    from long_context_compressed_amd import binding as B
    from long_context_compressed_amd.pipeline import CsaLayer, LayerConfig
    from synth import configs, inputs as synth_inputs
    base, over = FUSED_CASES[name]
    w = configs.workload(base, **over)
    print(f"[gpu] rope case={name} step=attn_fwd out_rot", flush=True)
    host = synth_inputs.make_inputs(w, want=("q", "kv", "qI", "kI_tok", "w"))
    cu_np = host["cu_seqlens"]
    L = CsaLayer(LayerConfig.of(w), len(host["lengths"]), w.total_tokens, host["max_seqlen"],
                 backward=False)
    cu = torch.tensor(cu_np, dtype=torch.int32, device="cuda")
    L.metadata(cu)
    dt = G.torch_dtype(w.dtype)
    kv64 = synth_inputs.to_f64(host["kv"])
    kv_cmp_r = G.rounded(O.compress(kv64, cu_np, w.ratio), dt)
    kvc = G.dev(kv_cmp_r if kv_cmp_r.size else np.zeros((1, w.head_dim)), dt)
    idx = None
    if w.mode == "sparse":
        # a fixed valid selection: the first min(k, n_vis) visible rows of each query
        T, kc = w.total_tokens, w.topk_cap
        idx = np.full((T, kc), -1, dtype=np.int32)
        cu_cmp = O.cmp_seqlens(cu_np, w.ratio)
        b_, p_ = O.token_positions(cu_np, T)
        for t in range(int(cu_np[-1])):
            nv = min(int(O.n_visible(p_[t], w.ratio)), w.topk)
            idx[t, :nv] = cu_cmp[b_[t]] + np.arange(nv)
        idx = torch.from_numpy(idx).cuda()
    q, kv = host["q"].cuda(), host["kv"].cuda()
    out_rot = torch.full_like(L.out, float("nan"))
    B.csa_sparse_attn_fwd(L.p, q, kvc, kv, idx, None, cu, L.cu_cmp, L.out, L.lse,
                          ws=L.ws_fwd, out_rot=out_rot)
    out_a = L.out.clone()
    B.csa_sparse_attn_fwd(L.p, q, kvc, kv, idx, None, cu, L.cu_cmp, L.out, L.lse, ws=L.ws_fwd)
    sep = torch.empty_like(L.out)
    B.csa_rope(L.out, sep, w.rope_dim, w.rope_theta, 1, len(host["lengths"]), cu)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       L.out.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
    assert torch.equal(out_rot.view(torch.uint8), sep.view(torch.uint8)), "fused != separate"
    n = int(cu_np[-1])
    pos = O.rope_positions(cu_np, w.total_tokens)
    o64 = G.back(L.out)
    D, rd = w.head_dim, w.rope_dim
    ref_rot = O.rope(o64, pos, rd, w.rope_theta, inverse=True)
    _check_rot("out_rot (of the GPU out)", G.back(out_rot)[:n, :, D - rd:],
               ref_rot[:n, :, D - rd:], w.dtype)
    rows = np.arange(n)
    Oref, _ = O.sparse_attn_fwd(synth_inputs.to_f64(host["q"]), kv_cmp_r, kv64,
                                None if idx is None else idx.cpu().numpy().astype(np.int64),
                                None, cu_np, w.ratio, w.window, w.scale, rows=rows)
    G.check("out_rot (oracle attention)", G.back(out_rot)[:n],
            O.rope(Oref, pos[:n], rd, w.rope_theta, inverse=True), w.dtype)
    if n < w.total_tokens:
        assert torch.all(out_rot[n:] == 0)
