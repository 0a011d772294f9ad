"""GPU parity of whole layer steps on the degenerate packs of the method: no sample at all,
empty samples between others, samples shorter than the ratio (no compressed row anywhere),
one-token samples, samples of exactly one and two groups, the HCA boundary lengths
r - 1, r, r + 1, and a window-only layer with one- and two-token samples, each followed by
capacity padding.  Every step of the layer runs (the MFMA kernels for the 64 x 512 bf16
shapes, the generic ones for the small fp32 shape) and is compared with the fp64 oracle's
layer step; padding rows must come back zero (idx rows: -1).
"""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synth import configs, inputs as synth_inputs
from tests import gpu_support as G

pytestmark = pytest.mark.gpu

EDGE = {
    "f32_no_samples": ("tiny_csa_f32_L256", dict(lengths=(), total_tokens=16,
                                                 teacher="selected")),
    "f32_all_shorter_than_ratio": ("tiny_csa_f32_L256", dict(lengths=(0, 3, 0, 2),
                                                             total_tokens=8,
                                                             teacher="selected")),
    "f32_one_token_samples_dense_teacher": ("tiny_csa_f32_L256", dict(lengths=(1, 1, 4, 1, 8),
                                                                      total_tokens=20)),
    "bf16_csa_tiny_samples": ("thd64k_csa_bf16", dict(lengths=(3, 0, 5, 4, 8, 1),
                                                      total_tokens=32, topk=64, topk_cap=64,
                                                      draw=None)),
    "bf16_csa_shorter_than_ratio": ("thd64k_csa_bf16", dict(lengths=(3, 2, 0, 1),
                                                            total_tokens=12, topk=64,
                                                            topk_cap=64, draw=None)),
    "bf16_hca_ratio_boundaries": ("thd64k_hca_bf16", dict(lengths=(127, 128, 129, 0),
                                                          total_tokens=400)),
    "bf16_window_only_short": ("thd64k_window_bf16", dict(lengths=(1, 2, 130), total_tokens=140,
                                                          draw=None)),
    "bf16_rope_tiny_samples": ("thd64k_csa_rope_bf16", dict(lengths=(3, 0, 5, 4, 8, 1),
                                                            total_tokens=32, topk=64,
                                                            topk_cap=64, draw=None)),
    "fp8_dense_teacher_tiny": ("csa128k_warmup_fp8", dict(lengths=(9, 0, 4, 2),
                                                          total_tokens=20, topk=64,
                                                          topk_cap=64)),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_degenerate_pack_layer(name):
    from long_context_compressed_amd.pipeline import CsaLayer, LayerConfig, to_device
    base, over = EDGE[name]
    w = configs.workload(base, **over)
    print(f"[gpu] edge case={name} lengths={over['lengths']}", flush=True)
    host = synth_inputs.make_inputs(w)
    h64 = {k: synth_inputs.to_f64(v) for k, v in host.items() if isinstance(v, torch.Tensor)}
    h64["cu_seqlens"] = host["cu_seqlens"]
    h64["max_seqlen"] = host["max_seqlen"]
    L = CsaLayer(LayerConfig.of(w), len(host["lengths"]), w.total_tokens, host["max_seqlen"],
                 backward=w.backward)
    dev = to_device(host)
    L.step(dev, dev["cu_seqlens"])
    torch.cuda.synchronize()
    n = int(host["cu_seqlens"][-1])
    T = w.total_tokens
    # the oracle chain with storage rounding: compressed rows and rotated operands in the
    # device dtype, scores and LSE in fp32, as the device buffers hold them
    ref = O.layer_step(h64, w, rows=np.arange(n), stored=True)
    kind = w.dtype
    Tc = int(O.cmp_seqlens(host["cu_seqlens"], w.ratio)[-1])
    assert torch.equal(L.cu_cmp.cpu().to(torch.int64),
                       torch.as_tensor(O.cmp_seqlens(host["cu_seqlens"], w.ratio)))
    if Tc:
        ref_kvc = ref["kv_cmp"]
        if w.rope_dim:   # the layer rotates its compressed rows in place
            ref_kvc = O.rope(ref_kvc, O.rope_positions(host["cu_seqlens"], Tc, ratio=w.ratio),
                             w.rope_dim, w.rope_theta)
        G.check("kv_cmp", G.back(L.kv_cmp)[:Tc], ref_kvc, kind)
    if "idx" in ref:
        got = L.idx.cpu().numpy()
        assert G.idx_sets_equal(got[:n], ref["idx"]) == 0
        assert np.all(got[n:] == -1)
    if n:
        G.check("O", G.back(L.out)[:n], ref["O"], kind)
        G.check("LSE", G.back(L.lse)[:n], ref["LSE"], kind)
        if "O_rot" in ref:
            G.check("O_rot", G.back(L.out_rot)[:n], ref["O_rot"], kind)
    assert torch.all(L.out[n:] == 0) and torch.all(L.lse[n:] == 0)
    if "loss" in ref:
        got_loss = float(L.loss.item())
        print(f"loss gpu={got_loss:.8e} ref={ref['loss']:.8e}", flush=True)
        assert abs(got_loss - ref["loss"]) <= G.TOL_LOSS_REL * abs(ref["loss"]) + 1e-12
        if n:
            G.check("kl", G.back(L.kl)[:n], ref["kl"], kind)
        assert torch.all(L.kl[n:] == 0)
    if w.backward:
        if n:
            G.check("dq", G.back(L.dq)[:n], ref["dq"], kind)
        assert torch.all(L.dq[n:] == 0)
        G.check("dkv", G.back(L.dkv), ref["dkv"], kind)
        if "dkI_tok" in ref:
            k2 = "f32" if (w.dtype == "f32" and w.idx_dtype == "f32") else "bf16"
            G.check("dkI_tok", G.back(L.dkI_tok), ref["dkI_tok"], k2)
            if n:
                G.check("dqI", G.back(L.dqI)[:n], ref["dqI"], k2)
    assert T >= n


def test_layer_forward_forms_compressed_offsets():
    """A layer forward called without a separate metadata call forms the compressed offsets
    itself (a forward that read a stale offsets buffer indexed rows through it); the offsets
    buffer starts zeroed here, so a forward that skipped them would give wrong outputs."""
    from long_context_compressed_amd.pipeline import CsaLayer, LayerConfig, to_device
    w = configs.workload("thd64k_csa_bf16", lengths=(37, 0, 90, 5), total_tokens=160, topk=64,
                         topk_cap=64, draw=None, backward=False)
    print("[gpu] case=forward_forms_offsets", flush=True)
    host = synth_inputs.make_inputs(w)
    h64 = {k: synth_inputs.to_f64(v) for k, v in host.items() if isinstance(v, torch.Tensor)}
    h64["cu_seqlens"] = host["cu_seqlens"]
    h64["max_seqlen"] = host["max_seqlen"]
    L = CsaLayer(LayerConfig.of(w), len(host["lengths"]), w.total_tokens, host["max_seqlen"],
                 backward=False)
    L.cu_cmp.zero_()
    dev = to_device(host)
    L.forward(dev, dev["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(L.cu_cmp.cpu().to(torch.int64),
                       torch.as_tensor(O.cmp_seqlens(host["cu_seqlens"], w.ratio)))
    n = int(host["cu_seqlens"][-1])
    ref = O.layer_step(h64, w, rows=np.arange(n), stored=True)
    G.check("O", G.back(L.out)[:n], ref["O"], w.dtype)
