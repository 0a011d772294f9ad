"""The allocation-free attention backward (csa_sparse_attn_bwd_noalloc) against the
workspace-taking csa_sparse_attn_bwd, through the C ABI, on two calls in a row: a larger
packed batch whose queries need many chunks of the library's static workspace, then a
smaller one (the second call reuses the array the first left behind).  Both calls get the
same forward outputs; results must agree to the bf16 parity bar (norm-relative 2e-2; the
two differ only in the order of the fp32 owner sums)."""
import numpy as np
import pytest
import torch

from synth import configs, inputs as synth_inputs
from tests import gpu_support as G

pytestmark = pytest.mark.gpu


def _run(lengths, total, topk, sink):
    from long_context_compressed_amd import binding as B
    from long_context_compressed_amd.pipeline import CsaLayer, LayerConfig, to_device
    base = "thd64k_csa_sink_bf16" if sink else "thd64k_csa_bf16"
    w = configs.workload(base, lengths=lengths, total_tokens=total, topk=topk, topk_cap=topk,
                         draw=None, teacher="none")
    print(f"[gpu] case=noalloc lengths={lengths} topk={topk} sink={sink}", flush=True)
    host = synth_inputs.make_inputs(w)
    dev = to_device(host)
    L = CsaLayer(LayerConfig.of(w), len(lengths), total, host["max_seqlen"], backward=True)
    L.forward(dev, dev["cu_seqlens"])
    n_min = B.csa_workspace_size_min(L.p, B.CSA_OP_ATTN_BWD)
    n_pref = B.csa_workspace_size(L.p, B.CSA_OP_ATTN_BWD)
    assert 0 < n_min <= n_pref
    outs = []
    for variant in ("workspace", "noalloc"):
        dq = torch.full_like(L.dq, float("nan"))
        dkc = torch.zeros_like(L.dkv_cmp)
        dkv = torch.zeros_like(L.dkv)
        dsk = torch.zeros_like(L.dsink)
        args = (L.p, dev["q"], L.kv_cmp, dev["kv"], L.idx, dev.get("sink"), dev["cu_seqlens"],
                L.cu_cmp, L.out, L.lse, dev["dO"], dq, dkc, dkv, dsk if sink else None)
        if variant == "workspace":
            B.csa_sparse_attn_bwd(*args, L.ws_bwd)
        else:
            B.csa_sparse_attn_bwd_noalloc(*args)
        torch.cuda.synchronize()
        outs.append((dq, dkc, dkv, dsk))
    n = int(host["cu_seqlens"][-1])
    Tc = int(L.cu_cmp[-1].item())
    (a_dq, a_dkc, a_dkv, a_ds), (b_dq, b_dkc, b_dkv, b_ds) = outs
    G.check("dq", G.back(b_dq[:n]), G.back(a_dq[:n]), "bf16")
    assert torch.all(b_dq[n:] == 0)
    G.check("dkv_cmp", G.back(b_dkc[:Tc]), G.back(a_dkc[:Tc]), "bf16")
    G.check("dkv", G.back(b_dkv), G.back(a_dkv), "bf16")
    assert torch.all(b_dkc[Tc:] == 0)
    if sink:
        G.check("dsink", G.back(b_ds), G.back(a_ds), "bf16")
    return n_min


def test_noalloc_backward_matches_workspace_backward_twice():
    # 1st call: 4 samples, k = 1024 (about 1.5 MB of workspace per query: many chunks of the
    # static array); 2nd call: a smaller batch with a sink
    big = _run((3000, 1700, 2500, 900), 8192, 1024, sink=False)
    small = _run((301, 515, 1027), 1856, 64, sink=True)
    assert small < big


def test_noalloc_rejects_a_shape_beyond_its_workspace():
    """A shape whose smallest chunk exceeds the static array is refused before any launch."""
    from long_context_compressed_amd import binding as B
    p = B.make_params(batch=1, total_tokens=1 << 20, max_seqlen=1 << 20, ratio=4, window=128,
                      topk=65536, topk_cap=65536, heads=64, head_dim=512, idx_heads=64,
                      idx_dim=128, scale=1.0 / np.sqrt(512), mode=B.CSA_SPARSE,
                      teacher=B.CSA_TEACHER_NONE, dtype=B.CSA_BF16, idx_dtype=B.CSA_BF16)
    assert B.csa_workspace_size_min(p, B.CSA_OP_ATTN_BWD) > 256 << 20
    fake = 4096
    st = B.lib().csa_sparse_attn_bwd_noalloc(
        __import__("ctypes").byref(p), fake, fake, fake, fake, None, fake, fake, fake, fake,
        fake, fake, fake, fake, None, None)
    assert st == B.CSA_ERR_WORKSPACE
