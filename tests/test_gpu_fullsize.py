"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Per-query outputs (top-k sets, O, LSE, KL, dq, dqI, dw) are checked against the fp64
oracle on sampled query rows: the first rows, rows around the dense-to-sparse switch
p = k*r, and the last rows of samples.  Attention gradients of shared rows (dkv_cmp and
window dkv) are checked element by element for the sampled queries: the backward is rerun
with dO zero outside them.  The indexer-key gradient needs every query and is checked
through identities that hold at any size:
  <dqI_t, qI_t> = sum_h dw[t,h] w[t,h]                   (per query)
  sum_t <dqI_t, qI_t> = <dkI_cmp, kI_cmp>                (indexer keys)
Element-wise checks of every gradient also run on the reduced instances of test_gpu_parity.
"""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from synth import configs, inputs as synth_inputs
from tests import gpu_support as G

pytestmark = pytest.mark.gpu

NAMES = ["tiny_csa_f32_L256", "csa_sparse_fwd_bf16_L4096", "thd64k_csa_bf16", "thd64k_hca_bf16",
         "thd64k_window_bf16", "csa128k_warmup_fp8", "thd64k_csa_rope_bf16"]


# relative rounding of a compressed indexer key on the GPU chain: bf16 storage (2^-9, with
# margin for fp32 accumulation) or one e4m3 code step on top of it (2^-4 relative, times the
# scale difference it can cause)
EPS_KEY = {"f32": 2.0 ** -20, "bf16": 2.0 ** -8, "fp8": 2.0 ** -2}


def _sample_rows(w, lens, cu, n_per=4):
    rows = []
    k_r = w.topk * w.ratio
    for b, L in enumerate(lens):
        s = int(cu[b])
        cand = [0, 1, L // 2, L - 2, L - 1]
        if w.mode == "sparse":
            cand += [k_r - 2, k_r - 1, k_r, k_r + 5]
        cand = [p for p in cand if 0 <= p < L]
        rows += [s + p for p in sorted(set(cand))[:n_per + 4]]
    return np.array(sorted(set(rows)), dtype=np.int64)


def _dot(a, b):
    return float((a.double() * b.double()).sum().item())


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_sampled(name):
    from long_context_compressed_amd import binding as B
    from long_context_compressed_amd.pipeline import CsaLayer, LayerConfig, to_device
    w = configs.workload(name)
    print(f"[gpu] fullsize case={name} step=inputs", flush=True)
    host = synth_inputs.make_inputs(w)
    dev = to_device(host)
    lens, cu = host["lengths"], host["cu_seqlens"]
    T = w.total_tokens
    layer = CsaLayer(LayerConfig.of(w), len(lens), T, host["max_seqlen"], backward=w.backward)
    print(f"[gpu] fullsize case={name} step=layer", flush=True)
    layer.step(dev, dev["cu_seqlens"])
    torch.cuda.synchronize()
    rows = _sample_rows(w, lens, cu)
    kind = w.dtype

    # ---- oracle on the sampled rows (full-size arrays only touched where needed)
    h64 = {"cu_seqlens": cu, "max_seqlen": host["max_seqlen"],
           "kv": synth_inputs.to_f64(host["kv"])}
    if w.has_indexer:
        h64["kI_tok"] = synth_inputs.to_f64(host["kI_tok"])
    for key in ("q", "qI", "w", "dO"):
        if key in host:
            a = np.zeros(tuple(host[key].shape))
            a[rows] = synth_inputs.to_f64(host[key][torch.as_tensor(rows)])
            h64[key] = a
    ref = O.layer_step(h64, w, rows=rows)

    # top-k: compare as sets; any difference must sit at a near-tie of the oracle scores
    if "idx" in ref:
        got = layer.idx[torch.as_tensor(rows).cuda()].cpu().numpy()
        flips = 0
        for i in range(rows.size):
            gs_, rs_ = set(got[i][got[i] >= 0].tolist()), set(ref["idx"][i][ref["idx"][i] >= 0].tolist())
            assert len(gs_) == len(rs_), rows[i]
            if gs_ != rs_:
                flips += 1
                sc = ref["scores"][i]
                row0 = O.cmp_seqlens(cu, w.ratio)[np.searchsorted(cu, rows[i], side="right") - 1]
                kth = np.sort(sc[np.isfinite(sc)])[::-1][len(rs_) - 1]
                t = rows[i]
                qn = np.linalg.norm(h64["qI"][t], axis=1)               # [H_I]
                for gsel in gs_ - rs_:
                    # the GPU rounds the compressed keys (bf16, then e4m3 for fp8) where the
                    # fp64 chain does not: |dz| <= eps |qI_h| |kI_j|, so a swap is only
                    # allowed within sum_h |w_h| eps |qI_h| |kI_j| of the k-th score
                    kn = np.linalg.norm(ref["kI_cmp"][gsel])
                    tol = EPS_KEY[w.idx_dtype] * float(np.abs(h64["w"][t]) @ qn) * kn
                    assert sc[gsel - row0] >= kth - tol, (t, sc[gsel - row0], kth, tol)
        print(f"top-k rows differing from the fp64 chain: {flips}/{rows.size}", flush=True)
        if w.dtype == "f32":
            assert flips <= 1
    G.check("O(sampled)", G.back(layer.out[torch.as_tensor(rows).cuda()]), ref["O"],
            kind, rel_tol=3e-2 if kind != "f32" else None)
    G.check("LSE(sampled)", G.back(layer.lse[torch.as_tensor(rows).cuda()]), ref["LSE"], kind)
    if "O_rot" in ref:
        G.check("O_rot(sampled)", G.back(layer.out_rot[torch.as_tensor(rows).cuda()]),
                ref["O_rot"], kind, rel_tol=3e-2 if kind != "f32" else None)
    if "kl" in ref:
        G.check("kl(sampled)", G.back(layer.kl[torch.as_tensor(rows).cuda()]), ref["kl"],
                "f32" if kind == "f32" else "bf16", abs_tol=1e-4, rel_tol=5e-2)
    if not w.backward:
        return
    G.check("dq(sampled)", G.back(layer.dq[torch.as_tensor(rows).cuda()]), ref["dq"], kind,
            rel_tol=3e-2 if kind != "f32" else None, abs_tol=1e-4 if kind == "f32" else None)
    if "dqI" in ref:
        # the loss of a query is defined over its candidate set (the selected rows for a
        # selected-set teacher): compare where the GPU selected the fp64 chain's set
        k2 = "f32" if (w.dtype == "f32" and w.idx_dtype == "f32") else "bf16"
        sel = np.arange(rows.size)
        if w.teacher == "selected":
            got = layer.idx[torch.as_tensor(rows).cuda()].cpu().numpy()
            sel = np.array([i for i in range(rows.size) if set(got[i][got[i] >= 0].tolist()) ==
                            set(ref["idx"][i][ref["idx"][i] >= 0].tolist())], dtype=np.int64)
        rs = torch.as_tensor(rows[sel]).cuda()
        G.check("dqI(sampled)", G.back(layer.dqI[rs]), ref["dqI"][sel], k2, abs_tol=1e-4,
                rel_tol=5e-2)
        G.check("dw(sampled)", G.back(layer.dw[rs]), ref["dw"][sel], k2, abs_tol=1e-4,
                rel_tol=5e-2)

    # ---- shared-row gradients of the sampled queries only: dO is zero elsewhere, so every
    # other query contributes nothing (dS = P (dP - Dt) = 0 and P^T dO = 0)
    print(f"[gpu] fullsize case={name} step=shared-row gradients", flush=True)
    n = int(cu[-1])
    p = layer.p
    sink = dev.get("sink")
    keep = rows
    if "idx" in ref:   # rows whose selected set equals the fp64 chain's
        got = layer.idx[torch.as_tensor(rows).cuda()].cpu().numpy()
        same = [i for i in range(rows.size)
                if set(got[i][got[i] >= 0].tolist()) == set(ref["idx"][i][ref["idx"][i] >= 0].tolist())]
        keep = rows[same]
    rd = w.rope_dim
    Tc = int(O.cmp_seqlens(cu, w.ratio)[-1])
    kv_ref, kvc_ref, dO_ref = h64["kv"], ref["kv_cmp"], h64["dO"][keep]
    if rd:
        # the step left q and dO rotated in place (dO now the gradient of the unrotated
        # output); the direct call below works in the rotated frame, and so does its oracle
        tpos = O.rope_positions(cu, T)
        h64["q"][rows] = O.rope(h64["q"][rows], tpos[rows], rd, w.rope_theta)
        kv_ref = O.rope(h64["kv"], tpos, rd, w.rope_theta)
        kvc_ref = O.rope(ref["kv_cmp"], O.rope_positions(cu, Tc, ratio=w.ratio), rd,
                         w.rope_theta)
        dO_ref = O.rope(dO_ref, tpos[keep], rd, w.rope_theta)
    dO_sub = torch.zeros_like(dev["dO"])
    dO_sub[torch.as_tensor(keep).cuda()] = dev["dO"][torch.as_tensor(keep).cuda()]
    layer.dkv_cmp.zero_()
    layer.dkv.zero_()
    B.csa_sparse_attn_bwd(p, dev["q"], layer.kv_cmp, layer.kv_rot if rd else dev["kv"],
                          layer.idx if layer.cfg.has_indexer else None, sink, dev["cu_seqlens"],
                          layer.cu_cmp, layer.out, layer.lse, dO_sub, layer.dq, layer.dkv_cmp,
                          layer.dkv, layer.dsink if sink is not None else None, layer.ws_bwd)
    torch.cuda.synchronize()
    pos = np.searchsorted(rows, keep)
    ref_idx = None if "idx" not in ref else ref["idx"][pos]
    if w.mode == "window":
        ref_idx = np.full((keep.size, 1), -1)
    Or, Lr = ref["O"][pos], ref["LSE"][pos]
    _, dkc, dkw, _ = O.sparse_attn_bwd(h64["q"], kvc_ref, kv_ref, ref_idx, None, cu,
                                       w.ratio, w.window, w.scale, Or, Lr, dO_ref, rows=keep)
    G.check("dkv_cmp(sampled queries)", G.back(layer.dkv_cmp[:Tc]), dkc, kind,
            rel_tol=3e-2 if kind != "f32" else None, abs_tol=1e-4 if kind == "f32" else None)
    G.check("dkv window(sampled queries)", G.back(layer.dkv), dkw, kind,
            rel_tol=3e-2 if kind != "f32" else None, abs_tol=1e-4 if kind == "f32" else None)
    del dO_sub
    if "dqI" in ref:
        qI_dev = layer.qI8 if w.idx_dtype == "fp8" else dev["qI"]
        if w.idx_dtype == "fp8":
            qI_val = layer.qI8.cpu()
            qI_f = torch.from_numpy(O.dequantize_fp8(qI_val.numpy(), layer.qI_scale.cpu().numpy())).float()
            kI_f = torch.from_numpy(O.dequantize_fp8(layer.kI8[:Tc].cpu().numpy(), layer.kI_scale[:Tc].cpu().numpy())).float()
        else:
            qI_f = dev["qI"].float().cpu()
            kI_f = layer.kI_cmp[:Tc].float().cpu()
        del qI_dev
        dqI_g, dkI_g = layer.dqI, layer.dkI_cmp
        if rd:
            # qI and kI_cmp hold the rotated operands; the gradients were rotated back
            dqI_g, dkI_g = torch.empty_like(dqI_g), torch.empty_like(dkI_g)
            B.csa_rope(layer.dqI, dqI_g, rd, w.rope_theta, 0, len(lens), dev["cu_seqlens"])
            B.csa_rope(layer.dkI_cmp, dkI_g, rd, w.rope_theta, 0, len(lens), layer.cu_cmp)
            torch.cuda.synchronize()
        per_t = (dqI_g[:n].cpu().double() * qI_f[:n].double()).sum(dim=(1, 2))
        dww = (layer.dw[:n].cpu().double() * dev["w"][:n].cpu().double()).sum(dim=1)
        err = float((per_t - dww).abs().max())
        print(f"indexer identity per query: max |<dqI,qI> - <dw,w>| = {err:.3e} "
              f"(max {float(per_t.abs().max()):.3e})", flush=True)
        assert err <= 2e-2 * max(float(per_t.abs().max()), 1e-12)
        tot = float(per_t.sum())
        kk = float((dkI_g[:Tc].cpu().double() * kI_f.double()).sum())
        print(f"indexer key identity: sum_t <dqI,qI> = {tot:.6e}  <dkI,kI> = {kk:.6e}", flush=True)
        assert abs(tot - kk) <= 2e-2 * max(float(per_t.abs().sum()), 1e-12)
