"""One CSA/HCA layer step (forward + backward) chained over the C ABI.

`CsaLayer` preallocates every output, gradient and workspace buffer with torch once,
so a step enqueues only library kernels (and torch fill kernels that zero the
accumulated gradients) on the current stream.  The order follows the fused training
flow of "DeepSeek-V4 Attention Training Systems", section 8.2: compress, indexer score
+ top-k, selected-attention forward, teacher recompute with the eager indexer-loss
backward, then the attention backward and the compressor adjoints.

With a rotary band (rope_dim > 0) the step also applies the layer's positional rotations
(same page, section 4: positions restart per packed sample; section 12: per compressed
coordinate system, and the saved output survives the inverse rotation): the projected q,
qI and the incoming dO are rotated IN PLACE (rotary channels only, as a fused
norm/rotation producer would leave them), the window rows of kv into a buffer of the
layer's own (the compressor reads the unrotated rows), the compressed rows in place after
the compressor, the output inverse-rotated by the attention forward into `out_rot` while
`out` stays the saved unrotated output, and every gradient is rotated back.
"""
from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as B

MODE = {"sparse": B.CSA_SPARSE, "dense": B.CSA_DENSE, "window": B.CSA_WINDOW}
TEACHER = {"none": B.CSA_TEACHER_NONE, "selected": B.CSA_TEACHER_SELECTED,
           "dense": B.CSA_TEACHER_DENSE}
DTYPE = {"f32": B.CSA_F32, "bf16": B.CSA_BF16, "fp8": B.CSA_FP8_E4M3}


@dataclass
class LayerConfig:
    heads: int
    head_dim: int
    ratio: int
    window: int
    topk: int
    topk_cap: int
    idx_heads: int
    idx_dim: int
    dtype: str
    idx_dtype: str
    mode: str
    teacher: str
    scale: float
    rope_dim: int = 0
    rope_theta: float = 10000.0

    @classmethod
    def of(cls, w):
        return cls(heads=w.heads, head_dim=w.head_dim, ratio=w.ratio, window=w.window,
                   topk=w.topk, topk_cap=w.topk_cap, idx_heads=w.idx_heads, idx_dim=w.idx_dim,
                   dtype=w.dtype, idx_dtype=w.idx_dtype, mode=w.mode, teacher=w.teacher,
                   scale=w.scale, rope_dim=getattr(w, "rope_dim", 0),
                   rope_theta=getattr(w, "rope_theta", 10000.0))

    @property
    def has_indexer(self):
        return self.idx_heads > 0 and self.mode == "sparse"


class CsaLayer:
    """Buffers and calls of one layer step for a fixed capacity (T rows, max_seqlen)."""

    def __init__(self, cfg: LayerConfig, batch: int, total_tokens: int, max_seqlen: int,
                 device="cuda", backward: bool = True, grad_scale: float = 1.0,
                 bwd_ws_bytes: Optional[int] = None):
        """bwd_ws_bytes: cap on the attention backward's workspace (it then processes the
        queries in more chunks; never below the library's minimum)."""
        self.cfg = cfg
        self.timer = None          # optional object with mark(name) / done(name) around calls
        self.fused_topk = None     # fused scores + top-k: None until the first forward tries it
        self.backward = backward
        self.grad_scale = grad_scale
        dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        T, H, D, r = total_tokens, cfg.heads, cfg.head_dim, cfg.ratio
        self.T, self.B = T, batch
        self.n_cap = max_seqlen // r
        self.tc_cap = max(1, T // r)
        self.p = B.make_params(
            batch=batch, total_tokens=T, max_seqlen=max_seqlen, ratio=r, window=cfg.window,
            topk=max(1, cfg.topk), topk_cap=cfg.topk_cap, heads=H, head_dim=D,
            idx_heads=cfg.idx_heads, idx_dim=cfg.idx_dim, scale=cfg.scale, mode=MODE[cfg.mode],
            teacher=TEACHER[cfg.teacher], dtype=DTYPE[cfg.dtype],
            idx_dtype=DTYPE[cfg.idx_dtype] if cfg.idx_heads else B.CSA_BF16,
            rope_dim=cfg.rope_dim, rope_theta=cfg.rope_theta)
        z = lambda *s, dtype=torch.float32: torch.empty(*s, dtype=dtype, device=device)  # noqa
        self.cu_cmp = z(batch + 1, dtype=torch.int32)
        self.kv_cmp = z(self.tc_cap, D, dtype=dt)
        self.out = z(T, H, D, dtype=dt)
        self.rope = cfg.rope_dim > 0
        if self.rope:
            self.out_rot = z(T, H, D, dtype=dt)
            self.kv_rot = z(T, D, dtype=dt)
        self.lse = z(T, H)
        # selected-set teacher: the forward also returns the compressed-only normalizer
        self.lse_cmp = z(T, H) if (cfg.has_indexer and cfg.teacher == "selected") else None
        self.ws_fwd = self._ws(B.CSA_OP_ATTN_FWD, device)
        self.t_logits = None
        if cfg.has_indexer:
            HI, dI = cfg.idx_heads, cfg.idx_dim
            idt = torch.float32 if cfg.idx_dtype == "f32" else torch.bfloat16
            self.kI_cmp = z(self.tc_cap, dI, dtype=idt)
            if cfg.idx_dtype == "fp8":
                self.qI8 = z(T, HI, dI, dtype=torch.uint8)
                self.qI_scale = z(T, HI)
                self.kI8 = z(self.tc_cap, dI, dtype=torch.uint8)
                self.kI_scale = z(self.tc_cap)
            self._scores = None      # [T, n_cap] fp32, allocated only where a call needs it
            self._device = device
            self.idx = z(T, cfg.topk_cap, dtype=torch.int32)
            # the dense-teacher loss can form the student scores itself: with the fused
            # selection the step then needs no [T, n_cap] score matrix at all
            self.kl_recompute = (cfg.teacher == "dense" and
                                 B.csa_workspace_size(self.p, B.CSA_OP_INDEXER_KL) > 0)
            if cfg.teacher != "none":
                self.kl = z(T)
                self.loss = z(1)
                # teacher-logit cache: the forward keeps the compressed-candidate logits it
                # forms anyway and the loss reads them instead of gathering the rows again;
                # used where the library has a kernel for it (nonzero cached workspace)
                n_cached = B.csa_workspace_size(self.p, B.CSA_OP_INDEXER_KL_CACHED)
                if n_cached > 0 and backward:
                    ld_t = B.csa_teacher_logits_stride(self.p)
                    self.t_logits = z(T, H, ld_t)
                    self.ws_kl = self._ws(B.CSA_OP_INDEXER_KL_CACHED, device)
                else:
                    self.ws_kl = self._ws(B.CSA_OP_INDEXER_KL, device)
                if backward:
                    self.dqI = z(T, HI, dI)
                    self.dw = z(T, HI)
                    self.dkI_cmp = z(self.tc_cap, dI)
                    self.dkI_tok = z(T, dI)
        if backward:
            self.dq = z(T, H, D, dtype=dt)
            self.dkv_cmp = z(self.tc_cap, D)
            self.dkv = z(T, D)
            self.dsink = z(H)
            self.ws_bwd = self._ws(B.CSA_OP_ATTN_BWD, device, cap=bwd_ws_bytes)

    @property
    def scores(self):
        if self._scores is None:
            self._scores = torch.empty(self.T, max(1, self.n_cap), dtype=torch.float32,
                                       device=self._device)
        return self._scores

    def _ws(self, op, device, cap=None):
        n = B.csa_workspace_size(self.p, op)
        if n and cap is not None:
            n = max(min(n, int(cap)), B.csa_workspace_size_min(self.p, op))
        return torch.empty(max(n, 1), dtype=torch.uint8, device=device) if n else None

    # ------------------------------------------------------------------ steps
    def _call(self, name, fn, *args):
        if self.timer is not None:
            self.timer.mark(name)
        fn(*args)
        if self.timer is not None:
            self.timer.done(name)

    def metadata(self, cu_seqlens):
        self._call("cmp_seqlens", B.csa_cmp_seqlens, cu_seqlens, self.B, self.cfg.ratio,
                   self.cu_cmp)

    def _rope(self, name, x, offsets, inverse, out=None):
        self._call(name, B.csa_rope, x, x if out is None else out, self.cfg.rope_dim,
                   self.cfg.rope_theta, inverse, self.B, offsets)

    def forward(self, inp, cu_seqlens):
        """inp: dict of device tensors q, kv, [qI, kI_tok, w], [sink].  Forms the compressed
        offsets of cu_seqlens first: every later call indexes rows through them."""
        cfg, p = self.cfg, self.p
        self.metadata(cu_seqlens)
        self._call("compress_kv", B.csa_compress, p, inp["kv"], cu_seqlens, self.cu_cmp,
                   self.kv_cmp)
        kv = inp["kv"]
        if self.rope:
            self._rope("rope_kv_cmp", self.kv_cmp, self.cu_cmp, 0)
            self._rope("rope_kv", inp["kv"], cu_seqlens, 0, out=self.kv_rot)
            self._rope("rope_q", inp["q"], cu_seqlens, 0)
            kv = self.kv_rot
        idx = None
        if cfg.has_indexer:
            self._call("compress_kI", B.csa_compress, p, inp["kI_tok"], cu_seqlens, self.cu_cmp,
                       self.kI_cmp)
            if self.rope:
                self._rope("rope_kI_cmp", self.kI_cmp, self.cu_cmp, 0)
                self._rope("rope_qI", inp["qI"], cu_seqlens, 0)
            if cfg.idx_dtype == "fp8":
                self._call("quantize_qI", B.csa_quantize_fp8, inp["qI"], self.qI8, self.qI_scale)
                self._call("quantize_kI", B.csa_quantize_fp8, self.kI_cmp, self.kI8, self.kI_scale)
                qI, qs, kI, ks = self.qI8, self.qI_scale, self.kI8, self.kI_scale
            else:
                qI, qs, kI, ks = inp["qI"], None, self.kI_cmp, None
            if self.fused_topk is not False:
                # one pass: the selection never materializes the full score matrix; the
                # loss reads scores only where its teacher does (a dense teacher that forms
                # them itself needs none)
                mode = {"none": 0, "selected": 1,
                        "dense": 0 if self.kl_recompute else 2}[cfg.teacher]
                try:
                    self._call("index_topk", B.csa_index_topk, p, qI, qs, inp["w"], kI, ks,
                               cu_seqlens, self.cu_cmp, self.idx,
                               self.scores if mode else None, mode)
                    self.fused_topk = True
                except B.CsaError as e:
                    if self.fused_topk or e.status != B.CSA_ERR_UNSUPPORTED:
                        raise
                    self.fused_topk = False      # no fused kernel for this shape
            if not self.fused_topk:
                self._call("index_scores", B.csa_index_scores, p, qI, qs, inp["w"], kI, ks,
                           cu_seqlens, self.cu_cmp, self.scores)
                self._call("topk_select", B.csa_topk_select, p, self.scores, cu_seqlens,
                           self.cu_cmp, self.idx)
            idx = self.idx
        self._call("attn_fwd", B.csa_sparse_attn_fwd, p, inp["q"], self.kv_cmp, kv, idx,
                   inp.get("sink"), cu_seqlens, self.cu_cmp, self.out, self.lse, self.lse_cmp,
                   self.ws_fwd, None, self.t_logits, self.out_rot if self.rope else None)
        if cfg.has_indexer and cfg.teacher != "none":
            grads = self.backward
            if grads:
                self.dkI_cmp.zero_()
            scores = self._scores if (cfg.teacher != "dense" or not self.kl_recompute or
                                      not self.fused_topk) else None
            self._call("indexer_kl", B.csa_indexer_kl, p, inp["q"], self.kv_cmp, scores,
                       self.idx, qI, qs, inp["w"], kI, ks, cu_seqlens, self.cu_cmp,
                       self.grad_scale, self.kl, self.loss, self.dqI if grads else None,
                       self.dw if grads else None, self.dkI_cmp if grads else None, self.ws_kl,
                       self.lse_cmp, None, self.t_logits)
            if grads and self.rope:
                self._rope("rope_dqI", self.dqI, cu_seqlens, 1)

    def backward_step(self, inp, cu_seqlens):
        cfg, p = self.cfg, self.p
        self.dkv_cmp.zero_()
        self.dkv.zero_()
        sink = inp.get("sink")
        if sink is not None:
            self.dsink.zero_()
        if self.rope:
            # the incoming gradient is that of out_rot: rotate it to the gradient of out
            self._rope("rope_dO", inp["dO"], cu_seqlens, 0)
        self._call("attn_bwd", B.csa_sparse_attn_bwd, p, inp["q"], self.kv_cmp,
                   self.kv_rot if self.rope else inp["kv"],
                   self.idx if cfg.has_indexer else None, sink, cu_seqlens, self.cu_cmp, self.out,
                   self.lse, inp["dO"], self.dq, self.dkv_cmp, self.dkv,
                   self.dsink if sink is not None else None, self.ws_bwd)
        if self.rope:
            self._rope("rope_dq", self.dq, cu_seqlens, 1)
            self._rope("rope_dkv", self.dkv, cu_seqlens, 1)
            self._rope("rope_dkv_cmp", self.dkv_cmp, self.cu_cmp, 1)
        self._call("compress_bwd_kv", B.csa_compress_bwd, p, self.dkv_cmp, cu_seqlens,
                   self.cu_cmp, self.dkv)
        if cfg.has_indexer and cfg.teacher != "none":
            self.dkI_tok.zero_()
            if self.rope:
                self._rope("rope_dkI_cmp", self.dkI_cmp, self.cu_cmp, 1)
            self._call("compress_bwd_kI", B.csa_compress_bwd, p, self.dkI_cmp, cu_seqlens,
                       self.cu_cmp, self.dkI_tok)

    def step(self, inp, cu_seqlens):
        self.forward(inp, cu_seqlens)
        if self.backward:
            self.backward_step(inp, cu_seqlens)


def to_device(host, device="cuda", keys=("q", "kv", "qI", "kI_tok", "w", "dO", "sink")):
    """Copy the seeded host tensors of a workload to the device."""
    out = {k: host[k].to(device) for k in keys if k in host}
    out["cu_seqlens"] = torch.tensor(host["cu_seqlens"], dtype=torch.int32, device=device)
    return out
