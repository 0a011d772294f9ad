"""Workload table: the five layer configurations the path is measured and checked on.

Each workload is a packed THD batch (tokens of all samples concatenated on one
axis, delimited by cu_seqlens) with the layer hyper-parameters of one
DeepSeek-V4 attention layer type.  The shapes follow the page "DeepSeek-V4
Attention Training Systems": ratio-4 CSA with a lightning indexer and ratio-128
HCA without one (section 2, phase table), a 128-token local window and
512-wide shared KV (section 5.1 and the section 5.5 storage estimate), and a
128-wide indexer key (section 5.5).
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int                      # seed namespace (1..5 for the five layer configs)
    lengths: Optional[Tuple[int, ...]]   # fixed sample lengths, or None => drawn (see draw_lengths)
    total_tokens: int                # capacity rows T of the packed batch
    heads: int                       # H query heads
    head_dim: int                    # D, shared K=V width
    ratio: int                       # r, tokens per compressed entry
    window: int                      # W, local raw-KV window (includes the query token)
    topk: int                        # k selected compressed entries per query (CSA sparse)
    topk_cap: int                    # k rounded up to the kernel alignment (64)
    idx_heads: int                   # H_I indexer heads (0 => no indexer, HCA)
    idx_dim: int                     # d_I indexer width
    dtype: str                       # "f32" | "bf16" main operands
    idx_dtype: str                   # "f32" | "bf16" | "fp8" indexer operands
    mode: str                        # "sparse" (top-k) | "dense" (every visible entry)
    teacher: str                     # "none" | "selected" | "dense" KL teacher set
    backward: bool                   # whether the layer step includes backward
    input_std: str                   # "unit" => N(0,1); "inv_sqrt_d" => N(0,1)/sqrt(last dim)
    sink: bool = False               # optional per-head attention sink logit
    rope_dim: int = 0                # rotary band: last rope_dim channels of q/kv/qI/kI rows
    rope_theta: float = 10000.0      # rotary base
    draw: Optional[dict] = field(default=None, compare=False)   # length-draw rule

    @property
    def scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5

    @property
    def has_indexer(self) -> bool:
        return self.idx_heads > 0


WORKLOADS = {
    # tiny fp32 CSA, one 256-token sequence, dense KL teacher (warm-up phase)
    "tiny_csa_f32_L256": Workload(
        name="tiny_csa_f32_L256", cfg_id=1, lengths=(256,), total_tokens=256,
        heads=4, head_dim=64, ratio=4, window=16, topk=16, topk_cap=64,
        idx_heads=2, idx_dim=32, dtype="f32", idx_dtype="f32",
        mode="sparse", teacher="dense", backward=True, input_std="unit"),
    # CSA sparse forward, bf16, one 4096-token sequence
    "csa_sparse_fwd_bf16_L4096": Workload(
        name="csa_sparse_fwd_bf16_L4096", cfg_id=2, lengths=(4096,), total_tokens=4096,
        heads=64, head_dim=512, ratio=4, window=128, topk=512, topk_cap=512,
        idx_heads=64, idx_dim=128, dtype="bf16", idx_dtype="bf16",
        mode="sparse", teacher="none", backward=False, input_std="inv_sqrt_d"),
    # packed THD varlen CSA fwd+bwd, 8 ragged samples summing to 65536 tokens,
    # selected-set KL teacher (sparse-loss phase) -- the 64K THD layer step
    "thd64k_csa_bf16": Workload(
        name="thd64k_csa_bf16", cfg_id=3, lengths=None, total_tokens=65536,
        heads=64, head_dim=512, ratio=4, window=128, topk=1024, topk_cap=1024,
        idx_heads=64, idx_dim=128, dtype="bf16", idx_dtype="bf16",
        mode="sparse", teacher="selected", backward=True, input_std="inv_sqrt_d",
        draw={"n": 8, "lo": 1024, "hi": 16384, "total": 65536}),
    # the same layer step with a per-head attention sink logit
    "thd64k_csa_sink_bf16": Workload(
        name="thd64k_csa_sink_bf16", cfg_id=3, lengths=None, total_tokens=65536,
        heads=64, head_dim=512, ratio=4, window=128, topk=1024, topk_cap=1024,
        idx_heads=64, idx_dim=128, dtype="bf16", idx_dtype="bf16",
        mode="sparse", teacher="selected", backward=True, input_std="inv_sqrt_d", sink=True,
        draw={"n": 8, "lo": 1024, "hi": 16384, "total": 65536}),
    # the same layer step with the positional rotations: a 64-channel rotary band of the
    # 512-wide rows and of the 128-wide indexer rows, output inverse-rotated
    "thd64k_csa_rope_bf16": Workload(
        name="thd64k_csa_rope_bf16", cfg_id=3, lengths=None, total_tokens=65536,
        heads=64, head_dim=512, ratio=4, window=128, topk=1024, topk_cap=1024,
        idx_heads=64, idx_dim=128, dtype="bf16", idx_dtype="bf16",
        mode="sparse", teacher="selected", backward=True, input_std="inv_sqrt_d",
        rope_dim=64, draw={"n": 8, "lo": 1024, "hi": 16384, "total": 65536}),
    # window-only layer (no compressed history) on the same 64K THD batch as above
    "thd64k_window_bf16": Workload(
        name="thd64k_window_bf16", cfg_id=3, lengths=None, total_tokens=65536,
        heads=64, head_dim=512, ratio=4, window=128, topk=0, topk_cap=0,
        idx_heads=0, idx_dim=0, dtype="bf16", idx_dtype="bf16",
        mode="window", teacher="none", backward=True, input_std="inv_sqrt_d",
        draw={"n": 8, "lo": 1024, "hi": 16384, "total": 65536}),
    # dense mode at ratio 4 on the same 64K THD batch: every visible compressed entry plus
    # the window, no indexer (the dense phase of the curriculum, section 2)
    "thd64k_dense_bf16": Workload(
        name="thd64k_dense_bf16", cfg_id=3, lengths=None, total_tokens=65536,
        heads=64, head_dim=512, ratio=4, window=128, topk=0, topk_cap=0,
        idx_heads=0, idx_dim=0, dtype="bf16", idx_dtype="bf16",
        mode="dense", teacher="none", backward=True, input_std="inv_sqrt_d",
        draw={"n": 8, "lo": 1024, "hi": 16384, "total": 65536}),
    # HCA: ratio 128, no indexer, every completed entry + window, 4 x 16384
    "thd64k_hca_bf16": Workload(
        name="thd64k_hca_bf16", cfg_id=4, lengths=(16384,) * 4, total_tokens=65536,
        heads=64, head_dim=512, ratio=128, window=128, topk=0, topk_cap=0,
        idx_heads=0, idx_dim=0, dtype="bf16", idx_dtype="bf16",
        mode="dense", teacher="none", backward=True, input_std="inv_sqrt_d"),
    # long-context CSA sparse warm-up: 131072 tokens, fp8 indexer, dense teacher
    "csa128k_warmup_fp8": Workload(
        name="csa128k_warmup_fp8", cfg_id=5, lengths=(131072,), total_tokens=131072,
        heads=64, head_dim=512, ratio=4, window=128, topk=2048, topk_cap=2048,
        idx_heads=64, idx_dim=128, dtype="bf16", idx_dtype="fp8",
        mode="sparse", teacher="dense", backward=True, input_std="inv_sqrt_d"),
}


def workload(name: str, **overrides) -> Workload:
    """Look up a workload, optionally overriding fields (for reduced instances)."""
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w
