"""Seeded synthetic inputs for a workload.

Recipe (the same bytes go to the CPU oracle and to the GPU):
  * every tensor has its own stream: chunk c of tensor `tid` of workload
    `cfg_id`, variant `v`, is drawn from
    numpy default_rng(SeedSequence([cfg_id, tid, v, c])) as float32 standard
    normals, CHUNK elements per chunk, in row-major order;
  * the chunk is multiplied in float32 by the tensor's standard deviation
    (1 for "unit" workloads, 1/sqrt(last dim) for "inv_sqrt_d" workloads,
    1/sqrt(H_I) for the indexer head weights) and rounded once to the storage
    dtype (float32, or bfloat16 with round-to-nearest-even via torch);
  * capacity rows beyond the last sample (t >= cu_seqlens[B]) are filled with
    NaN so that any read of them as a key or a query shows up in the results.
Tensor ids: q=1, kv=2, qI=3, kI_tok=4, w=5, dO=6, lengths=7, sink=8.
Chunks are independent streams, so they are drawn in a thread pool.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .configs import Workload

CHUNK = 1 << 22
TID = {"q": 1, "kv": 2, "qI": 3, "kI_tok": 4, "w": 5, "dO": 6, "lengths": 7, "sink": 8}
_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.bfloat16}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_lengths(w: Workload, variant: int = 0):
    """Sample lengths of the packed batch.

    Fixed lengths are returned as given.  A drawn workload takes n-1 lengths
    uniformly from {lo..hi} and sets the last one to total - sum, redrawing
    until the last one is also in [lo, hi].  Lengths not divisible by the
    compression ratio are kept (their tails are part of the workload).
    """
    if w.lengths is not None:
        return [int(x) for x in w.lengths]
    d = w.draw
    rng = np.random.default_rng(np.random.SeedSequence([w.cfg_id, TID["lengths"], variant]))
    while True:
        head = rng.integers(d["lo"], d["hi"] + 1, size=d["n"] - 1)
        last = d["total"] - int(head.sum())
        if d["lo"] <= last <= d["hi"]:
            return [int(x) for x in head] + [int(last)]


def _fill(out_flat: torch.Tensor, cfg_id: int, tid: int, variant: int, std: float):
    n = out_flat.numel()
    nchunks = (n + CHUNK - 1) // CHUNK
    std32 = np.float32(std)

    def one(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([cfg_id, tid, variant, c]))
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if std32 != np.float32(1.0):
            v *= std32
        out_flat[lo:hi] = torch.from_numpy(v).to(out_flat.dtype)

    if nchunks == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunks)))


def _tensor(shape, dtype, cfg_id, name, variant, std, n_real_rows):
    t = torch.empty(shape, dtype=dtype)
    _fill(t.view(-1), cfg_id, TID[name], variant, std)
    if n_real_rows < shape[0]:
        t[n_real_rows:] = float("nan")
    return t


def make_inputs(w: Workload, variant: int = 0, strength: bool = False, lengths=None,
                want=("q", "kv", "qI", "kI_tok", "w", "dO", "sink")):
    """Build the seeded host inputs of a workload.

    Returns a dict of CPU torch tensors in their storage dtype plus metadata:
      lengths (list), cu_seqlens (int32 numpy, B+1), max_seqlen (int),
      q [T,H,D], kv [T,D], and if the layer has an indexer qI [T,H_I,d_I],
      kI_tok [T,d_I], w [T,H_I]; dO [T,H,D] if it has a backward; sink [H].
    `strength=True` draws every tensor at unit variance (larger logits, a
    sharper softmax) instead of the workload's 1/sqrt(d) scaling.
    """
    lens = [int(x) for x in (lengths if lengths is not None else draw_lengths(w, variant))]
    if sum(lens) > w.total_tokens:
        raise ValueError("sample lengths exceed the capacity of the packed batch")
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = w.total_tokens
    n_real = int(cu[-1])
    dt = _TORCH_DTYPE[w.dtype]
    idt = _TORCH_DTYPE[w.idx_dtype]

    def std(last_dim):
        if strength or w.input_std == "unit":
            return 1.0
        return 1.0 / float(last_dim) ** 0.5

    out = {"lengths": lens, "cu_seqlens": cu, "max_seqlen": max(lens) if lens else 0,
           "variant": variant, "strength": strength}
    if "q" in want:
        out["q"] = _tensor((T, w.heads, w.head_dim), dt, w.cfg_id, "q", variant, std(w.head_dim), n_real)
    if "kv" in want:
        out["kv"] = _tensor((T, w.head_dim), dt, w.cfg_id, "kv", variant, std(w.head_dim), n_real)
    if w.has_indexer:
        if "qI" in want:
            out["qI"] = _tensor((T, w.idx_heads, w.idx_dim), idt, w.cfg_id, "qI", variant,
                                std(w.idx_dim), n_real)
        if "kI_tok" in want:
            out["kI_tok"] = _tensor((T, w.idx_dim), idt, w.cfg_id, "kI_tok", variant, std(w.idx_dim), n_real)
        if "w" in want:
            # head weights are produced in fp32 by the caller's projection
            out["w"] = _tensor((T, w.idx_heads), torch.float32, w.cfg_id, "w", variant,
                               std(w.idx_heads), n_real)
    if w.backward and "dO" in want:
        out["dO"] = _tensor((T, w.heads, w.head_dim), dt, w.cfg_id, "dO", variant, std(w.head_dim), n_real)
    if w.sink and "sink" in want:
        out["sink"] = _tensor((w.heads,), torch.float32, w.cfg_id, "sink", variant, 1.0, w.heads)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a host tensor (bf16/fp32 values are exact in fp64)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
