#!/usr/bin/env python3
"""Throughput of one CSA/HCA attention-layer step (forward + backward) on one MI355X.

A step is one pass of the whole hot path over one packed THD batch of synthetic
input (seeded, resident in HBM before timing): compressor (main KV and indexer key),
[fp8 quantization], indexer scores, top-k, sparse attention forward, indexer KL with
its eager backward, sparse attention backward and the compressor adjoints.
Default workload: 8 ragged samples summing to 65536 tokens, ratio-4 CSA, 64 heads,
KV width 512, top-k 1024, window 128, selected-set KL teacher.

Prints ONE JSON line.  Every ABI call is bracketed by HIP events on the stream it runs
on, so the line also carries a per-call breakdown and the roofline of the dominant
kernel; the fp64 CPU oracle is timed on a bounded sample of query rows for the CPU
baseline (rank 0, N = 1 only).
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synth import configs, inputs  # noqa: E402

PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "f32": 157.3e12, "hbm": 8.0e12}
METRIC = "CSA fwd+bwd tokens/s at L=64K THD (with TFLOP/s, % MFMA peak, top-k GB/s)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="thd64k_csa_bf16", choices=sorted(configs.WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-workspace-gib", type=float, default=None,
                    help="cap the attention backward's workspace (more query chunks)")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the matrix-core loop and copy that measure the device's peaks")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print the per-kernel summary of a 'rocprofv3 --kernel-trace' run of "
                         "bench.py (files run_kernel_trace.csv) and exit: dispatches before the "
                         "trace marker are the layer steps, after it the stand-alone timings")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="print per-kernel matrix-core and LDS counters of a 'rocprofv3 --pmc "
                         "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                         "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_BUSY_CYCLES GRBM_GUI_ACTIVE' "
                         "run of bench.py and exit")
    ap.add_argument("--traced-steps", type=int, default=0,
                    help="steps (warm-up + timed) in the traced run, for per-step figures")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="also run one plain device-to-device copy of this many bytes before "
                         "the timed steps (a known-traffic reference for HBM counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the per-call HBM traffic summary of two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of 'bench.py --steps 1 --warmup 0 "
                         "--copy-bytes N' and exit")
    return ap.parse_args()


# kernels of each multi-kernel ABI call, by the demangled name prefix rocprofv3 reports
CALL_KERNELS = {
    "attn_bwd": ("k_attn_bwd_dq_mfma", "k_attn_bwd_keys", "k_attn_bwd_keys_dups",
                 "k_attn_bwd_dkv_mfma", "k_bwd_fill_zero", "k_bwd_csr_pass", "k_bwd_csr_scan",
                 "k_bwd_reduce_cmp", "k_bwd_reduce_win", "k_attn_bwd_generic"),
    "attn_fwd": ("k_attn_fwd_mfma", "k_attn_fwd_generic"),
    "indexer_kl": ("k_kl_cached", "k_kl_keys", "k_fill_zero_i32", "k_indexer_kl_mfma", "k_kl_generic", "k_sum", "k_kld_teacher",
                   "k_kld_queries", "k_kld_keys", "k_kld_dequant"),
    "index_topk": ("k_index_topk",),
    "index_scores": ("k_index_scores_mfma", "k_index_scores_generic"),
    "topk_select": ("k_topk_wave", "k_topk_wg"),
    "compress_learned (kv + kI)": ("k_compress_learned",),
    "compress_learned_bwd (kv + kI)": ("k_compress_learned_bwd",),
    "quantize": ("k_quantize_fp8",),
    "compress (kv + kI)": ("k_compress",),
    "compress_bwd (kv + kI)": ("k_compress_bwd",),
    "rope (all operands)": ("k_rope",),
}
# kernels launched by more than one call (the key-major planner and partial-sum reduction of the
# attention backward and the indexer loss): each dispatch belongs to the call whose own kernel
# was dispatched last before it (both calls open with a fill kernel of their own)
SHARED_KERNELS = ("k_attn_bwd_keys_plan", "k_attn_bwd_keys_reduce")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "thd64k_csa_bf16_traffic.md")


def source_hash():
    """Hash of the kernel sources: traffic counters taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_compressed_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _pmc_rows(d):
    import csv
    path = os.path.join(d, "run_counter_collection.csv")
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
            name = name.split("(")[0].replace("void ", "")
            name = name.split("::")[-1].split("<")[0]
            out.append((int(r["Dispatch_Id"]), name, r["Counter_Name"], float(r["Counter_Value"])))
    return out


def summarize_counters(d, steps):
    """Per kernel (dispatches of the traced steps summed).  GRBM_GUI_ACTIVE sums the cycle
    counters of the 8 XCDs (8x the kernel's duration in cycles), SQ_VALU_MFMA_BUSY_CYCLES the
    1024 SIMDs' busy cycles and SQ_LDS_* the 256 CUs' cycles, so: matrix-core busy =
    MFMA_BUSY / (GUI / 8 x 1024); bf16 matrix FLOP issued = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512;
    LDS bank-conflict share of the kernel's cycles = BANK_CONFLICT / 256 / (GUI / 8), and of the
    LDS-active cycles = BANK_CONFLICT / LDS_IDX_ACTIVE."""
    rows = _pmc_rows(d)
    per = {}
    for disp, name, cname, v in rows:
        per.setdefault(name, {}).setdefault(cname, {})[disp] = v
    print("| Kernel | Dispatches | MFMA busy | bf16 MFMA TFLOP per step | LDS bank conflicts, of kernel cycles | of LDS-active cycles |")
    print("| --- | --- | --- | --- | --- | --- |")
    out = []
    for name, cs in per.items():
        disp = set().union(*[set(x) for x in cs.values()])
        tot = {c: sum(x.values()) for c, x in cs.items()}
        gui = tot.get("GRBM_GUI_ACTIVE", 0.0)
        busy = tot.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        mops = tot.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        lds = tot.get("SQ_LDS_IDX_ACTIVE", 0.0)
        conf = tot.get("SQ_LDS_BANK_CONFLICT", 0.0)
        cyc = gui / 8.0
        out.append((gui, name, len(disp), busy / (cyc * 1024) if gui else 0.0,
                    mops * 512 / max(steps, 1) / 1e12, conf / 256 / cyc if gui else 0.0,
                    conf / lds if lds else 0.0))
    for gui, name, nd, util, tf, lk, lc in sorted(out, reverse=True):
        if name.startswith("k_mfma_") or name.startswith("k_trace_marker") or gui == 0:
            continue
        if not name.startswith("k_"):
            continue
        print(f"| {name} | {nd} | {100 * util:.1f} % | {tf:.3f} | {100 * lk:.1f} % | "
              f"{100 * lc:.1f} % |")


def summarize_pmc(fetch_dir, write_dir, copy_bytes):
    """Per-call HBM bytes of one step: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for the plain copy of copy_bytes bytes."""
    res = {}
    for label, d, cname in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = [r for r in _pmc_rows(d) if r[2] == cname]
        copies = [v for _, n, _, v in rows if "copyBuffer" in n]
        factor = copy_bytes / (max(copies) * 1024.0)
        per_call = {}
        current = None
        for _, n, _, v in sorted(rows):
            call = next((c for c, ks in CALL_KERNELS.items() if n in ks), None)
            if call is not None:
                current = call
            elif n in SHARED_KERNELS:
                call = current
            if call is not None:
                per_call[call] = per_call.get(call, 0.0) + v * 1024.0 * factor
        res[label] = {"factor": factor, "copy_kib": max(copies), "per_call_bytes": per_call}
    return res


def _kernel_short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    base = name.split("(")[0]
    short = base.split("::")[-1] if "<" not in base else base.split("<")[0].split("::")[-1] + \
        "<" + base.split("<", 1)[1]
    return short.replace("csa::", "")


def summarize_trace(d, steps):
    """Per-kernel calls, mean duration and per-step time of a kernel trace of bench.py; the
    dispatches after the k_trace_marker kernel (the stand-alone timings) are listed apart."""
    import csv
    rows = []
    with open(os.path.join(d, "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                         _kernel_short(r["Kernel_Name"])))
    rows.sort()
    cut = next((i for i, r in enumerate(rows) if r[2].startswith("k_trace_marker")), len(rows))
    first_step = next((i for i, r in enumerate(rows) if r[2].startswith("k_cmp_seqlens")), 0)
    parts = [("", rows[first_step:cut]), (" (stand-alone, after the steps)", rows[cut + 1:])]
    step_total = sum(e - b for b, e, _ in parts[0][1])
    print("| Kernel | Calls | Average (us) | Per step (ms) | Share |")
    print("| --- | --- | --- | --- | --- |")
    for tag, rs in parts:
        agg = {}
        for b, e, n in rs:
            c, t = agg.get(n, (0, 0))
            agg[n] = (c + 1, t + (e - b))
        for n, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
            if n.startswith("k_mfma_") or n.startswith("k_trace_marker"):
                continue
            per_step = f"{t / max(steps, 1) / 1e6:.2f}" if not tag and steps else "—"
            share = f"{100.0 * t / step_total:.2f} %" if not tag and step_total else "—"
            print(f"| {n}{tag} | {c} | {t / c / 1e3:.1f} | {per_step} | {share} |")
    if steps:
        print()
        print(f"Sum of the step kernels: {step_total / max(steps, 1) / 1e6:.2f} ms per step "
              f"({steps} steps traced).")


def load_traffic():
    """Per-call HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(blob)
    except Exception:
        return None
    if data.get("source_hash") != source_hash():
        return None
    return data.get("per_call_bytes")


def measured_peaks():
    """Peaks measured on this device: a loop of independent matrix-core operations on every
    SIMD (bf16 16x16x32 and fp8 16x16x128, 8 accumulation chains per wave, 4 waves per SIMD)
    and a device-to-device copy of 4 GiB (bytes read + written over its time)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_compressed_amd", "libcsa_probe.so"))
    lib.csa_probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
    lib.csa_probe_mfma_loop.restype = ctypes.c_int
    blocks, iters = 1024, 1000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, fp8, flop in (("bf16", 0, 16384), ("fp8", 1, 65536)):
        def run():
            rc = lib.csa_probe_mfma_loop(fp8, out.data_ptr(), blocks, iters, stream)
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
        run()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) * 1e-3)
        res[f"{name}_tflops"] = round(blocks * 4 * iters * 8 * flop / best / 1e12, 1)
    n = 1 << 30                        # 4 GiB of fp32
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    res["hbm_gbps"] = round(2 * 4 * n / best / 1e9, 1)
    del src, dst, out
    torch.cuda.empty_cache()
    return res


class EventTimer:
    """HIP events around each ABI call, on torch's current stream (the library's stream)."""

    def __init__(self):
        self.open = {}
        self.pairs = {}

    def mark(self, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.open[name] = e

    def done(self, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(name, []).append((self.open.pop(name), e))

    def mean_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.pairs.items()}


def work_counts(w, lengths):
    """Per-step algorithmic work from the packed lengths (no device data needed)."""
    r, W, k = w.ratio, w.window, w.topk
    cand = 0          # sum_t |X_t|: attended rows per query (compressed + window)
    vis = 0           # sum_t n_vis(t)
    vis_read = 0      # visible scores top-k must read (rows with n_vis > k)
    sel = 0           # sum_t |S_t| (or all visible in dense mode)
    tcmp = 0
    for L in lengths:
        p = np.arange(L, dtype=np.int64)
        nv = (p + 1) // r
        win = np.minimum(W, p + 1)
        if w.mode == "sparse":
            s = np.minimum(k, nv)
        elif w.mode == "dense":
            s = nv
        else:
            s = np.zeros_like(nv)
        cand += int((s + win).sum())
        vis += int(nv.sum())
        vis_read += int(nv[nv > k].sum()) if w.mode == "sparse" else 0
        sel += int(s.sum())
        tcmp += L // r
    return dict(cand=cand, vis=vis, vis_read=vis_read, sel=sel, tcmp=tcmp,
                tokens=int(sum(lengths)))


def roofline_table(w, c, T, kl_cached=False):
    """(bound, algorithmic amount per launch, unit, peak) per ABI call.

    The indexer loss reading the forward's cached teacher logits computes no teacher
    logits: it is priced against HBM on the bytes it cannot avoid (each (query, candidate)
    pair's 64 cached logits and its score once, qI read and dqI / dw written once per query,
    the indexer keys read and their gradient written once)."""
    H, D, HI, dI = w.heads, w.head_dim, w.idx_heads, w.idx_dim
    e = 4 if w.dtype == "f32" else 2
    ei = 1 if w.idx_dtype == "fp8" else (4 if w.idx_dtype == "f32" else 2)
    mm = "bf16" if w.dtype == "bf16" else "f32"
    teach = c["vis"] if w.teacher == "dense" else c["sel"]
    kl_flops = 2 * D * H * teach * (2 if w.teacher == "dense" else 1) + 4 * dI * HI * teach
    kl_entry = (mm, kl_flops)
    if kl_cached:
        kl_entry = ("hbm", teach * (4 * H + 4) + c["tokens"] * (HI * dI * (ei + 4) + HI * 8 + H * 4)
                    + c["tcmp"] * dI * (ei + 4))
    tab = {
        "compress_kv": ("hbm", c["tokens"] * D * e + c["tcmp"] * D * e),
        "compress_kI": ("hbm", c["tokens"] * dI * 2 + c["tcmp"] * dI * 2),
        "quantize_qI": ("hbm", c["tokens"] * HI * dI * (2 + 1) + c["tokens"] * HI * 4),
        "quantize_kI": ("hbm", c["tcmp"] * dI * (2 + 1) + c["tcmp"] * 4),
        "index_scores": ("fp8" if w.idx_dtype == "fp8" else mm, 2 * dI * HI * c["vis"]),
        # fused scores + top-k: the score products dominate (every visible entry is scored
        # when the loss reads scores; rows with n_vis <= k skip them otherwise)
        "index_topk": ("fp8" if w.idx_dtype == "fp8" else mm,
                       2 * dI * HI * (c["vis"] if w.teacher != "none" else c["vis_read"])),
        "topk_select": ("hbm", 4 * c["vis_read"] + 4 * T * max(w.topk_cap, 1)),
        "attn_fwd": (mm, 4 * D * H * c["cand"]),
        "indexer_kl": kl_entry,
        "attn_bwd": (mm, 10 * D * H * c["cand"]),
        "compress_bwd_kv": ("hbm", c["tcmp"] * D * 4 + 2 * c["tcmp"] * w.ratio * D * 4),
        "compress_bwd_kI": ("hbm", c["tcmp"] * dI * 4 + 2 * c["tcmp"] * w.ratio * dI * 4),
        # learned-score compressor: value and score rows read once, compressed rows written;
        # adjoint: value/score rows and d_x_cmp read, dx and dscore read-modify-written
        "compress_learned_kv": ("hbm", 2 * c["tokens"] * D * e + c["tcmp"] * D * e),
        "compress_learned_bwd_kv": ("hbm", 2 * c["tokens"] * D * e + c["tcmp"] * D * 4 +
                                    4 * c["tcmp"] * w.ratio * D * 4),
        "compress_learned_kI": ("hbm", 2 * c["tokens"] * dI * 2 + c["tcmp"] * dI * 2),
        "compress_learned_bwd_kI": ("hbm", 2 * c["tokens"] * dI * 2 + c["tcmp"] * dI * 4 +
                                    4 * c["tcmp"] * w.ratio * dI * 4),
    }
    # rotary band: in place the band of each row is read and written; the window rows of kv
    # are rotated into a buffer of their own (every channel read and written)
    rd = getattr(w, "rope_dim", 0)
    if rd:
        n, m = c["tokens"], c["tcmp"]
        ei = 4 if w.idx_dtype == "f32" else 2          # rotated before any fp8 quantization
        tab.update({
            "rope_q": ("hbm", 2 * n * H * rd * e), "rope_dO": ("hbm", 2 * n * H * rd * e),
            "rope_dq": ("hbm", 2 * n * H * rd * e), "rope_kv": ("hbm", 2 * n * D * e),
            "rope_kv_cmp": ("hbm", 2 * m * rd * e), "rope_qI": ("hbm", 2 * n * HI * rd * ei),
            "rope_kI_cmp": ("hbm", 2 * m * rd * ei), "rope_dqI": ("hbm", 2 * n * HI * rd * 4),
            "rope_dkv": ("hbm", 2 * n * rd * 4), "rope_dkv_cmp": ("hbm", 2 * m * rd * 4),
            "rope_dkI_cmp": ("hbm", 2 * m * rd * 4)})
    return tab


def standalone_topk(layer, dev, cu, reps):
    """Mean ms of csa_index_scores and csa_topk_select run as separate calls (HIP events on
    the stream they run on) for the layer's current inputs."""
    from long_context_compressed_amd import binding as B
    p, cfg = layer.p, layer.cfg
    if cfg.idx_dtype == "fp8":
        qI, qs, kI, ks = layer.qI8, layer.qI_scale, layer.kI8, layer.kI_scale
    else:
        qI, qs, kI, ks = dev["qI"], None, layer.kI_cmp, None
    scores = torch.empty((layer.T, max(1, layer.n_cap)), dtype=torch.float32, device="cuda")
    idx = torch.empty_like(layer.idx)
    timer = EventTimer()
    for i in range(reps + 1):
        tm = timer if i > 0 else None
        for name, fn, args in (
                ("index_scores", B.csa_index_scores,
                 (p, qI, qs, dev["w"], kI, ks, cu, layer.cu_cmp, scores)),
                ("topk_select", B.csa_topk_select, (p, scores, cu, layer.cu_cmp, idx))):
            if tm:
                tm.mark(name)
            fn(*args)
            if tm:
                tm.done(name)
    torch.cuda.synchronize()
    same = bool(torch.equal(idx, layer.idx))
    print(f"[bench] stand-alone scores + top-k: same selection as the fused call: {same}",
          file=sys.stderr, flush=True)
    if not same:
        raise RuntimeError("fused and stand-alone top-k selections differ")
    return {f"{k}_standalone": v for k, v in timer.mean_ms().items()}


def standalone_learned_compressor(layer, dev, w, cu, reps):
    """Mean ms of the learned-score compressor and its adjoint on the step's main KV rows
    (and indexer key rows), with seeded synthetic score rows and positional parameter;
    ratio-4 groups overlap their left neighbour, ratio-128 groups do not."""
    from long_context_compressed_amd import binding as B
    gen = torch.Generator(device="cuda")
    gen.manual_seed(97)
    overlap = w.ratio == 4
    span = (2 if overlap else 1) * w.ratio
    jobs = [("kv", dev["kv"])]
    if layer.cfg.has_indexer:
        jobs.append(("kI", dev["kI_tok"]))
    timer = EventTimer()
    for tag, x in jobs:
        dim = x.shape[-1]
        sc = torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype)
        bias = torch.randn((span, dim), generator=gen, device="cuda")
        out = torch.empty((layer.tc_cap, dim), dtype=x.dtype, device="cuda")
        dc = torch.randn((layer.tc_cap, dim), generator=gen, device="cuda")
        dx = torch.zeros(x.shape, dtype=torch.float32, device="cuda")
        ds = torch.zeros_like(dx)
        db = torch.zeros_like(bias)
        for i in range(reps + 1):
            tm = timer if i > 0 else None
            for name, fn, args in (
                    (f"compress_learned_{tag}", B.csa_compress_learned,
                     (layer.p, x, sc, bias, overlap, cu, layer.cu_cmp, out)),
                    (f"compress_learned_bwd_{tag}", B.csa_compress_learned_bwd,
                     (layer.p, x, sc, bias, dc, overlap, cu, layer.cu_cmp, dx, ds, db))):
                if tm:
                    tm.mark(name)
                fn(*args)
                if tm:
                    tm.done(name)
    torch.cuda.synchronize()
    return {f"{k}_standalone": v for k, v in timer.mean_ms().items()}


def standalone_hbm(layer, dev, w, cu, reps):
    """Kernel throughput of the HBM-bound compressor calls on the step's shapes: reps x n
    back-to-back launches between two HIP events (on the stream they run on), cycling over
    n copies of the operands that total at least 1 GiB, so that every launch reads HBM
    rather than the 256 MB last-level cache and no per-call event or launch gap is timed."""
    from long_context_compressed_amd import binding as B
    p = layer.p
    jobs = [("compress_kv", dev["kv"], layer.kv_cmp.shape[-1])]
    if layer.cfg.has_indexer:
        jobs.append(("compress_kI", dev["kI_tok"], layer.kI_cmp.shape[-1]))
    out = {}
    for tag, x, dim in jobs:
        tc = layer.tc_cap
        for kind in ("fwd", "bwd"):
            if kind == "fwd":
                one = x.numel() * x.element_size() + tc * dim * x.element_size()
            else:
                one = tc * dim * 4 + 2 * x.shape[0] * dim * 4
            n = max(1, -(-(1 << 30) // one))
            if kind == "fwd":
                sets = [(x.clone(), torch.empty((tc, dim), dtype=x.dtype, device="cuda"))
                        for _ in range(n)]
                call = lambda s: B.csa_compress(p, s[0], cu, layer.cu_cmp, s[1])   # noqa: E731
            else:
                sets = [(torch.randn((tc, dim), device="cuda"),
                         torch.zeros((x.shape[0], dim), device="cuda")) for _ in range(n)]
                call = lambda s: B.csa_compress_bwd(p, s[0], cu, layer.cu_cmp, s[1])  # noqa: E731
            for s in sets:
                call(s)
            torch.cuda.synchronize()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            for i in range(reps * n):
                call(sets[i % n])
            end.record()
            torch.cuda.synchronize()
            name = tag if kind == "fwd" else tag.replace("compress", "compress_bwd")
            out[f"{name}_standalone"] = start.elapsed_time(end) / (reps * n)
            del sets
    return out


def cpu_baseline(w, host, budget_s):
    """The fp64 oracle, as it stands, on evenly spaced query rows of the same workload."""
    from oracle import csa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    n_real = int(host["cu_seqlens"][-1])
    T = w.total_tokens
    h64 = {"cu_seqlens": host["cu_seqlens"], "max_seqlen": host["max_seqlen"]}
    # full-size arrays are only touched on the sampled rows (zero pages stay unallocated)
    for key in ("kv", "kI_tok"):
        if key in host:
            h64[key] = inputs.to_f64(host[key])
    if "sink" in host:
        h64["sink"] = inputs.to_f64(host["sink"])

    def rows_view(sample):
        for key in ("q", "qI", "w", "dO"):
            if key in host:
                a = np.zeros(tuple(host[key].shape), dtype=np.float64)
                a[sample] = inputs.to_f64(host[key][torch.as_tensor(sample)])
                h64[key] = a

    def run(n):
        sample = np.unique(np.linspace(0, n_real - 1, n).astype(np.int64))
        rows_view(sample)
        t0 = time.perf_counter()
        O.layer_step(h64, w, rows=sample)
        return time.perf_counter() - t0, sample.size

    t_fixed, _ = run(1)                      # one row + the full-size compressor passes
    t2, n2 = run(min(64, n_real))
    per_row = max((t2 - t_fixed) / max(n2 - 1, 1), 1e-5)
    # sample size: fill the budget, bounded so the sampled rows stay a few GB of host memory
    n = int(min(n_real, 4096, max(64, (budget_s - t_fixed) / per_row)))
    t, n = run(n)
    per_row = max((t - t_fixed) / max(n - 1, 1), 1e-9)
    est = t_fixed + per_row * (n_real - 1)
    return {"value": n_real / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {n_real} query rows, evenly spaced, plus the full-size compressor "
                      f"and compressor-adjoint passes ({t:.1f} s measured); whole-step time "
                      f"extrapolated linearly in the number of query rows"}


def main():
    args = parse()
    if args.summarize_pmc:
        res = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                            args.copy_bytes or (1 << 30))
        calls = sorted(set(res["fetch"]["per_call_bytes"]) | set(res["write"]["per_call_bytes"]))
        per_call = {c: res["fetch"]["per_call_bytes"].get(c, 0.0) +
                    res["write"]["per_call_bytes"].get(c, 0.0) for c in calls}
        print("| Call | HBM read (GB) | HBM write (GB) | total (GB) |")
        print("| --- | --- | --- | --- |")
        for c in calls:
            print(f"| {c} | {res['fetch']['per_call_bytes'].get(c, 0) / 1e9:.3f} | "
                  f"{res['write']['per_call_bytes'].get(c, 0) / 1e9:.3f} | {per_call[c] / 1e9:.3f} |")
        print()
        print(f"Copy calibration: FETCH_SIZE read {res['fetch']['copy_kib']:.0f} KiB and WRITE_SIZE "
              f"{res['write']['copy_kib']:.0f} KiB for the plain copy of {args.copy_bytes or (1 << 30)} "
              f"bytes; factors {res['fetch']['factor']:.4f} and {res['write']['factor']:.4f}.")
        print()
        print("```json")
        print(json.dumps({"source_hash": source_hash(), "per_call_bytes": per_call,
                          "fetch_factor": res["fetch"]["factor"],
                          "write_factor": res["write"]["factor"]}))
        print("```")
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.traced_steps)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.traced_steps)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (no collectives or "
              "sharding); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    from long_context_compressed_amd import binding
    from long_context_compressed_amd.pipeline import CsaLayer, LayerConfig, to_device
    binding.lib()
    w = configs.workload(args.workload)
    peaks = None
    if not args.no_measured_peaks:
        peaks = measured_peaks()
        print(f"[bench] measured peaks {peaks}", file=sys.stderr, flush=True)
    torch.cuda.reset_peak_memory_stats()
    t0 = time.time()
    host = inputs.make_inputs(w)
    dev = to_device(host)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s workload={w.name} "
          f"lengths={host['lengths']}", file=sys.stderr, flush=True)
    ws_cap = None if args.bwd_workspace_gib is None else int(args.bwd_workspace_gib * 2**30)
    layer = CsaLayer(LayerConfig.of(w), len(host["lengths"]), w.total_tokens,
                     host["max_seqlen"], backward=w.backward, bwd_ws_bytes=ws_cap)
    cu = dev["cu_seqlens"]
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        layer.step(dev, cu)
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    timer = EventTimer()
    layer.timer = timer
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        layer.step(dev, cu)
    end.record()
    torch.cuda.synchronize()
    layer.timer = None
    total_ms = start.elapsed_time(end)
    ms = total_ms / max(args.steps, 1)
    per_call = timer.mean_ms()
    mem = {"peak_allocated_gib": round(torch.cuda.max_memory_allocated() / 2**30, 2),
           "attn_bwd_workspace_gib": round(layer.ws_bwd.numel() / 2**30, 2)
           if getattr(layer, "ws_bwd", None) is not None else 0.0,
           "indexer_kl_workspace_gib": round(layer.ws_kl.numel() / 2**30, 2)
           if getattr(layer, "ws_kl", None) is not None else 0.0,
           "teacher_logit_cache_gib": round(layer.t_logits.numel() * 4 / 2**30, 2)
           if layer.t_logits is not None else 0.0}
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # a marker dispatch: in a kernel trace, what follows are the stand-alone timings
    import ctypes
    _probe = ctypes.CDLL(os.path.join(ROOT, "long_context_compressed_amd", "libcsa_probe.so"))
    _probe.csa_probe_marker.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    _probe.csa_probe_marker(None, torch.cuda.current_stream().cuda_stream)
    c = work_counts(w, host["lengths"])
    tab = roofline_table(w, c, w.total_tokens, kl_cached=layer.t_logits is not None)
    if layer.fused_topk:
        # the step selects with the fused call; the stand-alone top-k over a materialized
        # score matrix is timed after the step loop, on the same inputs
        per_call.update(standalone_topk(layer, dev, cu, reps=max(args.steps, 3)))
    if w.mode != "window":
        per_call.update(standalone_hbm(layer, dev, w, cu, reps=max(args.steps, 3)))
        # the learned-score compressor (the mean-pool one runs in the step)
        per_call.update(standalone_learned_compressor(layer, dev, w, cu, reps=max(args.steps, 3)))
    breakdown = {}
    for name, t in per_call.items():
        bound, amount = tab.get(name.replace("_standalone", ""), ("", 0))
        ent = {"ms": round(t, 4)}
        if bound == "hbm" and t > 0:
            ent["GB/s"] = round(amount / (t * 1e-3) / 1e9, 1)
            ent["frac_hbm"] = round(amount / (t * 1e-3) / PEAK["hbm"], 4)
        elif bound and t > 0:
            ent["TFLOP/s"] = round(amount / (t * 1e-3) / 1e12, 2)
            ent["frac_mfma"] = round(amount / (t * 1e-3) / PEAK[bound], 4)
        breakdown[name] = ent
    in_step = {k: v for k, v in per_call.items() if not k.endswith("_standalone")}
    dom = max(in_step, key=in_step.get)
    bound, amount = tab[dom]
    tdom = per_call[dom] * 1e-3
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": amount / tdom / 1e9, "peak": PEAK["hbm"] / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": amount / tdom / 1e12, "peak": PEAK[bound] / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if peaks:
        mp = peaks["hbm_gbps"] if bound == "hbm" else peaks[f"{bound}_tflops"]
        roof["measured_peak"] = mp
        roof["frac_measured"] = roof["achieved"] / mp
    traffic = load_traffic()
    roof["traffic"] = traffic.get(dom) if traffic else None
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = amount
    tokens = c["tokens"]
    value = tokens / (ms * 1e-3)
    attn_ms = per_call.get("attn_fwd", 0) + per_call.get("attn_bwd", 0)
    attn_flops = tab["attn_fwd"][1] + (tab["attn_bwd"][1] if w.backward else 0)
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "tokens": tokens, "samples": len(host["lengths"]),
                   "lengths": host["lengths"], "heads": w.heads, "head_dim": w.head_dim,
                   "ratio": w.ratio, "window": w.window, "topk": w.topk, "mode": w.mode,
                   "idx_heads": w.idx_heads, "idx_dim": w.idx_dim, "idx_dtype": w.idx_dtype,
                   "teacher": w.teacher, "rope_dim": w.rope_dim,
                   "bwd_workspace_cap_gib": args.bwd_workspace_gib,
                   "pass": "fwd+bwd" if w.backward else "fwd"},
        "roofline": roof,
        "attention_tflops": attn_flops / max(attn_ms * 1e-3, 1e-12) / 1e12 if attn_ms else None,
        "topk_gbps": (breakdown.get("topk_select") or
                      breakdown.get("topk_select_standalone", {})).get("GB/s"),
        "breakdown": breakdown,
        "work": c,
        "device_memory": mem,
        "measured_peaks": peaks,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
