"""Benchmark of the block-sparse, head-masked attention hot path on one MI355X.

A step is one pass of the whole path over one batch: block sums, scores,
rank, pins, compaction and attention over the kept blocks (head-masked), on
synthetic inputs already resident in HBM.  It runs as bsattn_select_forward,
which ranks inside the attention kernel where that kernel applies (bf16, D 64,
block 64, every block a candidate, at most 64 blocks, no head mask) and is
bsattn_select followed by bsattn_forward elsewhere; `two_call_ms_per_step`
times the same step as the two calls (--two-calls makes them the step).  The default workload is the SDXL self-attention shape (B=2 CFG pair,
10 heads, 64x64 latent = 4096 tokens, head_dim 64, 64-token blocks, 30%
budget) — the shape the SD.Next commit page quotes its timings on.

Prints one JSON line.  `value` is kept-block attention TFLOP/s of the whole
step (kept FLOPs / step time).  `roofline` covers the attention kernel (MFMA
bound); `selector` reports the selector's algorithmic GB/s against HBM;
`speedup_vs_dense` compares the same attention kernel at full density (budget
1.0, same layout and head mask).  `cpu_baseline` times the fp64 CPU oracle on
the same workload on this host's cores.  `per_config` repeats the step,
roofline, selector and speedup figures for every configuration (tiny fp32,
SDXL, joint text+image, video with its radial control, the 64-layer
head-masked stack with its head-mask skip); `reference` gives the platform's
own bf16 GEMM and dense sdpa rates on this GPU as context.

Every configuration first runs untimed steps for --prewarm-s seconds (the
GPU's clocks ramp up over the first tens of ms under load), then --warmup
untimed steps, then exactly --steps timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import head_masked_attention_amd as hm  # noqa: E402
import workloads  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
FP32_PEAK_TFLOPS = 157.3           # MI355X dense fp32 MFMA (the fp32 path's matrix instruction)
# the configurations reported under per_config: tiny fp32, SDXL, joint
# text+image, video (with the radial control), the 64-layer head-masked stack
PER_CONFIG = ["tiny_fp32", "sdxl_bf16", "joint_text_image_bf16", "video_radial_bf16", "head_masked_stack_bf16"]
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
ATTN_SOURCES = ["head_masked_attention_amd/csrc/attn_mfma.hip", "head_masked_attention_amd/csrc/common.h",
                "head_masked_attention_amd/csrc/rank.h",
                "head_masked_attention_amd/csrc/internal.h"]


def attn_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter summary, or
    None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"attn_mfma_kernel__{workload}__hbm_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip().lstrip("- ")
            if ":" in line and line.startswith(("kernel_source_sha256", "traffic_bytes_per_launch")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != attn_source_hash():
        return None
    return float(vals["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in vals else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--prewarm-s", type=float, default=0.5,
                   help="untimed steps for this many seconds before the warm-up steps of each configuration "
                        "(the GPU's clocks ramp up under load); 0: none")
    p.add_argument("--workload", default="sdxl_bf16", choices=sorted(workloads.ALL))
    p.add_argument("--layer", type=int, default=0, help="layer of the stacked workload (with --one-layer)")
    p.add_argument("--one-layer", action="store_true",
                   help="stacked workload: time one layer instead of all layers back to back")
    p.add_argument("--no-cold", action="store_true", help="skip the cache-cold secondary timings")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (HBM counter calibration)")
    p.add_argument("--two-calls", action="store_true",
                   help="run the step as bsattn_select + bsattn_forward even where bsattn_select_forward "
                        "fuses the ranking into the attention kernel")
    p.add_argument("--no-per-config", action="store_true",
                   help="skip the per-configuration figures of every workload")
    p.add_argument("--no-reference", action="store_true",
                   help="skip the platform reference figures (torch GEMM and sdpa)")
    p.add_argument("--kernels-only", choices=["select", "forward", "step", "fp8", "copy"], default=None,
                   help="profiling aid: stage the workload, run only this call (or a plain 256 MiB read + "
                        "256 MiB write copy) --warmup + --steps times, print its time")
    p.add_argument("--graph", action="store_true",
                   help="replay the step (and the per-call loops) as captured HIP graphs instead of "
                        "launching every call from the host")
    return p.parse_args()


def kept_flops(count: torch.Tensor, head_mask, block: int, D: int, H: int) -> float:
    """4 * block^2 * D per kept (b, h, query block, key block) of an active head."""
    c = count.to(torch.int64).cpu()
    if c.shape[1] == 1 and H > 1:
        c = c.expand(c.shape[0], H, c.shape[2])
    if head_mask is not None:
        c = c * head_mask.cpu().to(torch.int64)[None, :, None]
    return float(c.sum().item()) * 4.0 * block * block * D


def selector_bytes(w, bm: hm.BlockMask, n_cand: int, head_mask=None) -> float:
    """Q and K of the sparsifiable tokens read once, mask/count/index written.
    Under a head mask (bsattn_select_heads) only the active heads' Q and the
    K heads they use are read."""
    esize = 2 if w.dtype == "bf16" else 4
    q_heads, k_heads = w.H, w.kv_heads
    if head_mask is not None:
        rep = w.H // w.kv_heads
        q_heads = int(head_mask.sum())
        k_heads = int(sum(head_mask[g * rep:(g + 1) * rep].any() for g in range(w.kv_heads)))
    reads = w.B * (q_heads + k_heads) * n_cand * w.block * w.D * esize
    nb = w.nb
    kept = float(bm.count.to(torch.int64).sum().item())
    writes = w.B * w.H * nb * nb + w.B * w.H * nb * 4 + kept * 4
    return reads + writes


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, layers, flops_total, budget_s: float = 12.0):
    """The fp64 oracle on this host's cores, on a bounded sample of the same
    workload, scaled to the whole step.

    `layers` is a list of (q, k, v, head_mask_np) on the host.  Selection runs
    in full on every sampled layer; attention runs on every query row when
    that fits the time budget, else on a seeded sample of rows (each row of
    the masked-dense oracle costs the same), and its time is scaled by rows.
    """
    import oracle
    rng = np.random.default_rng(0)
    t_sel = t_att = 0.0
    rows_done = rows_total = 0
    for (q, k, v, hm_np) in layers:
        q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
        t0 = time.perf_counter()
        mask, _tie = oracle.select(q64, k64, w.block, list(w.segments), w.budget, w.window_tokens)
        t_sel += time.perf_counter() - t0
        n_rows = w.B * w.H * w.N
        rows_total += n_rows
        # one row's cost, measured on a small probe, sizes the sample
        probe = np.stack([rng.integers(0, w.B, 8), rng.integers(0, w.H, 8), rng.integers(0, w.N, 8)], 1)
        t0 = time.perf_counter()
        oracle.attention(q64, k64, v64, w.block, mask, head_mask=hm_np, rows=probe)
        per_row = (time.perf_counter() - t0) / 8
        want = int(max(64, min(n_rows, (budget_s / max(len(layers), 1)) / max(per_row, 1e-9))))
        if want >= n_rows:
            t0 = time.perf_counter()
            oracle.attention(q64, k64, v64, w.block, mask, head_mask=hm_np)
            t_att += time.perf_counter() - t0
            rows_done += n_rows
        else:
            rows = np.stack([rng.integers(0, w.B, want), rng.integers(0, w.H, want),
                             rng.integers(0, w.N, want)], 1)
            t0 = time.perf_counter()
            oracle.attention(q64, k64, v64, w.block, mask, head_mask=hm_np, rows=rows)
            t_att += time.perf_counter() - t0
            rows_done += want
    sec = t_sel + t_att * rows_total / rows_done
    full = rows_done == rows_total
    return {"value": flops_total / sec / 1e12,
            "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle", "cpu": cpu_model(),
            "sample": (f"{len(layers)} layer(s) of {w.name}: selection in full, masked-dense fp64 attention on "
                       + ("every query row" if full else
                          f"{rows_done} of {rows_total} query rows (seeded), time scaled by rows")
                       + f"; {t_sel + t_att:.1f} s measured, {sec:.2f} s per step extrapolated")}


class Timer:
    """Per-call GPU time of a call sequence.

    `eager`: `reps` back-to-back host launches timed with HIP events on the
    stream the kernels run on.  Otherwise the sequence is captured once into a
    HIP graph holding `reps` copies and one replay is timed.
    """

    def __init__(self, dev, stream, eager: bool):
        self.dev, self.stream, self.eager = dev, stream, eager

    def warm(self, fn, reps: int, warmup: int) -> float:
        for _ in range(warmup):
            fn(self.stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if self.eager:
            e0.record(self.stream)
            for _ in range(reps):
                fn(self.stream)
            e1.record(self.stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(self.dev)
        cap.wait_stream(self.stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for _ in range(reps):
                    fn(cap)
        self.stream.wait_stream(cap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            g.replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def cold(self, fn, reps: int, scratch: torch.Tensor) -> float:
        """Median time of one call after a 512 MiB scratch write that evicts
        the L2 and the MALL (outside the timed region)."""
        ts = []
        for _ in range(reps):
            scratch.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            fn(self.stream)
            e1.record(self.stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))


def stage_layers(w, layer_ids, dev):
    """Q/K/V (device) and head masks of the given layers."""
    layers = []
    for l in layer_ids:
        q, k, v = workloads.make_qkv(w, l)
        if w.layers > 1:
            hm_np = hm.head_mask(workloads.head_importance(w, l))
        elif w.head_mask is not None:
            hm_np = np.array(w.head_mask, np.uint8)
        else:
            hm_np = None
        layers.append(dict(q=q, k=k, v=v, qd=q.to(dev), kd=k.to(dev), vd=v.to(dev), hm_np=hm_np,
                           hmd=None if hm_np is None else torch.from_numpy(hm_np).to(dev)))
    return layers


def fused_applies(w, layers, two_calls: bool) -> bool:
    """bsattn_select_forward ranks inside the attention kernel for bf16, D 64,
    block 64, every block a candidate, at most 64 blocks, no head mask."""
    return (not two_calls and w.dtype == "bf16" and w.D == 64 and w.block == 64 and not w.segments
            and not w.window_tokens and w.nb <= 64 and w.budget < 1.0 and all(ly["hmd"] is None for ly in layers))


class Run:
    """One workload staged on the device, with its calls and timers."""

    def __init__(self, w, dev, args, stack: bool, layer: int = 0):
        self.w, self.dev, self.args = w, dev, args
        self.layer_ids = list(range(w.layers)) if stack else [layer]
        self.layers = stage_layers(w, self.layer_ids, dev)
        self.layout = hm.Layout(w.block, list(w.segments), w.window_tokens)
        _cls, self.n_cand = hm.layout_classes(self.layout, w.N)
        L = len(self.layers)
        self.bms = [hm.empty_block_mask(w.B, w.H, w.nb, dev) for _ in range(L)]
        self.bm_full = hm.empty_block_mask(w.B, w.H, w.nb, dev)
        self.ws = torch.empty(hm.select_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.block, w.D),
                              dtype=torch.uint8, device=dev)
        self.outs = [torch.empty_like(ly["qd"]) for ly in self.layers]
        self.stream = torch.cuda.current_stream(dev)
        self.timer = Timer(dev, self.stream, eager=not args.graph)
        self.fused = fused_applies(w, self.layers, args.two_calls)

    def select(self, i, st, budget=None, out=None):
        ly = self.layers[i]
        hm.select(ly["qd"], ly["kd"], self.layout, self.w.budget if budget is None else budget,
                  out=self.bms[i] if out is None else out, workspace=self.ws, stream=st)

    def select_heads(self, i, st):
        """The step's selection: under the layer's head mask where it has one
        (masked heads neither pooled nor ranked), else bsattn_select."""
        ly = self.layers[i]
        if ly["hmd"] is None:
            self.select(i, st)
            return
        hm.select_heads(ly["qd"], ly["kd"], self.layout, self.w.budget, ly["hmd"], out=self.bms[i],
                        workspace=self.ws, stream=st)

    def forward(self, i, st, bm=None, head_mask="layer"):
        ly = self.layers[i]
        hmask = ly["hmd"] if isinstance(head_mask, str) else head_mask
        hm.forward(ly["qd"], ly["kd"], ly["vd"], self.bms[i] if bm is None else bm, hmask, out=self.outs[i],
                   stream=st)

    def select_forward(self, i, st):
        ly = self.layers[i]
        hm.select_forward(ly["qd"], ly["kd"], ly["vd"], self.layout, self.w.budget, ly["hmd"], out=self.outs[i],
                          block_mask=self.bms[i], workspace=self.ws, stream=st)

    def two_call_step(self, st):
        for i in range(len(self.layers)):
            self.select_heads(i, st)
            self.forward(i, st)

    def step(self, st):
        """One pass of the hot path over the staged batch (every layer)."""
        if not self.fused:
            self.two_call_step(st)
            return
        for i in range(len(self.layers)):
            self.select_forward(i, st)

    def prewarm(self, seconds: float):
        """Untimed steps for `seconds` of wall time before any timed region.
        The GPU's clocks take a few tens of ms of load to reach their steady
        state (the SDXL step measured 49 us in its first 200 steps and 45 us
        from about the 500th on, same process), so without this the first
        figures of a run time the ramp."""
        if seconds <= 0:
            return
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                self.step(self.stream)
            torch.cuda.synchronize()

    def time_steps(self, steps: int, warmup: int, fn=None):
        """Host-clocked ms per step over `steps` steps, synchronised on both sides."""
        capture = fn is None and self.args.graph
        fn = fn or (lambda: self.step(self.stream))
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if capture:
            graph = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream(self.dev)
            cap.wait_stream(self.stream)
            with torch.cuda.stream(cap):
                with torch.cuda.graph(graph, stream=cap):
                    self.step(cap)
            self.stream.wait_stream(cap)
            torch.cuda.synchronize()
            fn = graph.replay
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def kernel_figures(self, reps: int, warmup: int):
        """Per-call figures on layer 0: attention roofline, selector GB/s,
        speedup against the same kernel at full density."""
        w, t = self.w, self.timer
        sel_ms = t.warm(lambda st: self.select(0, st), reps, warmup)
        sel_graph_ms = sel_ms if self.args.graph else Timer(self.dev, self.stream, eager=False).warm(
            lambda st: self.select(0, st), reps, warmup)
        fwd_ms = t.warm(lambda st: self.forward(0, st), reps, warmup)
        self.select(0, self.stream, budget=1.0, out=self.bm_full)
        dense_ms = t.warm(lambda st: self.forward(0, st, bm=self.bm_full), reps, warmup)
        for i in range(len(self.layers)):      # the step's own masks, outside every timed region
            self.select(i, self.stream)
        torch.cuda.synchronize()
        self.flops_layers = [kept_flops(self.bms[i].count, self.layers[i]["hmd"], w.block, w.D, w.H)
                             for i in range(len(self.layers))]
        flops0 = self.flops_layers[0]
        flops_dense0 = kept_flops(self.bm_full.count, self.layers[0]["hmd"], w.block, w.D, w.H)
        sel_bytes = selector_bytes(w, self.bms[0], self.n_cand)
        attn_tflops = flops0 / (fwd_ms * 1e-3) / 1e12
        sel_gbps = sel_bytes / (sel_ms * 1e-3) / 1e9
        bf16 = w.dtype == "bf16"
        roof = {"bound": "mfma", "kernel": "attn_mfma_kernel (bsattn_forward)" if bf16
                else "attn_f32_kernel (bsattn_forward, fp32 MFMA)",
                "achieved": attn_tflops, "peak": MFMA_BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": attn_tflops / (MFMA_BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS),
                "traffic": profiled_traffic(w.name) if bf16 else None,
                "traffic_unit": "bytes per launch (HBM fetch + write, rocprofv3 counters)",
                "flops_per_launch": flops0, "avg_launch_ms": fwd_ms}
        sel = {"bound": "hbm", "achieved": sel_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
               "frac": sel_gbps / HBM_PEAK_GBPS, "bytes_per_call": sel_bytes, "avg_call_ms": sel_ms,
               "graph_call_ms": sel_graph_ms,
               "graph_frac": sel_bytes / (sel_graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               "kernels": "pool_kernel + score_rank_kernel (bsattn_select)",
               "note": "avg_call_ms: host-launched calls; graph_call_ms: the same calls replayed from a "
                       "HIP graph (the kernels without the host's launch rate)"}
        step_sel_ms = min(sel_ms, sel_graph_ms)
        ly0 = self.layers[0]
        if ly0["hmd"] is not None:
            # the step's selection under the layer's head mask (bsattn_select_heads)
            h_ms = t.warm(lambda st: self.select_heads(0, st), reps, warmup)
            h_graph_ms = h_ms if self.args.graph else Timer(self.dev, self.stream, eager=False).warm(
                lambda st: self.select_heads(0, st), reps, warmup)
            torch.cuda.synchronize()
            h_bytes = selector_bytes(w, self.bms[0], self.n_cand, ly0["hm_np"])
            self.select(0, self.stream)        # every head's rows again, for the all-heads figure below
            torch.cuda.synchronize()
            sel["heads"] = {"avg_call_ms": h_ms, "graph_call_ms": h_graph_ms, "bytes_per_call": h_bytes,
                            "graph_frac": h_bytes / (h_graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                            "kernels": "pool_kernel + score_rank_kernel (bsattn_select_heads: the masked "
                                       "heads' Q, and K heads no active head uses, are not pooled; their rows "
                                       "come back empty)"}
            step_sel_ms = min(h_ms, h_graph_ms)
        speed = {"attention": dense_ms / fwd_ms, "step": dense_ms / (step_sel_ms + fwd_ms),
                 "dense_attention_ms": dense_ms, "dense_flops": flops_dense0, "ideal": flops_dense0 / flops0,
                 "note": "attention: the same kernel at budget 1.0 over the 30 % launch; step: that dense "
                         "launch over the step's selector (bsattn_select_heads under a head mask) + attention "
                         "(the selector's faster of host-launched and graph-replayed time); measured_step: that "
                         "dense launch over the host-timed step per layer (ms_per_step, the calls the step makes)"}
        return roof, sel, speed, fwd_ms

    def radial_figures(self, reps, warmup):
        w = self.w
        bm_rad = hm.radial(self.layout, w.N, w.budget, B=1, H=1, device=self.dev)
        rad_ms = self.timer.warm(lambda st: hm.radial(self.layout, w.N, w.budget, B=1, H=1, out=bm_rad, stream=st),
                                 reps, warmup)
        rad_fwd_ms = self.timer.warm(lambda st: self.forward(0, st, bm=bm_rad), reps, warmup)
        torch.cuda.synchronize()
        rad_flops = kept_flops(bm_rad.count, self.layers[0]["hmd"], w.block, w.D, w.H)
        return {"radial_ms": rad_ms, "attention_ms": rad_fwd_ms, "flops": rad_flops,
                "tflops": rad_flops / (rad_fwd_ms * 1e-3) / 1e12, "k": bm_rad.k,
                "note": "bsattn_radial: the band at the selector's k (the control the selector has to beat); "
                        "attention: bsattn_forward on the band"}

    def head_mask_figures(self, fwd_ms, reps, warmup):
        ly0 = self.layers[0]
        if ly0["hmd"] is None:
            return None
        all_heads = torch.ones(self.w.H, dtype=torch.uint8, device=self.dev)
        t_all = self.timer.warm(lambda st: self.forward(0, st, head_mask=all_heads), reps, warmup)
        return {"active_heads": int(ly0["hm_np"].sum()), "heads": self.w.H, "all_heads_ms": t_all,
                "masked_ms": fwd_ms, "time_skipped": 1.0 - fwd_ms / t_all,
                "ideal_skipped": 1.0 - float(ly0["hm_np"].sum()) / self.w.H}

    def sdpa_reference(self, reps):
        """torch's own scaled_dot_product_attention (dense, bf16) on layer 0's
        shape: the platform's flash attention, for context."""
        w, ly = self.w, self.layers[0]
        if w.dtype != "bf16":
            return None
        k, v = ly["kd"], ly["vd"]
        if w.kv_heads != w.H:
            k = k.repeat_interleave(w.H // w.kv_heads, dim=1)
            v = v.repeat_interleave(w.H // w.kv_heads, dim=1)
        fn = lambda st: torch.nn.functional.scaled_dot_product_attention(ly["qd"], k, v)
        ms = self.timer.warm(fn, reps, 2)
        fl = 4.0 * w.B * w.H * w.N * w.N * w.D
        return {"ms": ms, "tflops": fl / ms / 1e9, "note": "torch sdpa, dense, all heads (context only)"}


def gemm_reference(dev):
    """bf16 GEMM rate of torch (hipBLASLt) at 8192^3: the platform's practical
    matrix-core ceiling, for context."""
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    tf = 2.0 * n ** 3 / ms / 1e9
    return {"gemm_bf16_8192_tflops": tf, "gemm_frac_of_peak": tf / MFMA_BF16_PEAK_TFLOPS}


def per_config_entry(w, dev, args):
    """The figures of one configuration (its own step, kernels, controls)."""
    stack = w.layers > 1
    r = Run(w, dev, args, stack=stack)
    steps = max(2, min(args.steps, 5 if stack else 20))
    warmup = max(1, min(args.warmup, 2 if stack else 5))
    r.prewarm(args.prewarm_s)
    ms_step = r.time_steps(steps, warmup)
    reps = max(2, min(args.steps, 20))
    roof, sel, speed, fwd_ms = r.kernel_figures(reps, min(args.warmup, 5))
    speed["measured_step"] = speed["dense_attention_ms"] * len(r.layers) / ms_step
    flops = sum(r.flops_layers)
    e = {"config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "N": w.N, "D": w.D,
                    "block": w.block, "dtype": w.dtype, "budget": w.budget, "k": r.bms[0].k, "layers": w.layers,
                    "segments": [list(s) for s in w.segments], "window_tokens": w.window_tokens},
         "step": {"ms_per_step": ms_step, "value": flops / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
                  "calls": "bsattn_select_forward" if r.fused else "bsattn_select + bsattn_forward",
                  "layers_per_step": len(r.layers)},
         "roofline": roof, "selector": sel, "speedup_vs_dense": speed}
    if not args.no_cold:
        scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)   # 512 MiB
        e["cold"] = {"selector_ms": r.timer.cold(lambda st: r.select(0, st), 11, scratch),
                     "attention_ms": r.timer.cold(lambda st: r.forward(0, st), 11, scratch),
                     "note": "median of 11 single calls, each after a 512 MiB scratch write"}
        del scratch
    if w.radial:
        e["radial"] = r.radial_figures(reps, min(args.warmup, 5))
    hmf = r.head_mask_figures(fwd_ms, reps, min(args.warmup, 5))
    if hmf is not None:
        e["head_masking"] = hmf
    e["torch_sdpa_dense"] = r.sdpa_reference(3 if w.N > 20000 else 10)
    del r
    torch.cuda.empty_cache()
    return e


def kernels_only(args, w, dev, stack):
    """Run one call of the workload (layer 0; every layer for a stacked
    "step") --warmup + --steps times back to back, for a profiler to see
    only its kernels.  "copy": a plain elementwise read of 256 MiB and write of
    256 MiB, the known byte count that scales the HBM fetch/write counters."""
    if args.kernels_only == "copy":
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        fn = lambda: torch.mul(src, 1.0, out=dst)
    else:
        r = Run(w, dev, args, stack=stack and args.kernels_only == "step", layer=args.layer)
        r.select(0, r.stream)      # the block mask the forward reads
        if args.kernels_only == "fp8":
            # the fp8 consumer on the same block mask: Q, K, V quantised once
            # before the loop, then bsattn_forward_fp8 per call
            ly0 = r.layers[0]
            q8, qs = hm.quantize_fp8(ly0["qd"], stream=r.stream)
            k8, ks = hm.quantize_fp8(ly0["kd"], stream=r.stream)
            v8, vs = hm.quantize_fp8(ly0["vd"], stream=r.stream)
            out8 = torch.empty_like(ly0["qd"])
            fn = lambda: hm.forward_fp8(q8, k8, v8, qs, ks, vs, r.bms[0], ly0["hmd"], out=out8, stream=r.stream)
        else:
            fn = {"select": lambda: r.select(0, r.stream), "forward": lambda: r.forward(0, r.stream),
                  "step": lambda: r.step(r.stream)}[args.kernels_only]
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    print(json.dumps({"workload": w.name, "call": args.kernels_only, "steps": args.steps,
                      "ms_per_call": e0.elapsed_time(e1) / max(args.steps, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    w = workloads.ALL[args.workload]
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    stack = w.layers > 1 and not args.one_layer
    if args.kernels_only is not None:
        kernels_only(args, w, dev, stack)
        return
    r = Run(w, dev, args, stack=stack, layer=args.layer)
    layers, L = r.layers, len(r.layers)
    fused = r.fused

    # ---- whole-step throughput: K steps on the host clock, synchronised on
    # both sides.  The step is bsattn_select_forward where the fused kernel
    # applies, else bsattn_select + bsattn_forward; every call is launched
    # from the host (--graph captures the step once and replays it).  On
    # MI355X the replayed kernels start with a cold L2, so host launches are
    # the faster default here.
    r.prewarm(args.prewarm_s)
    ms_per_step = r.time_steps(args.steps, args.warmup)
    two_call_ms = None
    if fused and not args.graph:
        two_call_ms = r.time_steps(args.steps, args.warmup, fn=lambda: r.two_call_step(r.stream))

    reps = max(1, min(args.steps, 50))
    roof, sel, speed, fwd_ms = r.kernel_figures(reps, args.warmup)
    speed["measured_step"] = speed["dense_attention_ms"] * L / ms_per_step
    flops = sum(r.flops_layers)
    flops0 = r.flops_layers[0]

    fused_fig = None
    if fused:
        # the step's own call, alone: pool (K only) + attention with the
        # ranking inside; its rate counts the whole call (pool and ranking
        # included) against the kept FLOPs
        f_ms = r.timer.warm(lambda st: r.select_forward(0, st), reps, args.warmup)
        f_graph_ms = Timer(dev, r.stream, eager=False).warm(lambda st: r.select_forward(0, st), reps, args.warmup)
        fused_fig = {"call_ms": f_ms, "graph_call_ms": f_graph_ms,
                     "tflops": flops0 / (f_ms * 1e-3) / 1e12,
                     "frac": flops0 / (f_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "kernels": "pool_kernel (K only) + attn_mfma_kernel<FUSED> (bsattn_select_forward)",
                     "note": "the step's calls; roofline and selector above are the two-call kernels "
                             "(bsattn_forward, bsattn_select) on the same inputs"}

    # cold: L2 and MALL evicted before each call (secondary figures)
    cold = None
    if not args.no_cold:
        scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)   # 512 MiB
        cold = {"selector_ms": r.timer.cold(lambda st: r.select(0, st), 11, scratch),
                "attention_ms": r.timer.cold(lambda st: r.forward(0, st), 11, scratch),
                "note": "median of 11 single calls, each after a 512 MiB scratch write"}
        del scratch

    radial = r.radial_figures(reps, args.warmup) if w.radial else None

    # per-token key mask composed with the block mask (bsattn_forward_masked):
    # all keys live, and the last 1/16 of each batch's keys masked
    km_live = torch.ones(w.B, w.N, dtype=torch.uint8, device=dev)
    km_tail = km_live.clone()
    km_tail[:, w.N - w.N // 16:] = 0
    ly0 = layers[0]
    bms, outs = r.bms, r.outs
    key_mask = {
        "all_live_ms": r.timer.warm(lambda st: hm.forward(ly0["qd"], ly0["kd"], ly0["vd"], bms[0], ly0["hmd"],
                                                          out=outs[0], stream=st, key_mask=km_live),
                                    reps, args.warmup),
        "tail_masked_ms": r.timer.warm(lambda st: hm.forward(ly0["qd"], ly0["kd"], ly0["vd"], bms[0], ly0["hmd"],
                                                             out=outs[0], stream=st, key_mask=km_tail),
                                       reps, args.warmup),
        "note": "bsattn_forward_masked on the step's block mask; tail = last N/16 keys of each batch masked",
    }

    # the fp8 (E4M3) consumer on the step's block mask: per-head quantisation
    # of Q, K, V (reported separately, a producer-side cost) and the fp8
    # attention, against the fp8 MFMA peak
    fp8 = None
    if w.dtype == "bf16" and w.block == 64 and w.D in (64, 128):
        q8, qs = hm.quantize_fp8(ly0["qd"])
        k8, ks = hm.quantize_fp8(ly0["kd"])
        v8, vs = hm.quantize_fp8(ly0["vd"])
        out8 = torch.empty_like(outs[0])
        t = r.timer
        quant_ms = t.warm(lambda st: hm.quantize_fp8(ly0["qd"], out=q8, scale=qs, stream=st), reps, args.warmup)
        fp8_ms = t.warm(lambda st: hm.forward_fp8(q8, k8, v8, qs, ks, vs, bms[0], ly0["hmd"], out=out8, stream=st),
                        reps, args.warmup)
        fp8_dense_ms = t.warm(lambda st: hm.forward_fp8(q8, k8, v8, qs, ks, vs, r.bm_full, ly0["hmd"], out=out8,
                                                        stream=st), reps, args.warmup)
        fp8_km_ms = t.warm(lambda st: hm.forward_fp8(q8, k8, v8, qs, ks, vs, bms[0], ly0["hmd"], out=out8,
                                                     stream=st, key_mask=km_tail), reps, args.warmup)
        fp8_tf = flops0 / (fp8_ms * 1e-3) / 1e12
        fp8 = {"attention_ms": fp8_ms, "achieved": fp8_tf, "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
               "frac": fp8_tf / MFMA_FP8_PEAK_TFLOPS, "dense_attention_ms": fp8_dense_ms,
               "speedup_vs_dense": fp8_dense_ms / fp8_ms, "quantize_one_tensor_ms": quant_ms,
               "key_mask_tail_ms": fp8_km_ms,
               "note": "bsattn_forward_fp8 on E4M3 Q/K/V with per-head scales (bf16 out); quantisation of one "
                       "[B,H,N,D] tensor timed separately; key_mask_tail: bsattn_forward_fp8_masked with the "
                       "last N/16 keys of each batch masked"}
        del q8, k8, v8, out8

    # head masking: the same forward with every head active, for the share of
    # attention time the layer's head mask skips (the pages claim 50-70 %)
    head_masking = r.head_mask_figures(fwd_ms, reps, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        sample_ids = [0] if not stack else [0, w.layers // 3, 2 * w.layers // 3, w.layers - 1]
        sample = [(layers[i]["q"], layers[i]["k"], layers[i]["v"], layers[i]["hm_np"]) for i in sample_ids]
        # kept FLOPs of the sampled layers, so value compares like with like
        flops_sample = sum(r.flops_layers[i] for i in sample_ids)
        cpu = cpu_baseline(w, sample, flops_sample)

    if args.calibrate_copy:
        # an elementwise kernel that reads 256 MiB and writes 256 MiB: the known
        # byte count that scales the HBM fetch/write counters
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    reference = {"note": "the platform's own kernels on this GPU, for context (not part of the path)"}
    if not args.no_reference:
        reference.update(gemm_reference(dev))
        reference["torch_sdpa_dense_headline"] = r.sdpa_reference(10)

    hmask0 = layers[0]["hm_np"]
    res = {
        "metric": "block-sparse attn TFLOP/s on kept blocks & speedup vs dense at 30% budget",
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": args.prewarm_s,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; clustered Q/K for image workloads)",
        "step_launch": "hip graph replay" if args.graph else "host launches",
        "step_calls": "bsattn_select_forward (ranking fused into the attention kernel)" if fused
                      else "bsattn_select + bsattn_forward",
        "two_call_ms_per_step": two_call_ms,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "N": w.N, "D": w.D,
                   "block": w.block, "budget": w.budget, "k": bms[0].k,
                   "layers": L, "layer": r.layer_ids[0] if L == 1 else None,
                   "segments": [list(s) for s in w.segments], "window_tokens": w.window_tokens,
                   "active_heads": int(hmask0.sum()) if hmask0 is not None else w.H,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "selector": sel,
        "fused_step_call": fused_fig,
        "speedup_vs_dense": speed,
        "cold": cold,
        "radial": radial,
        "key_mask": key_mask,
        "fp8": fp8,
        "head_masking": head_masking,
        "pages_context": {
            "note": "figures printed by the SD.Next commit page and the haagenti_sparse pages, on unstated "
                    "hardware and precision: context, not targets",
            "dense_attention_sdxl_ms": 1.2, "selection_overhead_sdxl_ms_before_after": [1.84, 0.23],
            "budget_30pct_vs_dense_before_after": [0.36, 1.19], "head_masking_compute_skipped_claim": [0.5, 0.7],
        },
        "cpu_baseline": cpu,
        "reference": reference,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""), "host": platform.node()},
    }
    del r, layers, bms, outs
    torch.cuda.empty_cache()

    # every configuration of the workload set, each with its own step,
    # kernel figures and controls (the headline's entry is the line above)
    if not args.no_per_config:
        per = {}
        for name in PER_CONFIG:
            wc = workloads.ALL[name]
            print(f"[bench] per-config {name}", file=sys.stderr, flush=True)
            per[name] = per_config_entry(wc, dev, args)
        res["per_config"] = per
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
