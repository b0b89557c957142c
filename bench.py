"""Benchmark of the block-sparse, head-masked attention hot path on one MI355X.

A step is one pass of the whole path over one batch: bsattn_select (block
sums, scores, rank, pins, compaction) followed by bsattn_forward (attention
over the kept blocks, head-masked) on synthetic inputs already resident in
HBM.  The default workload is the SDXL self-attention shape (B=2 CFG pair,
10 heads, 64x64 latent = 4096 tokens, head_dim 64, 64-token blocks, 30%
budget) — the shape the SD.Next commit page quotes its timings on.

Prints one JSON line.  `value` is kept-block attention TFLOP/s of the whole
step (kept FLOPs / step time).  `roofline` covers the attention kernel (MFMA
bound); `selector` reports the selector's algorithmic GB/s against HBM;
`speedup_vs_dense` compares the same attention kernel at full density (budget
1.0, same layout and head mask).  `cpu_baseline` times the fp64 CPU oracle on
the same workload on this host's cores.
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
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
ATTN_SOURCES = ["head_masked_attention_amd/csrc/attn_mfma.hip", "head_masked_attention_amd/csrc/common.h",
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
            if ":" in line and line.strip().startswith(("kernel_source_sha256", "traffic_bytes_per_launch")):
                k, v = line.strip().split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != attn_source_hash():
        return None
    return float(vals["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in vals else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="sdxl_bf16", choices=sorted(workloads.ALL))
    p.add_argument("--layer", type=int, default=0, help="layer of the stacked workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (HBM counter calibration)")
    p.add_argument("--eager", action="store_true",
                   help="launch every step from the host instead of replaying a captured HIP graph")
    return p.parse_args()


def kept_flops(count: torch.Tensor, head_mask, block: int, D: int, H: int) -> float:
    """4 * block^2 * D per kept (b, h, query block, key block) of an active head."""
    c = count.to(torch.int64).cpu()
    if c.shape[1] == 1 and H > 1:
        c = c.expand(c.shape[0], H, c.shape[2])
    if head_mask is not None:
        c = c * head_mask.cpu().to(torch.int64)[None, :, None]
    return float(c.sum().item()) * 4.0 * block * block * D


def selector_bytes(w, bm: hm.BlockMask, n_cand: int) -> float:
    """Q and K of the sparsifiable tokens read once, mask/count/index written."""
    esize = 2 if w.dtype == "bf16" else 4
    reads = w.B * (w.H + w.kv_heads) * n_cand * w.block * w.D * esize
    nb = w.nb
    kept = float(bm.count.to(torch.int64).sum().item())
    writes = w.B * w.H * nb * nb + w.B * w.H * nb * 4 + kept * 4
    return reads + writes


def cpu_baseline(w, q, k, v, layout_segments, head_mask_np, flops_total):
    import oracle
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    reps, t_total = 0, 0.0
    while t_total < 5.0 and reps < 20:
        t0 = time.perf_counter()
        mask, _tie = oracle.select(q64, k64, w.block, layout_segments, w.budget, w.window_tokens)
        oracle.attention(q64, k64, v64, w.block, mask, head_mask=head_mask_np)
        t_total += time.perf_counter() - t0
        reps += 1
    sec = t_total / reps
    return {"value": flops_total / sec / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"full {w.name} step (select + masked-dense attention on every row), "
                      f"{reps} reps, {sec:.3f} s per step, fp64"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    w = workloads.ALL[args.workload]
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    q, k, v = workloads.make_qkv(w, args.layer)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    layout = hm.Layout(w.block, list(w.segments), w.window_tokens)
    head_mask_np = None
    if w.layers > 1:
        head_mask_np = hm.head_mask(workloads.head_importance(w, args.layer))
    elif w.head_mask is not None:
        head_mask_np = np.array(w.head_mask, np.uint8)
    head_mask = None if head_mask_np is None else torch.from_numpy(head_mask_np).to(dev)

    _cls, n_cand = hm.layout_classes(layout, w.N)
    nb = w.nb
    bm = hm.empty_block_mask(w.B, w.H, nb, dev)
    bm_full = hm.empty_block_mask(w.B, w.H, nb, dev)
    ws = torch.empty(hm.select_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.block, w.D),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream(dev)

    def step():
        hm.select(qd, kd, layout, w.budget, out=bm, workspace=ws, stream=stream)
        hm.forward(qd, kd, vd, bm, head_mask, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # One step = select + forward.  By default the step is captured once as a
    # HIP graph and replayed, so the host's per-call launch cost stays out of
    # the GPU timeline; --eager launches every call from the host.
    run_step = step
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                hm.select(qd, kd, layout, w.budget, out=bm, workspace=ws, stream=cap)
                hm.forward(qd, kd, vd, bm, head_mask, out=out, stream=cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        run_step = graph.replay
        for _ in range(args.warmup):
            run_step()
        torch.cuda.synchronize()
    # whole-step throughput: K steps, host clock, synchronised on both sides
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    def timed_launches(fn):
        """Average launch time of fn over K back-to-back launches, HIP events
        recorded on the stream the kernels run on."""
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    sel_ms = timed_launches(lambda: hm.select(qd, kd, layout, w.budget, out=bm, workspace=ws, stream=stream))
    fwd_ms = timed_launches(lambda: hm.forward(qd, kd, vd, bm, head_mask, out=out, stream=stream))
    # the same attention kernel at full density (budget 1.0: same layout and head mask)
    hm.select(qd, kd, layout, 1.0, out=bm_full, workspace=ws, stream=stream)
    dense_ms = timed_launches(lambda: hm.forward(qd, kd, vd, bm_full, head_mask, out=out, stream=stream))

    # the step's own result, outside every timed region
    hm.select(qd, kd, layout, w.budget, out=bm, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    flops = kept_flops(bm.count, head_mask, w.block, w.D, w.H)
    flops_dense = kept_flops(bm_full.count, head_mask, w.block, w.D, w.H)
    sel_bytes = selector_bytes(w, bm, n_cand)
    attn_tflops = flops / (fwd_ms * 1e-3) / 1e12
    sel_gbps = sel_bytes / (sel_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, list(w.segments), head_mask_np, flops)

    if args.calibrate_copy:
        # an elementwise kernel that reads 256 MiB and writes 256 MiB: the known
        # byte count that scales the HBM fetch/write counters
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()

    res = {
        "metric": "block-sparse attn TFLOP/s on kept blocks & speedup vs dense at 30% budget",
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; clustered Q/K for image workloads)",
        "step_launch": "eager" if args.eager else "hip graph replay",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "N": w.N, "D": w.D,
                   "block": w.block, "budget": w.budget, "k": bm.k, "layer": args.layer,
                   "segments": [list(s) for s in w.segments], "window_tokens": w.window_tokens,
                   "active_heads": int(head_mask_np.sum()) if head_mask_np is not None else w.H,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "attn_mfma_kernel" if w.dtype == "bf16" else "attn_vec_kernel",
                     "achieved": attn_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": profiled_traffic(w.name),
                     "traffic_unit": "bytes per launch (HBM fetch + write, rocprofv3 counters)",
                     "flops_per_launch": flops, "avg_launch_ms": fwd_ms},
        "selector": {"bound": "hbm", "achieved": sel_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": sel_gbps / HBM_PEAK_GBPS, "bytes_per_call": sel_bytes, "avg_call_ms": sel_ms},
        "speedup_vs_dense": {"attention": dense_ms / fwd_ms, "step": dense_ms / (sel_ms + fwd_ms),
                             "dense_attention_ms": dense_ms, "dense_flops": flops_dense,
                             "ideal": flops_dense / flops},
        "cpu_baseline": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""), "host": platform.node()},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
