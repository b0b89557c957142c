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

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        hm.select(qd, kd, layout, w.budget, out=bm, workspace=ws, stream=stream)
        ev[i][1].record(stream)
        hm.forward(qd, kd, vd, bm, head_mask, out=out, stream=stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    fwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_per_step = wall * 1e3 / args.steps

    # the same attention kernel at full density (budget 1.0: same layout and head mask)
    hm.select(qd, kd, layout, 1.0, out=bm_full, workspace=ws, stream=stream)
    for _ in range(args.warmup):
        hm.forward(qd, kd, vd, bm_full, head_mask, out=out, stream=stream)
    evd = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        evd[i][0].record(stream)
        hm.forward(qd, kd, vd, bm_full, head_mask, out=out, stream=stream)
        evd[i][1].record(stream)
    torch.cuda.synchronize()
    dense_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evd]))

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
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
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
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.kv_heads, "N": w.N, "D": w.D,
                   "block": w.block, "budget": w.budget, "k": bm.k, "layer": args.layer,
                   "segments": [list(s) for s in w.segments], "window_tokens": w.window_tokens,
                   "active_heads": int(head_mask_np.sum()) if head_mask_np is not None else w.H,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "attn_mfma_kernel" if w.dtype == "bf16" else "attn_vec_kernel",
                     "achieved": attn_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
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
