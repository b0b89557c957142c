"""Seeded synthetic inputs for the tests, the smoke check and the bench.

This module holds input data only: shapes, token layouts, seeds and random
tensors.  It contains none of the method's arithmetic (no pooling, scoring,
ranking, masking or attention) and is the only module the GPU path and the
oracle both receive data from.

The five workloads follow the shapes of the reference pages' scenarios: a tiny
fp32 case, the SDXL self-attention shape (64x64 latent, classifier-free
guidance pair), a joint text+image transformer at 2048x2048 (text padded to
512 tokens, 128x128 image patches), a video length (8 frames of 64x64), and a
64-layer x 32-head stack with per-layer head masks.  No dataset or trained
weights exist here; Q/K for the image workloads carry spatial cluster
structure so that pooled scores are structured the way real activations are.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    block: int
    dtype: str                      # "bf16" or "fp32"
    budget: float
    segments: tuple = ()            # ((kind, length), ...) ; () = no layout
    window_tokens: int = 0
    head_mask: tuple | None = None  # fixed per-head mask, or None
    layers: int = 1
    grid: tuple | None = None       # (frames, rows, cols) of the sparsifiable tokens
    clusters: int = 0               # 16 = a 4x4 tiling of each frame into centroid regions
    cluster_scale: float = 2.0
    radial: bool = False            # also run the radial band control
    seed: int = 0
    notes: str = ""
    Hkv: int = 0                    # 0 = same as H

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def nb(self) -> int:
        return self.N // self.block

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


TINY = Workload(
    name="tiny_fp32", B=1, H=2, N=256, D=32, block=32, dtype="fp32", budget=0.5,
    head_mask=(1, 0), notes="8x8 block grid, Q,K,V iid N(0,1) from seed 0")
SDXL = Workload(
    name="sdxl_bf16", B=2, H=10, N=4096, D=64, block=64, dtype="bf16", budget=0.3,
    grid=(1, 64, 64), clusters=16,
    notes="SDXL self-attention: 64x64 latent, CFG pair, 16 spatial clusters")
JOINT = Workload(
    name="joint_text_image_bf16", B=1, H=24, N=16896, D=128, block=64, dtype="bf16", budget=0.3,
    segments=(("text", 128), ("padding", 384), ("image", 16384)),
    grid=(1, 128, 128), clusters=16,
    notes="2048x2048 joint transformer: text padded to 512 (128 live), 128x128 patches")
VIDEO = Workload(
    name="video_radial_bf16", B=1, H=24, N=33280, D=128, block=64, dtype="bf16", budget=0.3,
    segments=(("text", 128), ("padding", 384), ("video", 32768)),
    grid=(8, 64, 64), radial=True,
    notes="video length: 8 frames of 64x64, text padded to 512 (128 live)")
STACK = Workload(
    name="head_masked_stack_bf16", B=1, H=32, N=4096, D=128, block=64, dtype="bf16", budget=0.3,
    segments=(("conditioning", 64), ("image", 4032)), window_tokens=512, layers=64,
    notes="64 layers x 32 heads; 64 global tokens as a leading pinned prefix; "
          "512-token window; per-layer head masks from U(0,1) importance")

VIDEO_GQA = Workload(
    name="video_gqa_bf16", B=1, H=24, N=33280, D=128, block=64, dtype="bf16", budget=0.3,
    segments=(("text", 128), ("padding", 384), ("video", 32768)),
    grid=(8, 64, 64), Hkv=6, radial=True,
    notes="the video length with grouped K/V heads (4 query heads per K/V head)")

ALL = {w.name: w for w in (TINY, SDXL, JOINT, VIDEO, STACK, VIDEO_GQA)}


def _sparse_span(w: Workload):
    """(start, length) of the sparsifiable tokens (the whole sequence without a layout)."""
    if not w.segments:
        return 0, w.N
    start = 0
    for kind, length in w.segments:
        if kind in ("image", "video"):
            return start, length
        start += length
    return 0, 0


def _cluster_ids(w: Workload) -> np.ndarray:
    """Cluster id per sparsifiable token: a 4x4 tiling of every frame."""
    frames, rows, cols = w.grid
    side = int(round(np.sqrt(w.clusters)))
    r = np.arange(rows)[:, None] * side // rows
    c = np.arange(cols)[None, :] * side // cols
    ids = (r * side + c).ravel()
    return np.tile(ids, frames)


def make_qkv(w: Workload, layer: int = 0, device="cpu"):
    """Q [B,H,N,D], K and V [B,Hkv,N,D] in the workload dtype.

    Draw order from torch.Generator(seed): centroids (clustered workloads),
    then Q noise, K noise, V.  Every value is drawn in fp32 and rounded once
    (round to nearest even) to bf16 for the bf16 workloads.
    """
    seed = w.seed + layer if w.layers > 1 else w.seed
    g = torch.Generator().manual_seed(seed)
    Hkv = w.kv_heads
    mu = None
    if w.clusters:
        mu = torch.randn((w.H, w.clusters, w.D), generator=g, dtype=torch.float32)
    q = torch.randn((w.B, w.H, w.N, w.D), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, Hkv, w.N, w.D), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, Hkv, w.N, w.D), generator=g, dtype=torch.float32)
    if mu is not None:
        s0, n = _sparse_span(w)
        ids = torch.from_numpy(_cluster_ids(w)).long()
        assert ids.numel() == n
        cent = mu[:, ids, :] * w.cluster_scale          # [H, n, D]
        q[:, :, s0:s0 + n, :] += cent[None]
        k[:, :, s0:s0 + n, :] += cent[None, :Hkv]
    dt = w.torch_dtype
    return q.to(dt).to(device), k.to(dt).to(device), v.to(dt).to(device)


def head_importance(w: Workload, layer: int) -> np.ndarray:
    """Per-head importance of one layer: U(0,1)^H from seed 10000 + layer."""
    g = torch.Generator().manual_seed(10000 + layer)
    return torch.rand((w.H,), generator=g, dtype=torch.float64).numpy()


def small_case(B=1, H=2, Hkv=None, N=512, D=64, block=64, dtype="bf16", seed=0, scale=1.0,
               device="cpu"):
    """Generic iid N(0,1)*scale Q/K/V for parity tests at small sizes."""
    Hkv = Hkv or H
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, N, D), generator=g) * scale
    k = torch.randn((B, Hkv, N, D), generator=g) * scale
    v = torch.randn((B, Hkv, N, D), generator=g)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return q.to(dt).to(device), k.to(dt).to(device), v.to(dt).to(device)


def growing_scores_case(B=1, H=2, Hkv=None, nb=10, D=64, step=2.0, jump_block=None, jump=0.0, seed=0):
    """bf16 Q/K/V (block 64) whose scores change steeply from one key block to
    the next: every query row is +-(1 + N(0, 0.05)) in all D entries (the sign
    alternates by row), and every key of block j is s_j + N(0, 0.1) in all
    entries, with s_j = step * j, plus `jump` from block `jump_block` on.  For
    the +1 rows a score grows by about D * step per key block (the -1 rows
    shrink); V is iid N(0, 1).  Used to drive the online softmax through large
    increases of a row's maximum, up to exponentials that overflow fp32."""
    Hkv = Hkv or H
    N = nb * 64
    g = torch.Generator().manual_seed(seed)
    sign = torch.where(torch.arange(N) % 2 == 0, 1.0, -1.0)
    q = sign[None, None, :, None] * (1.0 + 0.05 * torch.randn((B, H, N, D), generator=g))
    level = step * (torch.arange(N) // 64).to(torch.float32)
    if jump_block is not None:
        level = level + jump * (torch.arange(N) // 64 >= jump_block).to(torch.float32)
    k = level[None, None, :, None] + 0.1 * torch.randn((B, Hkv, N, D), generator=g)
    v = torch.randn((B, Hkv, N, D), generator=g)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def random_head_mask(H: int, seed: int) -> np.ndarray:
    """A random 0/1 head mask with at least one active head (test input)."""
    rng = np.random.default_rng(seed)
    m = (rng.random(H) < 0.5).astype(np.uint8)
    m[rng.integers(H)] = 1
    return m
