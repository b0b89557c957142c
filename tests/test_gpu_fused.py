"""GPU parity of bsattn_select_forward (selection and attention in one call)
against the CPU oracle and against bsattn_select followed by bsattn_forward.

Where the fused kernel runs (bf16, D 64, block 64, every block a candidate,
at most 64 blocks) its block mask must equal the oracle's outside near-tie
rows, like bsattn_select's, and its output must match the oracle's attention
over the oracle's mask on those rows at the bf16 bar (max abs 2e-2, mean abs
2e-3).  Rows whose lists equal the separate calls' lists must give the
separate calls' output bit for bit.  Other shapes run the two calls, and must
equal them exactly.
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_close, compare_masks, download_mask, to64

pytestmark = pytest.mark.gpu


def check_fused(cuda, q, k, v, segs, block, budget, window=0, what=""):
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    lay = hm.Layout(block, list(segs), window)
    out, bm = hm.select_forward(qd, kd, vd, lay, budget)
    bm_sep = hm.select(qd, kd, lay, budget)
    out_sep = hm.forward(qd, kd, vd, bm_sep)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    mask, tie = oracle.select(q64, k64, block, list(segs), budget, window)
    compare_masks(bm, mask, tie)
    assert bm.k == bm_sep.k and bm.is_dense == bm_sep.is_dense
    ref = oracle.attention(q64, k64, v64, block, mask)
    got = to64(out)
    keep_rows = np.repeat(tie == 0, block, axis=-1)
    assert_close(got[keep_rows], ref[keep_rows], "bf16", what)
    # every row, near ties included: the attention over the call's own mask
    own = oracle.attention(q64, k64, v64, block, download_mask(bm)[0])
    assert_close(got, own, "bf16", what + " (own mask)")
    same = np.repeat((download_mask(bm)[0] == download_mask(bm_sep)[0]).all(-1), block, axis=-1)
    assert np.array_equal(got[same], to64(out_sep)[same])
    return got


def test_fused_sdxl_workload(cuda):
    w = workloads.SDXL
    q, k, v = workloads.make_qkv(w)
    check_fused(cuda, q, k, v, [], w.block, w.budget, what="fused sdxl")


CASES = [
    # (name, B, H, Hkv, nb, budget)
    ("ragged_37_blocks", 2, 3, 3, 37, 0.3),
    ("max_64_blocks_gqa", 1, 4, 2, 64, 0.25),
    ("mqa_low_budget", 1, 4, 1, 20, 0.05),
    ("two_blocks", 1, 2, 2, 2, 0.5),
    ("all_but_one_block", 1, 2, 2, 20, 0.95),     # k = n - 1: near-full lists, still selective
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_small(cuda, case):
    name, B, H, Hkv, nb, budget = case
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=64 * nb, D=64, seed=301)
    check_fused(cuda, q, k, v, [], 64, budget, what=name)


def test_fused_mixed_magnitude_queries(cuda):
    # query elements spread over seven binades (each scaled by 2^e, e in
    # -6..0, seeded): the 64-token block sums round in fp32, so their value
    # depends on the order of the additions, which the workgroup's own query
    # sum keeps equal to the pool kernel's
    q, k, v = workloads.small_case(B=1, H=4, Hkv=2, N=64 * 48, D=64, seed=303)
    g = torch.Generator().manual_seed(304)
    e = torch.randint(-6, 1, q.shape, generator=g).float()
    q = (q.float() * torch.exp2(e)).to(q.dtype)
    check_fused(cuda, q, k, v, [], 64, 0.3, what="mixed-magnitude queries")


FALLBACK = [
    # shapes the fused kernel does not take: the two calls run
    ("layout_segments", 1, 2, 2, 64 * 12, 64, 64, (("text", 64), ("image", 64 * 11)), 0.3, 0),
    ("window", 1, 2, 2, 64 * 12, 64, 64, (), 0.3, 128),
    ("d128", 1, 2, 2, 64 * 10, 128, 64, (), 0.3, 0),
    ("block32", 1, 2, 2, 32 * 20, 64, 32, (), 0.3, 0),
    ("over_64_blocks", 1, 2, 2, 64 * 70, 64, 64, (), 0.3, 0),
    ("dense_budget", 1, 2, 2, 64 * 10, 64, 64, (), 1.0, 0),
]


@pytest.mark.parametrize("case", FALLBACK, ids=[c[0] for c in FALLBACK])
def test_fused_fallback_equals_two_calls(cuda, case):
    name, B, H, Hkv, N, D, block, segs, budget, window = case
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, block=block, seed=302)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    lay = hm.Layout(block, list(segs), window)
    out, bm = hm.select_forward(qd, kd, vd, lay, budget)
    bm_sep = hm.select(qd, kd, lay, budget)
    out_sep = hm.forward(qd, kd, vd, bm_sep)
    torch.cuda.synchronize()
    (m, c, i), (m2, c2, i2) = download_mask(bm), download_mask(bm_sep)
    assert np.array_equal(m, m2) and np.array_equal(c, c2)
    valid = np.arange(i.shape[-1]) < c[..., None]           # entries past count are unspecified
    assert np.array_equal(i[valid], i2[valid])
    assert torch.equal(out, out_sep)


def test_fused_with_head_mask_runs_the_two_calls(cuda):
    q, k, v = workloads.small_case(B=1, H=4, N=64 * 16, D=64, seed=303)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    hmask = torch.tensor([1, 0, 1, 1], dtype=torch.uint8, device=cuda)
    lay = hm.Layout(64, [])
    out, bm = hm.select_forward(qd, kd, vd, lay, 0.3, hmask)
    out_sep = hm.forward(qd, kd, vd, hm.select(qd, kd, lay, 0.3), hmask)
    torch.cuda.synchronize()
    assert torch.equal(out, out_sep)
    assert bool(torch.all(out[:, 1] == 0))


def test_fused_strided_views(cuda):
    # [B, N, H, D] storage viewed as [B, H, N, D] for Q, K, V and the output
    B, H, nb, D = 2, 4, 24, 64
    N = 64 * nb
    g = torch.Generator().manual_seed(304)
    base = [torch.randn((B, N, H, D), generator=g).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.to(cuda).transpose(1, 2) for t in base)
    out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=cuda).transpose(1, 2)
    got_out, bm = hm.select_forward(q, k, v, hm.Layout(64, []), 0.3, out=out)
    torch.cuda.synchronize()
    assert got_out.data_ptr() == out.data_ptr()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    mask, tie = oracle.select(q64, k64, 64, [], 0.3)
    compare_masks(bm, mask, tie)
    keep_rows = np.repeat(tie == 0, 64, axis=-1)
    ref = oracle.attention(q64, k64, v64, 64, mask)
    assert_close(to64(out)[keep_rows], ref[keep_rows], "bf16", "fused strided views")
