"""GPU parity of bsattn_forward_masked (per-token key mask composed with the
block mask) against the CPU oracle.

Covers the MFMA path (D 64 and 128, GQA) and the fp32 / block-32 vector path,
stages whose 32 keys are partly masked, wholly masked and all live, query
blocks whose every kept key is masked (output exactly 0), a mask shared by the
batch, a strided mask, and a packed layout whose segments are not
block-aligned: padding tokens inside pinned tiles masked per token, the
straddling tiles then exact.  Tolerances as for bsattn_forward.
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_close, to64, upload_mask

pytestmark = pytest.mark.gpu

CASES = [
    # (name, B, H, Hkv, N, D, block, dtype, density)
    ("bf16_d64", 2, 3, 3, 64 * 13, 64, 64, "bf16", 0.5),
    ("bf16_d128", 1, 3, 3, 64 * 11, 128, 64, "bf16", 0.5),
    ("bf16_d128_gqa", 1, 4, 2, 64 * 9, 128, 64, "bf16", 0.6),
    ("bf16_d64_mqa", 2, 4, 1, 64 * 7, 64, 64, "bf16", 0.6),
    ("fp32_d64_block64", 1, 2, 2, 64 * 6, 64, 64, "fp32", 0.6),
    ("fp32_d32_block32", 2, 2, 1, 32 * 10, 32, 32, "fp32", 0.5),
    ("bf16_d128_block32_vec", 1, 2, 2, 32 * 8, 128, 32, "bf16", 0.6),
]


def key_mask_for(B, N, block, seed):
    """Random live keys plus structured stretches: a wholly masked 32-key
    stage, a partly masked one, and a wholly masked block."""
    rng = np.random.default_rng(seed)
    km = (rng.random((B, N)) < 0.8).astype(np.uint8)
    km[:, 32:64] = 0                     # one 32-key stage entirely masked
    km[:, 64:96] = 1
    km[:, 70:73] = 0                     # a few keys of the next stage
    km[-1, 2 * block:3 * block] = 0      # a whole block of the last batch
    return km


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_key_mask_random(cuda, case):
    name, B, H, Hkv, N, D, block, dtype, density = case
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, block=block, dtype=dtype, seed=21)
    nb = N // block
    rng = np.random.default_rng(22)
    mask = (rng.random((B, H, nb, nb)) < density).astype(np.uint8)
    mask[0, 0, 1, :] = 0
    mask[0, 0, 1, 1] = 1                 # keeps only block 1 (wholly masked keys 32..63 when block = 32)
    km = key_mask_for(B, N, block, 23)
    # a query block of the last batch that keeps only the wholly masked block
    mask[-1, -1, 0, :] = 0
    mask[-1, -1, 0, 2] = 1
    hmask = workloads.random_head_mask(H, seed=24)
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda),
                     torch.from_numpy(hmask).to(cuda), key_mask=torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), block, mask, head_mask=hmask, key_mask=km)
    got = to64(out)
    assert np.isfinite(got).all()
    assert_close(got, ref, dtype, name)
    assert np.all(got[:, hmask == 0] == 0)
    if hmask[-1]:
        assert np.all(got[-1, -1, 0:block] == 0)      # every kept key masked: exactly 0


def test_key_mask_all_live_equals_unmasked(cuda):
    q, k, v = workloads.small_case(B=2, H=3, N=64 * 12, D=64, seed=25)
    nb = 12
    mask = (np.random.default_rng(26).random((2, 3, nb, nb)) < 0.5).astype(np.uint8)
    bm = upload_mask(mask, cuda)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    a = hm.forward(qd, kd, vd, bm)
    b = hm.forward(qd, kd, vd, bm, key_mask=torch.ones(2, 64 * 12, dtype=torch.uint8, device=cuda))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_key_mask_shared_and_strided(cuda):
    B, H, N, D, block = 2, 2, 64 * 8, 128, 64
    q, k, v = workloads.small_case(B=B, H=H, N=N, D=D, seed=27)
    mask = (np.random.default_rng(28).random((B, H, 8, 8)) < 0.6).astype(np.uint8)
    km1 = (np.random.default_rng(29).random(N) < 0.7).astype(np.uint8)
    bm = upload_mask(mask, cuda)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    shared = hm.forward(qd, kd, vd, bm, key_mask=torch.from_numpy(km1).to(cuda))
    big = torch.zeros(B, N + 96, dtype=torch.uint8, device=cuda)
    big[:, :N] = torch.from_numpy(km1).to(cuda)
    strided = hm.forward(qd, kd, vd, bm, key_mask=big[:, :N])
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), block, mask, key_mask=km1)
    assert_close(to64(shared), ref, "bf16")
    assert torch.equal(shared, strided)


def test_straddling_layout_exact_with_token_mask(cuda):
    # text 100 live + 60 padding tokens: blocks 0..2 straddle text/padding and
    # are pinned; masking the padding tokens per key makes those tiles exact
    # (the padding keys never reach a row), as the masked_block backend does
    segs = [("text", 100), ("padding", 60), ("image", 64 * 10 - 160 + 64 * 6)]
    N = sum(n for _, n in segs)
    assert N % 64 == 0
    B, H, D = 1, 3, 64
    q, k, v = workloads.small_case(B=B, H=H, N=N, D=D, seed=30)
    km = np.ones((B, N), np.uint8)
    km[:, 100:160] = 0
    lay = hm.Layout(64, segs)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    bm = hm.select(qd, kd, lay, 0.4)
    out = hm.forward(qd, kd, vd, bm, key_mask=torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    m = bm.mask.cpu().numpy()
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, m, key_mask=km)
    got = to64(out)
    assert_close(got, ref, "bf16")
    # the padding keys never reach a row: changing them leaves every output unchanged
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 100:160] = 9.0
    v2[:, :, 100:160] = -9.0
    out2 = hm.forward(qd, k2.to(cuda), v2.to(cuda), bm, key_mask=torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_sparse_attention_through_the_stage(cuda):
    # the stage serves a long self-attention call (select + forward, with the
    # token mask), declines a short one (dense through the same kernel) and
    # hands a causal one back to the caller
    segs = [("text", 100), ("padding", 60), ("image", 64 * 10 - 160 + 64 * 6)]
    N = sum(n for _, n in segs)
    q, k, v = workloads.small_case(B=1, H=2, N=N, D=64, seed=31)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    km = np.ones((1, N), np.uint8)
    km[:, 100:160] = 0
    kmd = torch.from_numpy(km).to(cuda)
    lay = hm.Layout(64, segs)
    stage = hm.Stage(min_length=512, n_steps=4, schedule=(0.5, 0.25, 2))
    out, d = hm.sparse_attention(qd, kd, vd, stage, lay, step=3, key_mask=kmd)
    torch.cuda.synchronize()
    assert d["outcome"] == hm.STAGE_SPARSE and d["budget"] == 0.25 and d["use_key_mask"]
    bm = hm.select(qd, kd, lay, 0.25)
    ref = hm.forward(qd, kd, vd, bm, key_mask=kmd)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    short = hm.Stage(min_length=4096)
    out2, d2 = hm.sparse_attention(qd, kd, vd, short, lay)
    torch.cuda.synchronize()
    assert d2["outcome"] == hm.DECLINE_SHORT and d2["first_report"]
    assert torch.equal(out2, hm.forward(qd, kd, vd))
    out3, d3 = hm.sparse_attention(qd, kd, vd, stage, lay, causal=True)
    assert out3 is None and d3["outcome"] == hm.DECLINE_CAUSAL
