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
from parity import assert_close, compare_masks, download_mask, to64, upload_mask

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


def test_stage_schedule_against_the_oracle(cuda):
    """sparse_attention over a two-value budget schedule with a token key
    mask, each served step checked against the oracle: the block mask against
    oracle.select at that step's budget (bit-exact outside near-tie rows), the
    output against oracle.attention with the key mask on the GPU's own mask
    (every row) and on the oracle's mask (rows without near ties).  A call the
    stage declines as short is the oracle's dense attention with the key mask."""
    segs = [("text", 100), ("padding", 60), ("image", 64 * 24 - 160)]
    N = sum(n for _, n in segs)
    B, H, D = 2, 3, 64
    q, k, v = workloads.small_case(B=B, H=H, N=N, D=D, seed=41)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    rng = np.random.default_rng(42)
    km = (rng.random((B, N)) > 0.05).astype(np.uint8)      # scattered masked keys
    km[:, 100:160] = 0                                      # the padding tokens
    km[1, N - 64 + 7:] = 0                                  # most of batch 1's last block
    kmd = torch.from_numpy(km).to(cuda)
    lay = hm.Layout(64, segs)
    stage = hm.Stage(min_length=1024, n_steps=4, schedule=(0.5, 0.25, 2))
    bm = hm.empty_block_mask(B, H, N // 64, cuda)
    seen = set()
    for step, budget in ((0, 0.5), (1, 0.5), (2, 0.25), (3, 0.25), (7, 0.25)):
        out, d = hm.sparse_attention(qd, kd, vd, stage, lay, step=step, key_mask=kmd, block_mask=bm)
        torch.cuda.synchronize()
        assert d["outcome"] == hm.STAGE_SPARSE and d["budget"] == budget and d["use_key_mask"]
        ref_mask, tie = oracle.select(q64, k64, 64, segs, budget)
        compare_masks(bm, ref_mask, tie)
        own = bm.mask.cpu().numpy()
        got = to64(out)
        assert_close(got, oracle.attention(q64, k64, v64, 64, own, key_mask=km), "bf16", f"step {step}")
        rows = np.repeat(tie == 0, 64, axis=-1)
        ref = oracle.attention(q64, k64, v64, 64, ref_mask, key_mask=km)
        assert_close(got[rows], ref[rows], "bf16", f"step {step} oracle mask")
        seen.add(budget)
    assert seen == {0.5, 0.25}
    # declined: shorter than the stage's minimum length -> dense with the key mask
    short = hm.Stage(min_length=8192)
    out, d = hm.sparse_attention(qd, kd, vd, short, lay, key_mask=kmd)
    torch.cuda.synchronize()
    assert d["outcome"] == hm.DECLINE_SHORT
    ones = np.ones((N // 64, N // 64), np.uint8)
    assert_close(to64(out), oracle.attention(q64, k64, v64, 64, ones, key_mask=km), "bf16", "declined short")


@pytest.mark.parametrize("dtype,D,block", [("bf16", 64, 64), ("bf16", 128, 64), ("fp32", 64, 32)])
def test_every_key_masked_gives_zero(cuda, dtype, D, block):
    """A key mask that masks every key of one batch entry, and for the other
    only the keys of the last key block: the first entry's rows are all exactly
    0 (no live key in any kept block), the second entry's rows follow the oracle
    (rows that keep only the last block are 0 as well).  bf16 and fp32 paths,
    and the fp8 consumer for the bf16 shapes."""
    B, H, Hkv, nb = 2, 4, 2, 7
    N = nb * block
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, block=block, dtype=dtype, seed=97)
    rng = np.random.default_rng(98)
    mask = (rng.random((B, H, nb, nb)) < 0.4).astype(np.uint8)
    mask[1, 0, 2, :] = 0
    mask[1, 0, 2, nb - 1] = 1                     # a row keeping only the last block
    km = np.ones((B, N), np.uint8)
    km[0, :] = 0
    km[1, (nb - 1) * block:] = 0
    kmd = torch.from_numpy(km).to(cuda)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    out = hm.forward(qd, kd, vd, upload_mask(mask, cuda), key_mask=kmd)
    torch.cuda.synchronize()
    got = to64(out)
    assert np.all(got[0] == 0)
    assert np.all(got[1, 0, 2 * block:3 * block] == 0)
    ref = oracle.attention(to64(q), to64(k), to64(v), block, mask, key_mask=km)
    assert_close(got, ref, dtype, "every key masked")
    if dtype == "bf16":
        q8, qs = hm.quantize_fp8(qd)
        k8, ks = hm.quantize_fp8(kd)
        v8, vs = hm.quantize_fp8(vd)
        out8 = hm.forward_fp8(q8, k8, v8, qs, ks, vs, upload_mask(mask, cuda), key_mask=kmd)
        torch.cuda.synchronize()
        got8 = to64(out8)
        assert np.all(got8[0] == 0)
        assert np.all(got8[1, 0, 2 * block:3 * block] == 0)


def test_sparse_attention_under_a_head_mask(cuda):
    """A served call with a head mask selects only the active heads
    (bsattn_select_heads): the output equals the forward over a full
    selection under the same head mask, and the selection's rows of the
    masked heads are empty."""
    segs = [("conditioning", 64), ("image", 64 * 20)]
    N = sum(n for _, n in segs)
    H = 4
    q, k, v = workloads.small_case(B=1, H=H, Hkv=2, N=N, D=128, seed=33)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    hmask = np.array([0, 1, 1, 0], np.uint8)
    hmd = torch.from_numpy(hmask).to(cuda)
    lay = hm.Layout(64, segs, 256)
    stage = hm.Stage(min_length=512, n_steps=4, schedule=0.3)
    bm = hm.empty_block_mask(1, H, N // 64, cuda)
    out, d = hm.sparse_attention(qd, kd, vd, stage, lay, step=1, head_mask=hmd, block_mask=bm)
    torch.cuda.synchronize()
    assert d["outcome"] == hm.STAGE_SPARSE
    ref = hm.forward(qd, kd, vd, hm.select(qd, kd, lay, d["budget"]), hmd)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    m, c, _ = download_mask(bm)
    assert not m[:, hmask == 0].any() and not c[:, hmask == 0].any()
    assert c[:, hmask != 0].all()


@pytest.mark.parametrize("pattern", ["second_half", "first_half", "alternating"])
@pytest.mark.parametrize("D", [64, 128])
def test_key_mask_one_half_of_every_block(cuda, pattern, D):
    # the two wavefront pairs of a workgroup take the two 32-key halves of
    # every kept block (D 64) or alternate kept blocks (D 128): masking one
    # half of every block leaves one pair with no live key at all, and rows
    # with one, two or an odd number of kept blocks split unevenly
    B, H, nb = 1, 3, 9
    N = 64 * nb
    q, k, v = workloads.small_case(B=B, H=H, N=N, D=D, seed=41)
    rng = np.random.default_rng(42)
    mask = (rng.random((B, H, nb, nb)) < 0.55).astype(np.uint8)
    mask[0, 0, 0, :] = 0
    mask[0, 0, 0, 4] = 1                 # one kept block
    mask[0, 1, 2, :] = 0
    mask[0, 1, 2, [1, 7]] = 1            # two
    mask[0, 2, 5, :] = 1                 # every block (nine)
    km = np.ones((B, N), np.uint8)
    for blk in range(nb):
        lo = 64 * blk
        if pattern == "second_half" or (pattern == "alternating" and blk % 2 == 0):
            km[:, lo + 32:lo + 64] = 0
        else:
            km[:, lo:lo + 32] = 0
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda),
                     key_mask=torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, mask, key_mask=km)
    got = to64(out)
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", f"{pattern}_d{D}")


def test_key_mask_sdxl_workload_full(cuda):
    # the bench's key-mask launch: the SDXL workload's 30 % selection with the
    # last N/16 keys of every batch entry masked, every output row against
    # the oracle
    w = workloads.SDXL
    q, k, v = workloads.make_qkv(w)
    mask, _tie = oracle.select(to64(q), to64(k), w.block, [], w.budget)
    km = np.ones((w.B, w.N), np.uint8)
    km[:, w.N - w.N // 16:] = 0
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda),
                     key_mask=torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), w.block, mask, key_mask=km)
    got = to64(out)
    assert np.isfinite(got).all()
    mx, mean = assert_close(got, ref, "bf16", "sdxl key mask")
    print(f"[key mask sdxl] max abs {mx:.3g} mean abs {mean:.3g}", flush=True)
