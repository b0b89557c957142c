"""Seeded random configurations through select, forward and select_forward,
against the CPU oracle.

Each case draws its own shape (batch, query and K/V heads, head dim, block,
dtype, length), layout (segments of every kind, lengths not aligned to the
block), window, budget (dense budgets included), head mask and per-token key
mask, so that combinations no hand-written case covers still meet the same
bar: block masks bit-exact outside the oracle's near-tie rows, and outputs
within the dtype's tolerance of the oracle's attention over the oracle's mask
(SD.Next commit view: the selector, layout and flex-consumer paragraphs;
haagenti_sparse crate docs for the head mask).  Where the fused call applies
it is checked the same way.
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_close, compare_masks, download_mask, to64, upload_mask

pytestmark = pytest.mark.gpu

KINDS = ["text", "conditioning", "audio", "other", "image", "video", "padding"]


def draw_case(seed: int) -> dict:
    rng = np.random.default_rng(1000 + seed)
    dtype = "fp32" if rng.random() < 0.2 else "bf16"
    block = 32 if (dtype == "fp32" or rng.random() < 0.2) else 64
    D = int(rng.choice([32, 64, 128]))
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 4))
    H = Hkv * int(rng.choice([1, 2, 4]))
    nb = int(rng.integers(3, 41))
    N = nb * block
    segs = []
    if rng.random() < 0.6:
        # 1 to 4 segments, lengths not aligned to the block, summing to N
        n_seg = int(rng.integers(1, 5))
        cuts = np.sort(rng.choice(np.arange(1, N), size=n_seg - 1, replace=False)) if n_seg > 1 else []
        bounds = [0, *[int(c) for c in cuts], N]
        segs = [(KINDS[int(rng.integers(len(KINDS)))], bounds[i + 1] - bounds[i]) for i in range(n_seg)]
    window = int(rng.choice([0, 0, block // 2, 2 * block, 3 * block + 16]))
    budget = float(rng.choice([rng.uniform(0.05, 0.95), rng.uniform(0.05, 0.95), 1.0]))
    head_mask = (rng.random(H) < 0.6).astype(np.uint8) if rng.random() < 0.4 else None
    key_mask = None
    if rng.random() < 0.3:
        key_mask = (rng.random((B, N)) >= rng.choice([0.1, 0.5])).astype(np.uint8)
        if rng.random() < 0.5:
            key_mask[:, block:2 * block] = 0            # one wholly masked key block
    return dict(seed=seed, dtype=dtype, block=block, D=D, B=B, H=H, Hkv=Hkv, N=N, segs=segs,
                window=window, budget=budget, head_mask=head_mask, key_mask=key_mask)


CASES = [draw_case(s) for s in range(60)]


def case_id(c):
    return (f"s{c['seed']}_{c['dtype']}_b{c['block']}_d{c['D']}_B{c['B']}H{c['H']}kv{c['Hkv']}"
            f"_n{c['N'] // c['block']}_seg{len(c['segs'])}")


@pytest.mark.parametrize("c", CASES, ids=[case_id(c) for c in CASES])
def test_random_config(cuda, c):
    q, k, v = workloads.small_case(B=c["B"], H=c["H"], Hkv=c["Hkv"], N=c["N"], D=c["D"], block=c["block"],
                                   dtype=c["dtype"], seed=500 + c["seed"])
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    lay = hm.Layout(c["block"], list(c["segs"]), c["window"])
    q64, k64, v64 = to64(q), to64(k), to64(v)

    # selection
    bm = hm.select(qd, kd, lay, c["budget"])
    torch.cuda.synchronize()
    ref, tie = oracle.select(q64, k64, c["block"], list(c["segs"]), c["budget"], c["window"])
    compare_masks(bm, ref, tie)
    n_cand = int((oracle.classes(list(c["segs"]), c["N"], c["block"]) == 0).sum())
    if n_cand > 0:
        k_ref, dense_ref = oracle.budget(n_cand, c["budget"])
        assert bm.k == k_ref and bool(bm.is_dense) == bool(dense_ref)

    # attention over the oracle's mask (near-tie rows included: both sides see the same mask)
    hmask = None if c["head_mask"] is None else torch.from_numpy(c["head_mask"]).to(cuda)
    kmask = None if c["key_mask"] is None else torch.from_numpy(c["key_mask"]).to(cuda)
    out = hm.forward(qd, kd, vd, upload_mask(ref, cuda), hmask, key_mask=kmask)
    torch.cuda.synchronize()
    want = oracle.attention(q64, k64, v64, c["block"], ref, head_mask=c["head_mask"], key_mask=c["key_mask"])
    got = to64(out)
    assert_close(got, want, c["dtype"], case_id(c))
    if c["head_mask"] is not None:
        assert np.all(got[:, c["head_mask"] == 0] == 0)

    # the call's own mask gives the oracle's attention over that mask too
    own = download_mask(bm)[0]
    out_own = hm.forward(qd, kd, vd, bm, hmask, key_mask=kmask)
    torch.cuda.synchronize()
    want_own = oracle.attention(q64, k64, v64, c["block"], own, head_mask=c["head_mask"],
                                key_mask=c["key_mask"])
    assert_close(to64(out_own), want_own, c["dtype"], case_id(c) + " (own mask)")

    # select + forward in one call (fused where it applies, else the two calls)
    if c["key_mask"] is None:
        out_f, bm_f = hm.select_forward(qd, kd, vd, lay, c["budget"], hmask)
        torch.cuda.synchronize()
        compare_masks(bm_f, ref, tie)
        want_f = oracle.attention(q64, k64, v64, c["block"], download_mask(bm_f)[0], head_mask=c["head_mask"])
        assert_close(to64(out_f), want_f, c["dtype"], case_id(c) + " (select_forward)")


def draw_long_case(seed: int) -> dict:
    """Selections over 129 to 520 blocks (the radix-ranked rows): random
    layouts with pinned and dropped runs, windows, GQA and budgets from a
    single kept candidate up to all but one."""
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([32, 64, 128]))
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.choice([1, 2]))
    nb = int(rng.integers(129, 521))
    N = nb * 64
    segs = []
    if rng.random() < 0.7:
        n_seg = int(rng.integers(2, 6))
        cuts = np.sort(rng.choice(np.arange(1, N), size=n_seg - 1, replace=False))
        bounds = [0, *[int(c) for c in cuts], N]
        segs = [(KINDS[int(rng.integers(len(KINDS)))], bounds[i + 1] - bounds[i]) for i in range(n_seg)]
        if not any(kd in ("image", "video") for kd, _ in segs):
            segs[-1] = ("video", segs[-1][1])
    window = int(rng.choice([0, 0, 96, 640]))
    mode = rng.random()
    budget = float(rng.uniform(0.05, 0.95)) if mode < 0.7 else (1e-4 if mode < 0.85 else 0.995)
    return dict(seed=seed, D=D, H=H, Hkv=Hkv, N=N, segs=segs, window=window, budget=budget)


LONG_CASES = [draw_long_case(s) for s in range(24)]


@pytest.mark.parametrize("c", LONG_CASES, ids=[f"s{c['seed']}_d{c['D']}_H{c['H']}kv{c['Hkv']}_n{c['N'] // 64}"
                                                f"_seg{len(c['segs'])}" for c in LONG_CASES])
def test_random_long_selection(cuda, c):
    q, k, _ = workloads.small_case(B=1, H=c["H"], Hkv=c["Hkv"], N=c["N"], D=c["D"], seed=7000 + c["seed"])
    lay = hm.Layout(64, list(c["segs"]), c["window"])
    bm = hm.select(q.to(cuda), k.to(cuda), lay, c["budget"])
    torch.cuda.synchronize()
    ref, tie = oracle.select(to64(q), to64(k), 64, list(c["segs"]), c["budget"], c["window"])
    compare_masks(bm, ref, tie)
