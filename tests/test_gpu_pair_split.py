"""Seeded random parity cases for how the attention kernel splits a row's
keys between its two wavefront pairs, against the CPU oracle.

At D 64 each pair takes one 32-key half of every kept block; at D 128 the
pairs take alternate kept blocks.  The masks here give rows of one block, two
blocks, odd and even counts and every block, under head masks, GQA and
per-token key masks (random keys, and one half of every block masked, which
leaves one pair with no live key), so that every way a row's work can fall
between the pairs meets the bf16 bar (max abs 2e-2, mean abs 2e-3).  The
fused call's ranking, which the four wavefronts of a workgroup share, is
checked on random short-row shapes the same way as in the fused suite.
Sources: SD.Next commit view, flex-consumer paragraph (only the selected
tiles are computed); haagenti_sparse crate docs (masked heads give zeros).
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_close, to64, upload_mask
from test_gpu_fused import check_fused

pytestmark = pytest.mark.gpu


def draw_rows(rng, B, H, nb):
    """A block mask whose rows keep 1, 2, a random count or all nb blocks."""
    mask = np.zeros((B, H, nb, nb), np.uint8)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                c = int(rng.choice([1, 2, int(rng.integers(1, nb + 1)), int(rng.integers(1, nb + 1)), nb]))
                mask[b, h, i, rng.choice(nb, size=min(c, nb), replace=False)] = 1
    return mask


def draw_key_mask(rng, B, N):
    kind = int(rng.integers(4))
    if kind == 0:
        return None
    km = np.ones((B, N), np.uint8)
    if kind == 1:
        km = (rng.random((B, N)) >= 0.3).astype(np.uint8)
    else:
        half = kind - 2                       # 0: first 32 keys of every block masked, 1: second
        for blk in range(N // 64):
            km[:, 64 * blk + 32 * half:64 * blk + 32 * half + 32] = 0
    return km


@pytest.mark.parametrize("seed", range(24))
def test_pair_split_random_rows(cuda, seed):
    rng = np.random.default_rng(500 + seed)
    D = 64 if seed % 2 == 0 else 128
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.choice([1, 2]))
    nb = int(rng.integers(2, 23))
    N = 64 * nb
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=600 + seed)
    mask = draw_rows(rng, B, H, nb)
    hmask = (rng.random(H) < 0.7).astype(np.uint8) if rng.random() < 0.5 else None
    km = draw_key_mask(rng, B, N)
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda),
                     None if hmask is None else torch.from_numpy(hmask).to(cuda),
                     key_mask=None if km is None else torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, mask, head_mask=hmask, key_mask=km)
    got = to64(out)
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", f"seed {seed} D {D} B{B} H{H}/{Hkv} nb {nb}")
    if hmask is not None:
        assert np.all(got[:, hmask == 0] == 0)


@pytest.mark.parametrize("seed", range(12))
def test_fused_ranking_random_shapes(cuda, seed):
    rng = np.random.default_rng(700 + seed)
    Hkv = int(rng.integers(1, 4))
    H = Hkv * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 3))
    nb = int(rng.integers(2, 65))
    budget = float(rng.uniform(0.05, 0.9))
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=64 * nb, D=64, seed=800 + seed,
                                   scale=float(rng.choice([0.25, 1.0, 4.0])))
    check_fused(cuda, q, k, v, [], 64, budget, what=f"seed {seed} B{B} H{H}/{Hkv} nb {nb} budget {budget:.2f}")
