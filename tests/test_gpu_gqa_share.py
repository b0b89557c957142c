"""GPU parity of the GQA path that shares K/V stage tiles between the query
heads of a group (one block mask for every head, no head mask, an even
number of query heads per K/V head) against the CPU oracle, at the bf16 bar
(max abs 2e-2, mean abs 2e-3): radial and layout-only masks shared by all
heads, no mask at all, a key mask on top, and the cases that must take the
per-head path instead (odd group size, a head mask, per-head masks)."""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_close, to64, upload_mask

pytestmark = pytest.mark.gpu


def run(cuda, q, k, v, mask, **kw):
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), None if mask is None else upload_mask(mask, cuda), **kw)
    torch.cuda.synchronize()
    return to64(out)


@pytest.mark.parametrize("H,Hkv,D", [(8, 2, 128), (4, 2, 64), (6, 1, 128), (4, 1, 64)])
def test_shared_radial_mask(cuda, H, Hkv, D):
    B, N, block = 2, 64 * 14, 64
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=90)
    segs = [("text", 64), ("padding", 64), ("video", N - 128)]
    mask = oracle.radial(N, block, segs, 0.3)           # [NB, NB], one mask for every (b, h)
    got = run(cuda, q, k, v, mask)
    ref = oracle.attention(to64(q), to64(k), to64(v), block, mask)
    assert_close(got, ref, "bf16", f"radial H{H} Hkv{Hkv} D{D}")
    assert np.all(got[:, :, 64:128] == 0)               # dropped padding rows


@pytest.mark.parametrize("D", [64, 128])
def test_no_mask_dense(cuda, D):
    B, H, Hkv, N = 1, 4, 2, 64 * 9
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=91)
    got = run(cuda, q, k, v, None)
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, np.ones((N // 64, N // 64), np.uint8))
    assert_close(got, ref, "bf16", f"dense D{D}")


@pytest.mark.parametrize("D", [64, 128])
def test_shared_mask_with_key_mask(cuda, D):
    B, H, Hkv, N = 2, 4, 2, 64 * 10
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=92)
    nb = N // 64
    rng = np.random.default_rng(93)
    mask = (rng.random((1, 1, nb, nb)) < 0.5).astype(np.uint8)
    mask[0, 0, 2, :] = 0                                # an empty row
    mask[0, 0, 5, :] = 0
    mask[0, 0, 5, 1] = 1                                # only block 1, whose keys are all masked
    km = (rng.random((B, N)) < 0.8).astype(np.uint8)
    km[:, 64:128] = 0
    got = run(cuda, q, k, v, mask, key_mask=torch.from_numpy(km).to(cuda))
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, mask, key_mask=km)
    assert_close(got, ref, "bf16", f"shared mask + key mask D{D}")
    assert np.all(got[:, :, 2 * 64:3 * 64] == 0) and np.all(got[:, :, 5 * 64:6 * 64] == 0)


def test_per_head_fallbacks(cuda):
    """Odd group size, a head mask and per-head masks take the per-head path."""
    B, N, D = 1, 64 * 8, 128
    nb = N // 64
    rng = np.random.default_rng(94)
    shared = (rng.random((1, 1, nb, nb)) < 0.5).astype(np.uint8)
    # odd group size (3 query heads per K/V head)
    q, k, v = workloads.small_case(B=B, H=6, Hkv=2, N=N, D=D, seed=95)
    assert_close(run(cuda, q, k, v, shared), oracle.attention(to64(q), to64(k), to64(v), 64, shared), "bf16", "rep 3")
    # a head mask with a shared block mask
    q, k, v = workloads.small_case(B=B, H=4, Hkv=2, N=N, D=D, seed=96)
    hmask = np.array([1, 0, 1, 1], np.uint8)
    got = run(cuda, q, k, v, shared, head_mask=torch.from_numpy(hmask).to(cuda))
    assert_close(got, oracle.attention(to64(q), to64(k), to64(v), 64, shared, head_mask=hmask), "bf16", "head mask")
    assert np.all(got[:, 1] == 0)
    # per-head masks
    per_head = (rng.random((1, 4, nb, nb)) < 0.5).astype(np.uint8)
    got = run(cuda, q, k, v, per_head)
    assert_close(got, oracle.attention(to64(q), to64(k), to64(v), 64, per_head), "bf16", "per-head masks")


@pytest.mark.parametrize("D,nb", [(128, 10), (64, 9)])
@pytest.mark.parametrize("masked", [False, True], ids=["plain", "key_mask"])
def test_padded_grid_stays_in_bounds(cuda, D, nb, masked):
    # B 1, four query heads on two K/V heads: nb * 2 shared-tile workgroups
    # (20 or 18), a grid padded to 24.  The padding workgroups must exit
    # without touching memory: Q, K, V and O are batch 0 of two-batch
    # buffers, and the output buffer's second batch must keep its fill.
    B, H, Hkv, N = 1, 4, 2, nb * 64
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=97)
    bufs = []
    for t in (q, k, v):
        big = torch.zeros((2,) + tuple(t.shape[1:]), dtype=t.dtype, device=cuda)
        big[:1].copy_(t.to(cuda))
        bufs.append(big[:1])
    out_big = torch.full((2, H, N, D), 7.0, dtype=torch.bfloat16, device=cuda)
    mask = np.ones((1, 1, nb, nb), np.uint8)
    km = np.ones((1, N), np.uint8) if masked else None
    hm.forward(*bufs, upload_mask(mask, cuda), out=out_big[:1],
               key_mask=None if km is None else torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    assert bool(torch.all(out_big[1] == 7.0))
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, mask, key_mask=km)
    assert_close(to64(out_big[:1]), ref, "bf16", f"padded grid D{D} nb{nb}")
