"""bsattn_select_no_alloc (static per-GPU scratch, no workspace argument)
against bsattn_select on the same inputs, through the C ABI.

Two calls in a row, the second on a smaller input, so the second reads a
scratch array that still holds the first call's larger sums.
"""
import ctypes

import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
from head_masked_attention_amd import _binding as B_
import oracle
import workloads
from parity import compare_masks, to64

pytestmark = pytest.mark.gpu


def _c_select_no_alloc(lib, q, k, layout, budget, out, stream):
    tq, tk = B_._tensor(q), B_._tensor(k)
    lay, _keep = layout._c()
    bm = out._c()
    st = lib.bsattn_select_no_alloc(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(lay), float(budget),
                                    ctypes.byref(bm), ctypes.c_void_p(stream.cuda_stream))
    return st, bm


def _garbage_mask(B, H, nb, dev, fill):
    bm = hm.empty_block_mask(B, H, nb, dev)
    bm.mask.fill_(fill)
    bm.count.fill_(-fill)
    bm.index.fill_(fill)
    return bm


def _same_result(a: hm.BlockMask, b: hm.BlockMask):
    ma, ca, ia = a.mask.cpu().numpy(), a.count.cpu().numpy(), a.index.cpu().numpy()
    mb, cb, ib = b.mask.cpu().numpy(), b.count.cpu().numpy(), b.index.cpu().numpy()
    assert np.array_equal(ma, mb)
    assert np.array_equal(ca, cb)
    n = ca.reshape(-1)
    fa, fb = ia.reshape(n.size, -1), ib.reshape(n.size, -1)
    for r in range(n.size):
        assert np.array_equal(fa[r, :n[r]], fb[r, :n[r]]), f"row {r}"


CASES = [
    # (B, H, Hkv, N, D, block, segments, budget, window, seed)
    (1, 8, 8, 512 + 64 * 120, 128, 64, (("text", 100), ("padding", 412), ("image", 64 * 120)), 0.3, 256, 31),
    (2, 2, 1, 64 * 20, 64, 64, (), 0.25, 0, 32),
]


def test_no_alloc_matches_select_on_two_calls_in_a_row(lib, cuda):
    stream = torch.cuda.current_stream(cuda)
    for (B, H, Hkv, N, D, block, segs, budget, window, seed) in CASES:
        print(f"[no-alloc] B{B} H{H} Hkv{Hkv} N{N} D{D} block{block} budget{budget}", flush=True)
        q, k, _ = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=seed)
        qd, kd = q.to(cuda), k.to(cuda)
        layout = hm.Layout(block, list(segs), window)
        nb = N // block
        ref = hm.select(qd, kd, layout, budget, out=_garbage_mask(B, H, nb, cuda, 3))
        out = _garbage_mask(B, H, nb, cuda, 5)
        st, bm = _c_select_no_alloc(lib, qd, kd, layout, budget, out, stream)
        assert st == 0, B_.status_string(st)
        torch.cuda.synchronize()
        assert (bm.k, bm.is_dense) == (ref.k, int(ref.is_dense))
        _same_result(out, ref)
        om, tie = oracle.select(to64(q), to64(k), block, list(segs), budget, window)
        compare_masks(out, om, tie)


def test_no_alloc_dense_budget_and_limit(lib, cuda):
    stream = torch.cuda.current_stream(cuda)
    q, k, _ = workloads.small_case(B=1, H=2, N=64 * 10, D=64, seed=33)
    qd, kd = q.to(cuda), k.to(cuda)
    layout = hm.Layout(64, [])
    ref = hm.select(qd, kd, layout, 1.0, out=_garbage_mask(1, 2, 10, cuda, 3))
    out = _garbage_mask(1, 2, 10, cuda, 5)
    st, bm = _c_select_no_alloc(lib, qd, kd, layout, 1.0, out, stream)
    assert st == 0 and bm.is_dense == 1
    torch.cuda.synchronize()
    _same_result(out, ref)
    # a request whose pooled sums exceed the scratch array is refused before
    # anything is enqueued
    need = hm.select_workspace_bytes(1, 64, 64, 64 * 1024, 64, 128)
    assert need > 32 << 20
    big_q = torch.empty((1, 64, 64 * 1024, 128), dtype=torch.bfloat16, device=cuda)
    big_out = hm.empty_block_mask(1, 64, 1024, cuda)
    st, _ = _c_select_no_alloc(lib, big_q, big_q, layout, 0.3, big_out, stream)
    assert st == 7   # BSATTN_ERR_WORKSPACE
