"""GPU parity of bsattn_forward against the CPU oracle.

The GPU forward is fed the oracle's own block mask (uploaded as CSR lists),
so attention parity is independent of selection parity.  bf16 outputs must be
within max abs 2e-2 and mean abs 2e-3 of the fp64 oracle, fp32 outputs within
1e-5.  Large workloads are compared on sampled rows the oracle computes one
by one; masked heads are checked for exact zeros on every row.
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_close, sample_rows, to64, upload_mask

pytestmark = pytest.mark.gpu


def random_mask(B, H, nb, density, seed, empty_rows=True):
    rng = np.random.default_rng(seed)
    m = (rng.random((B, H, nb, nb)) < density).astype(np.uint8)
    if empty_rows:
        m[0, 0, nb // 2, :] = 0
        m[-1, -1, 0, :] = 0
    return m


CASES = [
    # (name, B, H, Hkv, N, D, block, dtype, density)
    ("bf16_d64", 2, 3, 3, 64 * 21, 64, 64, "bf16", 0.4),
    ("bf16_d128", 1, 3, 3, 64 * 19, 128, 64, "bf16", 0.35),
    ("bf16_d128_gqa", 1, 4, 2, 64 * 12, 128, 64, "bf16", 0.5),
    ("bf16_d64_gqa_mqa", 2, 4, 1, 64 * 9, 64, 64, "bf16", 0.6),
    ("fp32_d32_block32", 1, 2, 2, 32 * 16, 32, 32, "fp32", 0.4),
    ("fp32_d64_block64", 1, 2, 2, 64 * 7, 64, 64, "fp32", 0.5),
    ("fp32_d128_block32", 1, 2, 1, 32 * 9, 128, 32, "fp32", 0.5),
    ("bf16_d32_block32_vec", 1, 2, 2, 32 * 11, 32, 32, "bf16", 0.5),
    ("bf16_d128_block32_vec", 1, 2, 2, 32 * 8, 128, 32, "bf16", 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_random_masks(cuda, case):
    name, B, H, Hkv, N, D, block, dtype, density = case
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, block=block, dtype=dtype, seed=5)
    nb = N // block
    mask = random_mask(B, H, nb, density, seed=6)
    hmask = workloads.random_head_mask(H, seed=8)
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda),
                     torch.from_numpy(hmask).to(cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), block, mask, head_mask=hmask)
    got = to64(out)
    assert_close(got, ref, dtype, name)
    assert np.all(got[:, hmask == 0] == 0)
    assert np.all(got[0, 0, (nb // 2) * block:(nb // 2 + 1) * block] == 0)


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (64, "fp32")])
def test_forward_dense_null_mask(cuda, D, dtype):
    q, k, v = workloads.small_case(B=1, H=2, N=64 * 10, D=D, dtype=dtype, seed=9)
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, np.ones((10, 10), np.uint8))
    assert_close(to64(out), ref, dtype)


def test_forward_shared_mask_and_explicit_scale(cuda):
    q, k, v = workloads.small_case(B=2, H=3, N=64 * 8, D=64, seed=10)
    m = random_mask(1, 1, 8, 0.5, seed=11, empty_rows=False)[0, 0]
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(m, cuda), scale=0.05)
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, m, scale=0.05)
    assert_close(to64(out), ref, "bf16")


def test_forward_strided_views(cuda):
    # [B, N, H, D] storage viewed as [B, H, N, D]
    B, H, N, D = 1, 4, 64 * 6, 128
    g = torch.Generator().manual_seed(12)
    base = [torch.randn((B, N, H, D), generator=g).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.to(cuda).transpose(1, 2) for t in base)
    out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=cuda).transpose(1, 2)
    m = random_mask(1, H, 6, 0.6, seed=13, empty_rows=False)
    hm.forward(q, k, v, upload_mask(m, cuda), out=out)
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, m)
    assert_close(to64(out), ref, "bf16")


def test_forward_deterministic(cuda):
    q, k, v = workloads.small_case(B=1, H=4, N=64 * 16, D=128, seed=14, device=cuda)
    m = upload_mask(random_mask(1, 4, 16, 0.4, seed=15), cuda)
    a = hm.forward(q, k, v, m)
    b = hm.forward(q, k, v, m)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- the workloads ---------------------------------------------------------------

def test_forward_tiny_fp32_workload(cuda):
    w = workloads.TINY
    q, k, v = workloads.make_qkv(w)
    mask, tie = oracle.select(to64(q), to64(k), w.block, [], w.budget)
    hmask = np.array(w.head_mask, np.uint8)
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda),
                     torch.from_numpy(hmask).to(cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), w.block, mask, head_mask=hmask)
    got = to64(out)
    assert_close(got, ref, "fp32")
    assert np.all(got[:, 1] == 0)


def test_forward_sdxl_workload_full(cuda):
    w = workloads.SDXL
    q, k, v = workloads.make_qkv(w)
    mask, tie = oracle.select(to64(q), to64(k), w.block, [], w.budget)
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), w.block, mask)
    mx, mean = assert_close(to64(out), ref, "bf16", w.name)
    print(f"[forward {w.name}] max abs {mx:.3g} mean abs {mean:.3g}", flush=True)


def _layout_blocks(w, cls):
    live_pinned = np.nonzero(cls == oracle.PINNED)[0]
    dropped = np.nonzero(cls == oracle.DROPPED)[0]
    sparse = np.nonzero(cls == oracle.SPARSE)[0]

    def pick(b, h, rng):
        chosen = list(live_pinned) + list(dropped[:1]) + [sparse[0], sparse[-1]]
        chosen += list(rng.choice(sparse[1:-1], size=4, replace=False))
        return chosen
    return pick


@pytest.mark.parametrize("name", ["joint_text_image_bf16", "video_radial_bf16", "video_gqa_bf16"])
def test_forward_large_workload_sampled(cuda, name):
    w = workloads.ALL[name]
    q, k, v = workloads.make_qkv(w)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    mask, tie = oracle.select(q64, k64, w.block, list(w.segments), w.budget)
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda))
    torch.cuda.synchronize()
    got = out.cpu()
    cls = oracle.classes(list(w.segments), w.N, w.block)
    rows = sample_rows(w.B, w.H, w.nb, w.block, _layout_blocks(w, cls), 8, seed=16)
    ref = oracle.attention(q64, k64, v64, w.block, mask, rows=rows)
    got_rows = got[rows[:, 0], rows[:, 1], rows[:, 2]].double().numpy()
    mx, mean = assert_close(got_rows, ref, "bf16", name)
    print(f"[forward {name}] {len(rows)} sampled rows: max abs {mx:.3g} mean abs {mean:.3g}", flush=True)
    # dropped (padding) query rows are exactly zero everywhere
    dropped = np.nonzero(cls == oracle.DROPPED)[0]
    for qb in dropped:
        assert torch.all(got[:, :, qb * w.block:(qb + 1) * w.block] == 0)


@pytest.mark.parametrize("name", ["video_radial_bf16", "video_gqa_bf16"])
def test_forward_radial_mask_sampled(cuda, name):
    w = workloads.ALL[name]
    q, k, v = workloads.make_qkv(w)
    lay = hm.Layout(w.block, list(w.segments))
    rad = hm.radial(lay, w.N, w.budget, device=cuda)
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), rad)
    torch.cuda.synchronize()
    ref_mask = oracle.radial(w.N, w.block, list(w.segments), w.budget)
    cls = oracle.classes(list(w.segments), w.N, w.block)
    rows = sample_rows(w.B, w.H, w.nb, w.block, _layout_blocks(w, cls), 4, seed=17)
    ref = oracle.attention(to64(q), to64(k), to64(v), w.block, ref_mask, rows=rows)
    got_rows = out.cpu()[rows[:, 0], rows[:, 1], rows[:, 2]].double().numpy()
    assert_close(got_rows, ref, "bf16", name + " radial")


@pytest.mark.parametrize("layer", [0, 21, 42, 63])
def test_forward_head_masked_stack_layer(cuda, layer):
    w = workloads.STACK
    q, k, v = workloads.make_qkv(w, layer)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    mask, tie = oracle.select(q64, k64, w.block, list(w.segments), w.budget, w.window_tokens)
    hmask = oracle.head_mask(workloads.head_importance(w, layer), 0.5, 4)
    assert hmask.sum() == 16
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda),
                     torch.from_numpy(hmask).to(cuda))
    torch.cuda.synchronize()
    got = out.cpu()
    assert torch.all(got[:, torch.from_numpy(hmask == 0)] == 0)
    active = np.nonzero(hmask)[0]

    def pick(b, h, rng):
        return [0] + list(rng.choice(np.arange(1, w.nb), size=4, replace=False))
    rows = sample_rows(1, w.H, w.nb, w.block, pick, 8, seed=18)
    rows = rows[np.isin(rows[:, 1], active)]
    ref = oracle.attention(q64, k64, v64, w.block, mask, head_mask=hmask, rows=rows)
    got_rows = got[rows[:, 0], rows[:, 1], rows[:, 2]].double().numpy()
    assert_close(got_rows, ref, "bf16", f"stack layer {layer}")


# ---- end to end: the GPU's own selection feeding the GPU forward ----------------

def test_end_to_end_select_forward_sdxl(cuda):
    w = workloads.SDXL
    q, k, v = workloads.make_qkv(w)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    bm = hm.select(qd, kd, hm.Layout(w.block, []), w.budget)
    out = hm.forward(qd, kd, vd, bm)
    dense = hm.forward(qd, kd, vd)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    mask, tie = oracle.select(q64, k64, w.block, [], w.budget)
    ref = oracle.attention(q64, k64, v64, w.block, mask)
    got = to64(out)
    keep_rows = np.repeat(tie == 0, w.block, axis=-1)          # [B,H,N]
    assert_close(got[keep_rows], ref[keep_rows], "bf16", "end to end")
    # clustered Q/K concentrate attention inside the selected blocks, so the
    # 30% selection stays close to dense here
    assert np.abs(got - to64(dense)).max() < 0.1


def test_selection_changes_the_output(cuda):
    # iid inputs spread attention over every block: a selection that stopped
    # changing the output (a dense fallback) fails this
    q, k, v = workloads.small_case(B=1, H=4, N=64 * 32, D=128, seed=21, device=cuda)
    bm = hm.select(q, k, hm.Layout(64, []), 0.3)
    sparse = hm.forward(q, k, v, bm)
    dense = hm.forward(q, k, v)
    torch.cuda.synchronize()
    assert (sparse.float() - dense.float()).abs().max().item() > 10 * 2e-2


def test_padding_contents_do_not_reach_live_rows(cuda):
    w = workloads.JOINT
    q, k, v = workloads.small_case(B=1, H=2, N=w.N, D=128, seed=19, device=cuda)
    lay = hm.Layout(64, list(w.segments))
    a = hm.forward(q, k, v, hm.select(q, k, lay, 0.3))
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in (q2, k2, v2):
        t[:, :, 128:512] = torch.randn_like(t[:, :, 128:512].float()).to(t.dtype) * 30
    b = hm.forward(q2, k2, v2, hm.select(q2, k2, lay, 0.3))
    torch.cuda.synchronize()
    live = torch.cat([torch.arange(0, 128), torch.arange(512, w.N)]).to(cuda)
    assert torch.equal(a[:, :, live], b[:, :, live])
    assert torch.all(b[:, :, 128:512] == 0)


GROWING = [
    # (name, H, Hkv, D, step, jump_block, jump)
    ("d64_steps", 2, 2, 64, 2.0, None, 0.0),
    ("d128_steps", 2, 2, 128, 1.5, None, 0.0),
    ("d64_overflow_jump", 2, 2, 64, 0.5, 6, 25.0),
    ("d128_gqa_shared_overflow_jump", 4, 2, 128, 1.0, 5, 30.0),
]


@pytest.mark.parametrize("case", GROWING, ids=[g[0] for g in GROWING])
@pytest.mark.parametrize("masked", [False, True], ids=["plain", "key_mask"])
def test_forward_steeply_growing_scores(cuda, case, masked):
    # Scores rise by tens of log2 units from one key block to the next (and by
    # hundreds at the jump, where exponentials against the old row maximum
    # overflow fp32), so the online softmax must raise a row's running maximum
    # on stages after its first one; the alternate rows' scores fall instead.
    # Every block is kept, in ascending order, in one mask shared by all heads.
    name, H, Hkv, D, step, jump_block, jump = case
    nb = 10
    q, k, v = workloads.growing_scores_case(B=1, H=H, Hkv=Hkv, nb=nb, D=D, step=step,
                                            jump_block=jump_block, jump=jump, seed=31)
    mask = np.ones((1, 1, nb, nb), np.uint8)
    km = np.ones((1, nb * 64), np.uint8) if masked else None
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda),
                     key_mask=None if km is None else torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, mask, key_mask=km)
    got = to64(out)
    assert np.all(np.isfinite(got))
    assert_close(got, ref, "bf16", f"growing scores {name} {'key mask' if masked else 'plain'}")


@pytest.mark.parametrize("dtype,D,block", [("bf16", 64, 64), ("bf16", 128, 64), ("fp32", 32, 32)])
@pytest.mark.parametrize("active", ["none", "one", "last"])
def test_forward_extreme_head_masks(cuda, dtype, D, block, active):
    """No active head (every output exactly 0), a single active head, and
    only the last head active, with a GQA layout: the head-masked work order
    handles the degenerate counts of active and masked heads."""
    B, H, Hkv, nb = 2, 8, 2, 6
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=nb * block, D=D, block=block, dtype=dtype, seed=95)
    rng = np.random.default_rng(96)
    mask = (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)
    hmask = np.zeros(H, np.uint8)
    if active == "one":
        hmask[3] = 1
    elif active == "last":
        hmask[H - 1] = 1
    out = hm.forward(q.to(cuda), k.to(cuda), v.to(cuda), upload_mask(mask, cuda), torch.from_numpy(hmask).to(cuda))
    torch.cuda.synchronize()
    got = to64(out)
    assert np.all(got[:, hmask == 0] == 0)
    ref = oracle.attention(to64(q), to64(k), to64(v), block, mask, head_mask=hmask)
    assert_close(got, ref, dtype, f"head mask {active}")
