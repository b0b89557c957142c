"""GPU parity of the fp8 (E4M3) consumer against the CPU oracle.

bsattn_quantize_fp8: codes and scales bit-exact against the oracle's
quantiser (every rounding decision is taken in fp32 on both sides).

bsattn_forward_fp8: fed the GPU's own codes and scales, compared with the
fp64 oracle on the dequantized inputs.  The kernel rounds P to E4M3 for the
P V product and sums the same rounded P for the denominators, so the output
is an exact weighted mean of V under weights perturbed by the rounding:
each weight moves by at most 2^-4 of itself (3 mantissa bits, half a step).
With independent roundings the error of an output is about
0.036 * sqrt(sum_j w_j^2 (v_j - o)^2); for rows spread over >= 10 keys and
V ~ N(0, 1) that stays below 0.01 typically and below 0.06 in the worst of
~10^6 outputs, plus bf16 output rounding (2^-9 relative).  Bar: max abs
6e-2, mean abs 6e-3.

Rows whose weight sits on a few keys move by the rounding of those weights
themselves: with two keys of weights w and 1 - w, the output moves by
w (1 - w) |d1 - d2| |v1 - v2| <= 2^-5 |v1 - v2|.  The clustered workloads'
rows (SDXL, joint text+image) are of that kind; rounding P to E4M3 alone
(exact row maximum, round to nearest even, computed on the CPU over the SDXL
workload's 5.2 million outputs) moves them by up to 0.135 (mean 0.0042).
Bar for those workloads: max abs 0.15, mean abs 6e-3.
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import sample_rows, to64, upload_mask

pytestmark = pytest.mark.gpu

FP8_MAX_ABS = 6e-2
FP8_MEAN_ABS = 6e-3
FP8_PEAKED_MAX_ABS = 0.15     # the clustered SDXL workload (rows concentrated on few keys)


@pytest.mark.parametrize("B,H,N,D", [(2, 3, 64 * 5, 128), (1, 4, 64 * 7, 64), (1, 2, 32 * 9, 32)])
def test_quantize_bit_exact(cuda, B, H, N, D):
    q, _, _ = workloads.small_case(B=B, H=H, N=N, D=D, seed=70, scale=3.0)
    q[0, 1] = 0                                    # an all-zero head: scale 1, codes 0
    q[-1, 0, 5, :] *= 40.0                         # one head with a dominant row
    codes, scale = hm.quantize_fp8(q.to(cuda))
    torch.cuda.synchronize()
    ref_codes, ref_scale = oracle.quantize_e4m3(to64(q))
    assert np.array_equal(scale.cpu().numpy(), ref_scale)
    got = codes.cpu().numpy()
    assert np.array_equal(got, ref_codes), f"{int((got != ref_codes).sum())} codes differ"


def run_fp8(cuda, q, k, v, mask=None, hmask=None):
    q8, qs = hm.quantize_fp8(q.to(cuda))
    k8, ks = hm.quantize_fp8(k.to(cuda))
    v8, vs = hm.quantize_fp8(v.to(cuda))
    bm = None if mask is None else upload_mask(mask, cuda)
    hmd = None if hmask is None else torch.from_numpy(hmask).to(cuda)
    out = hm.forward_fp8(q8, k8, v8, qs, ks, vs, bm, hmd)
    torch.cuda.synchronize()
    deq = [oracle.dequantize_e4m3(c.cpu().numpy(), s.cpu().numpy()) for c, s in ((q8, qs), (k8, ks), (v8, vs))]
    return to64(out), deq


def check(got, ref, what, max_abs=FP8_MAX_ABS):
    err = np.abs(got - ref)
    print(f"[fp8 {what}] max abs {err.max():.3g} mean abs {err.mean():.3g}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= max_abs, what
    assert err.mean() <= FP8_MEAN_ABS, what


CASES = [
    # (name, B, H, Hkv, N, D, density)
    ("d128", 1, 3, 3, 64 * 12, 128, 0.4),
    ("d64", 2, 3, 3, 64 * 10, 64, 0.5),
    ("d128_gqa", 1, 4, 2, 64 * 9, 128, 0.5),
    ("d64_mqa", 1, 4, 1, 64 * 8, 64, 0.6),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_fp8_random_masks(cuda, case):
    name, B, H, Hkv, N, D, density = case
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=71)
    nb = N // 64
    rng = np.random.default_rng(72)
    mask = (rng.random((B, H, nb, nb)) < density).astype(np.uint8)
    mask[0, 0, nb // 2, :] = 0                     # an empty row
    hmask = workloads.random_head_mask(H, seed=73)
    got, (qd, kd, vd) = run_fp8(cuda, q, k, v, mask, hmask)
    ref = oracle.attention(qd, kd, vd, 64, mask, head_mask=hmask)
    check(got, ref, name)
    assert np.all(got[:, hmask == 0] == 0)
    assert np.all(got[0, 0, (nb // 2) * 64:(nb // 2 + 1) * 64] == 0)


def test_forward_fp8_dense_sdxl_shape(cuda):
    w = workloads.SDXL
    q, k, v = workloads.make_qkv(w)
    q, k, v = q[:1, :2], k[:1, :2], v[:1, :2]     # two heads of the clustered SDXL inputs
    q8, qs = hm.quantize_fp8(q.contiguous().to(cuda))
    k8, ks = hm.quantize_fp8(k.contiguous().to(cuda))
    v8, vs = hm.quantize_fp8(v.contiguous().to(cuda))
    bm = hm.select(q.contiguous().to(cuda), k.contiguous().to(cuda), hm.Layout(64, []), w.budget)
    out = hm.forward_fp8(q8, k8, v8, qs, ks, vs, bm)
    torch.cuda.synchronize()
    deq = [oracle.dequantize_e4m3(c.cpu().numpy(), s.cpu().numpy()) for c, s in ((q8, qs), (k8, ks), (v8, vs))]
    rows = np.stack([np.zeros(256, int), np.random.default_rng(74).integers(0, 2, 256),
                     np.random.default_rng(75).integers(0, w.N, 256)], 1)
    ref = oracle.attention(*deq, 64, bm.mask.cpu().numpy(), rows=rows)
    got = to64(out)[rows[:, 0], rows[:, 1], rows[:, 2]]
    check(got, ref, "sdxl sampled rows", max_abs=FP8_PEAKED_MAX_ABS)


def test_forward_fp8_sdxl_workload_full(cuda):
    # the bench's fp8 launch: the whole SDXL workload (both batch entries,
    # every head) over the oracle's 30 % selection, every output row
    w = workloads.SDXL
    q, k, v = workloads.make_qkv(w)
    mask, _tie = oracle.select(to64(q), to64(k), w.block, [], w.budget)
    got, (qd, kd, vd) = run_fp8(cuda, q, k, v, mask)
    ref = oracle.attention(qd, kd, vd, 64, mask)
    check(got, ref, "sdxl workload", max_abs=FP8_PEAKED_MAX_ABS)


@pytest.mark.parametrize("name,max_abs", [("joint_text_image_bf16", FP8_PEAKED_MAX_ABS),
                                          ("video_radial_bf16", FP8_MAX_ABS)])
def test_forward_fp8_large_workload_sampled(cuda, name, max_abs):
    # the fp8 launch at the joint text+image (clustered Q/K: peaked rows) and
    # video (iid) sizes over the oracle's selection, on sampled rows of every
    # block class (pinned text rows, sparse rows at both ends, padding rows)
    from test_gpu_forward import _layout_blocks
    w = workloads.ALL[name]
    q, k, v = workloads.make_qkv(w)
    mask, _tie = oracle.select(to64(q), to64(k), w.block, list(w.segments), w.budget)
    got, (qd, kd, vd) = run_fp8(cuda, q, k, v, mask)
    cls = oracle.classes(list(w.segments), w.N, w.block)
    rows = sample_rows(w.B, w.H, w.nb, w.block, _layout_blocks(w, cls), 6, seed=76)
    ref = oracle.attention(qd, kd, vd, w.block, mask, rows=rows)
    check(got[rows[:, 0], rows[:, 1], rows[:, 2]], ref, f"{name} sampled rows", max_abs=max_abs)
    dropped = np.nonzero(cls == oracle.DROPPED)[0]
    for qb in dropped:
        assert np.all(got[:, :, qb * w.block:(qb + 1) * w.block] == 0)


def key_mask_fp8(B, N, seed):
    """Live keys with the structure of padded prompts: a masked tail per batch,
    one wholly masked 64-key block, one partly masked block, random holes."""
    rng = np.random.default_rng(seed)
    km = (rng.random((B, N)) < 0.85).astype(np.uint8)
    km[:, 64:128] = 0                              # a whole key block masked
    km[:, 128:160] = 0                             # half of the next one
    km[-1, N - 96:] = 0                            # a masked tail on the last batch entry
    return km


@pytest.mark.parametrize("case", CASES[:2] + CASES[2:3], ids=[c[0] for c in CASES[:2] + CASES[2:3]])
def test_forward_fp8_key_mask(cuda, case):
    name, B, H, Hkv, N, D, density = case
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=76)
    nb = N // 64
    rng = np.random.default_rng(77)
    mask = (rng.random((B, H, nb, nb)) < density).astype(np.uint8)
    mask[:, :, :, 1] = 1                           # every row keeps the wholly masked block
    mask[0, 0, 3, :] = 0
    mask[0, 0, 3, 1] = 1                           # a row whose only kept block is wholly masked
    hmask = workloads.random_head_mask(H, seed=78)
    km = key_mask_fp8(B, N, 79)
    q8, qs = hm.quantize_fp8(q.to(cuda))
    k8, ks = hm.quantize_fp8(k.to(cuda))
    v8, vs = hm.quantize_fp8(v.to(cuda))
    out = hm.forward_fp8(q8, k8, v8, qs, ks, vs, upload_mask(mask, cuda), torch.from_numpy(hmask).to(cuda),
                         key_mask=torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    deq = [oracle.dequantize_e4m3(c.cpu().numpy(), s.cpu().numpy()) for c, s in ((q8, qs), (k8, ks), (v8, vs))]
    ref = oracle.attention(*deq, 64, mask, head_mask=hmask, key_mask=km)
    got = to64(out)
    check(got, ref, name + " key mask")
    assert np.all(got[:, hmask == 0] == 0)
    if hmask[0]:
        assert np.all(got[0, 0, 3 * 64:4 * 64] == 0)   # every kept key masked: zero row


def test_forward_fp8_key_mask_all_live_and_shared(cuda):
    B, H, N, D = 2, 2, 64 * 8, 128
    q, k, v = workloads.small_case(B=B, H=H, N=N, D=D, seed=80)
    nb = N // 64
    mask = (np.random.default_rng(81).random((B, H, nb, nb)) < 0.5).astype(np.uint8)
    bm = upload_mask(mask, cuda)
    q8, qs = hm.quantize_fp8(q.to(cuda))
    k8, ks = hm.quantize_fp8(k.to(cuda))
    v8, vs = hm.quantize_fp8(v.to(cuda))
    plain = hm.forward_fp8(q8, k8, v8, qs, ks, vs, bm)
    live = hm.forward_fp8(q8, k8, v8, qs, ks, vs, bm, key_mask=torch.ones(B, N, dtype=torch.uint8, device=cuda))
    km1 = key_mask_fp8(1, N, 82)[0]
    shared = hm.forward_fp8(q8, k8, v8, qs, ks, vs, bm, key_mask=torch.from_numpy(km1).to(cuda))
    torch.cuda.synchronize()
    assert torch.equal(plain, live)               # all-live stages run the unmasked arithmetic
    deq = [oracle.dequantize_e4m3(c.cpu().numpy(), s.cpu().numpy()) for c, s in ((q8, qs), (k8, ks), (v8, vs))]
    ref = oracle.attention(*deq, 64, mask, key_mask=km1)
    check(to64(shared), ref, "shared key mask")


def draw_fp8_case(seed: int) -> dict:
    rng = np.random.default_rng(9000 + seed)
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 4))
    H = Hkv * int(rng.choice([1, 2, 4]))
    nb = int(rng.integers(3, 41))
    density = float(rng.choice([0.1, 0.3, 0.6, 1.0]))
    use_hmask = bool(rng.random() < 0.4)
    use_kmask = bool(rng.random() < 0.4)
    return dict(seed=seed, D=D, B=B, H=H, Hkv=Hkv, nb=nb, density=density, hmask=use_hmask, kmask=use_kmask)


FP8_RANDOM = [draw_fp8_case(s) for s in range(20)]


@pytest.mark.parametrize("c", FP8_RANDOM, ids=[f"s{c['seed']}_d{c['D']}_B{c['B']}H{c['H']}kv{c['Hkv']}_n{c['nb']}"
                                               for c in FP8_RANDOM])
def test_forward_fp8_random_configs(cuda, c):
    """Seeded shapes, densities (every row keeps its diagonal block), head and
    key masks through quantize + forward_fp8: codes bit-exact, outputs within
    the fp8 bar of the oracle on the dequantized inputs, masked heads exactly
    zero.  Q, K and V are N(0, 1), the regime the bar is derived for: with Q
    and K at 1.5x the rows are peakier, and rounding P to E4M3 alone (a CPU
    emulation with the exact row maximum) then moves some outputs by 0.086."""
    B, H, Hkv, nb, D = c["B"], c["H"], c["Hkv"], c["nb"], c["D"]
    N = 64 * nb
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, seed=9100 + c["seed"])
    rng = np.random.default_rng(9200 + c["seed"])
    mask = (rng.random((B, H, nb, nb)) < c["density"]).astype(np.uint8)
    mask[:, :, np.arange(nb), np.arange(nb)] = 1
    hmask = workloads.random_head_mask(H, seed=9300 + c["seed"]) if c["hmask"] else None
    km = key_mask_fp8(B, N, 9400 + c["seed"]) if c["kmask"] else None
    q8, qs = hm.quantize_fp8(q.to(cuda))
    k8, ks = hm.quantize_fp8(k.to(cuda))
    v8, vs = hm.quantize_fp8(v.to(cuda))
    out = hm.forward_fp8(q8, k8, v8, qs, ks, vs, upload_mask(mask, cuda),
                         None if hmask is None else torch.from_numpy(hmask).to(cuda),
                         key_mask=None if km is None else torch.from_numpy(km).to(cuda))
    torch.cuda.synchronize()
    for codes, scale, x in ((q8, qs, q), (k8, ks, k), (v8, vs, v)):
        ref_codes, ref_scale = oracle.quantize_e4m3(to64(x))
        assert np.array_equal(scale.cpu().numpy(), ref_scale)
        assert np.array_equal(codes.cpu().numpy(), ref_codes)
    deq = [oracle.dequantize_e4m3(cc.cpu().numpy(), s.cpu().numpy()) for cc, s in ((q8, qs), (k8, ks), (v8, vs))]
    ref = oracle.attention(*deq, 64, mask, head_mask=hmask, key_mask=km)
    got = to64(out)
    check(got, ref, f"random s{c['seed']}")
    if hmask is not None:
        assert np.all(got[:, hmask == 0] == 0)
