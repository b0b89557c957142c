"""GPU parity of bsattn_select and bsattn_radial against the CPU oracle.

Block masks must be bit-exact except on rows the oracle flags as near ties
(last kept and first dropped score within 1e-4 relative); those rows are
counted and their CSR lists are still checked for internal consistency.
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_csr_consistent, compare_masks, download_mask, to64

pytestmark = pytest.mark.gpu


def run_select(q, k, segs, block, budget, window=0):
    lay = hm.Layout(block, list(segs), window)
    bm = hm.select(q, k, lay, budget)
    torch.cuda.synchronize()
    return bm


def oracle_select(q, k, segs, block, budget, window=0):
    return oracle.select(to64(q), to64(k), block, list(segs), budget, window)


SMALL = [
    # (name, B, H, Hkv, N, D, block, dtype, segments, budget, window)
    ("ragged_d64", 2, 3, 3, 64 * 37, 64, 64, "bf16", (), 0.3, 0),
    ("layout_window_d128", 1, 2, 2, 512 + 64 * 100, 128, 64, "bf16",
     (("text", 100), ("padding", 412), ("image", 6400)), 0.25, 256),
    ("gqa_d64", 1, 4, 2, 64 * 50, 64, 64, "bf16", (), 0.4, 0),
    ("fp32_block32_d32", 2, 2, 2, 32 * 45, 32, 32, "fp32", (), 0.3, 0),
    ("bf16_block32_d128", 1, 2, 2, 32 * 70, 128, 32, "bf16", (("image", 32 * 60), ("audio", 320)), 0.2, 0),
    ("n_cand_600_e16", 1, 2, 2, 64 * 600, 64, 64, "bf16", (), 0.3, 0),
    ("n_cand_1100_e32", 1, 1, 1, 64 * 1100, 32, 64, "bf16", (), 0.1, 0),
    ("n_cand_2048_max", 1, 1, 1, 64 * 2048, 32, 64, "bf16", (), 0.05, 0),   # the largest candidate count
    ("split_candidates", 1, 2, 2, 64 * 40, 64, 64, "bf16",
     (("image", 64 * 10), ("text", 64 * 3), ("video", 64 * 20), ("padding", 64 * 2), ("image", 64 * 5)), 0.3, 200),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_select_small(cuda, case):
    name, B, H, Hkv, N, D, block, dtype, segs, budget, window = case
    q, k, _ = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, block=block, dtype=dtype, seed=7)
    bm = run_select(q.to(cuda), k.to(cuda), segs, block, budget, window)
    ref, tie = oracle_select(q, k, segs, block, budget, window)
    excluded = compare_masks(bm, ref, tie)
    # near ties grow with the candidate count; a bound keeps the check from
    # passing vacuously
    assert excluded <= max(2, ref.shape[0] * ref.shape[1] * ref.shape[2] // 10)
    assert bm.k == oracle.budget(int((oracle.classes(list(segs), N, block) == 0).sum()), budget)[0]


@pytest.mark.parametrize("name", ["tiny_fp32", "sdxl_bf16", "joint_text_image_bf16", "video_radial_bf16", "video_gqa_bf16"])
def test_select_workload(cuda, name):
    w = workloads.ALL[name]
    q, k, _ = workloads.make_qkv(w)
    bm = run_select(q.to(cuda), k.to(cuda), w.segments, w.block, w.budget, w.window_tokens)
    ref, tie = oracle_select(q, k, w.segments, w.block, w.budget, w.window_tokens)
    excluded = compare_masks(bm, ref, tie)
    rows = ref.shape[0] * ref.shape[1] * ref.shape[2]
    print(f"[select {name}] near-tie rows excluded: {excluded} of {rows}", flush=True)
    assert excluded <= rows // 50


@pytest.mark.parametrize("layer", [0, 21, 42, 63])
def test_select_head_masked_stack_layers(cuda, layer):
    w = workloads.STACK
    q, k, _ = workloads.make_qkv(w, layer)
    bm = run_select(q.to(cuda), k.to(cuda), w.segments, w.block, w.budget, w.window_tokens)
    ref, tie = oracle_select(q, k, w.segments, w.block, w.budget, w.window_tokens)
    compare_masks(bm, ref, tie)
    assert bm.k == 18


def test_select_full_budget_reports_dense(cuda):
    w = workloads.JOINT
    q, k, _ = workloads.small_case(B=1, H=2, N=w.N, D=64, seed=3)
    bm = run_select(q.to(cuda), k.to(cuda), w.segments, 64, 1.0)
    assert bm.is_dense and bm.k == 256
    ref, tie = oracle_select(q, k, w.segments, 64, 1.0)
    assert tie.sum() == 0
    m, c, i = download_mask(bm)
    assert np.array_equal(m, ref)
    assert_csr_consistent(m, c, i)


def test_select_scale_invariance_and_determinism(cuda):
    q, k, _ = workloads.small_case(B=2, H=2, N=64 * 64, D=128, seed=11, device=cuda)
    lay = hm.Layout(64, [])
    a = hm.select(q, k, lay, 0.3)
    b = hm.select(q * 2, k * 0.5, lay, 0.3)          # exact in bf16
    c = hm.select(q, k, lay, 0.3)
    torch.cuda.synchronize()
    assert torch.equal(a.mask, b.mask) and torch.equal(a.count, b.count)
    assert torch.equal(a.mask, c.mask) and torch.equal(a.count, c.count)
    for r in range(a.count.numel()):
        n = int(a.count.view(-1)[r])
        assert torch.equal(a.index.view(-1, 64)[r, :n], c.index.view(-1, 64)[r, :n])


def test_mask_density(cuda):
    w = workloads.SDXL
    q, k, _ = workloads.make_qkv(w)
    bm = run_select(q.to(cuda), k.to(cuda), w.segments, w.block, w.budget)
    assert abs(hm.mask_density(bm) - 19 / 64) < 1e-12


# ---- radial band ----------------------------------------------------------------

@pytest.mark.parametrize("segs,N,block,density,window", [
    ((), 64 * 40, 64, 0.3, 0),
    ((("text", 128), ("padding", 384), ("video", 64 * 200)), 512 + 64 * 200, 64, 0.3, 0),
    ((("image", 64 * 10), ("text", 64 * 3), ("video", 64 * 20), ("padding", 64 * 2), ("image", 64 * 5)),
     64 * 40, 64, 0.25, 300),
    ((), 32 * 9, 32, 0.5, 0),
    ((("text", 128), ("padding", 384), ("video", 64 * 200)), 512 + 64 * 200, 64, 1.0, 0),
    # candidates with a one-block gap: equal distances on both sides of the gap
    ((("image", 64 * 3), ("text", 64), ("image", 64 * 3)), 64 * 7, 64, 0.5, 0),
    ((("image", 32 * 7), ("audio", 32 * 2), ("video", 32 * 11), ("padding", 32), ("image", 32 * 9)),
     32 * 30, 32, 0.4, 0),
])
def test_radial_small(cuda, segs, N, block, density, window):
    lay = hm.Layout(block, list(segs), window)
    bm = hm.radial(lay, N, density, B=2, H=3, device=cuda)
    torch.cuda.synchronize()
    ref = oracle.radial(N, block, list(segs), density, window)
    m, c, i = download_mask(bm)
    for b in range(2):
        for h in range(3):
            assert np.array_equal(m[b, h], ref)
    assert_csr_consistent(m, c, i)


def test_radial_video_workload_matches_selector_density(cuda):
    w = workloads.VIDEO
    lay = hm.Layout(w.block, list(w.segments))
    rad = hm.radial(lay, w.N, w.budget, device=cuda)
    q, k, _ = workloads.make_qkv(w)
    sel = hm.select(q.to(cuda), k.to(cuda), lay, w.budget)
    torch.cuda.synchronize()
    ref = oracle.radial(w.N, w.block, list(w.segments), w.budget)
    m, c, i = download_mask(rad)
    assert np.array_equal(m[0, 0], ref)
    assert_csr_consistent(m, c, i)
    # same kept pairs per row as the selector: 155 per video row, 514 per live text row
    sc = sel.count.cpu().numpy()
    assert np.array_equal(np.broadcast_to(c, sc.shape), sc)
    assert set(np.unique(c).tolist()) == {0, 155, 514}


def boundary_case(n, D, k, seed, negative=False):
    """fp32 Q/K whose block-mean scores put every row's last-kept / first-dropped
    pair just outside the 1e-4 near-tie window (1.0001e-4 .. 1.2e-4 relative),
    at magnitudes just below and just above powers of two.

    Q block i = (1 + i // D) * e_(i % D) on every token; K block j = column
    v[:, j] on every token, so score(i, j) = (1 + i // D) * v[i % D, j]
    exactly.  Rows of one pattern d = i % D share v[d, :]; the D-periodic
    diagonal positions get the smallest values so removing the diagonal never
    moves the boundary.
    """
    rng = np.random.default_rng(seed)
    v = np.zeros((D, n))
    for d in range(D):
        diag_like = [j for j in range(n) if j % D == d]
        others = [j for j in range(n) if j % D != d]
        order = rng.permutation(others)
        x = float(2.0 ** rng.integers(-3, 4)) * (1 - 2.0 ** -12 if rng.random() < 0.5 else 1 + 2.0 ** -12)
        delta = rng.uniform(1.0001e-4, 1.2e-4)
        vals = np.empty(len(order))
        top = k - 1                                  # non-diagonal kept per row
        vals[top - 1] = x * (1 + delta)              # last kept
        vals[top] = x                                # first dropped
        for r in range(top - 2, -1, -1):
            vals[r] = vals[r + 1] * (1 + rng.uniform(2e-3, 1e-2))
        for r in range(top + 1, len(order)):
            vals[r] = vals[r - 1] * (1 - rng.uniform(2e-3, 1e-2))
        if negative:
            vals = -vals[::-1]
            vals_ordered = np.empty_like(vals)
            vals_ordered[:] = vals
            # negate and reverse keeps the boundary gap; ranks flip accordingly
        v[d, order] = np.float32(vals)
        v[d, diag_like] = np.float32(np.min(vals) - 1.0) if not negative else np.float32(np.min(vals) * 1.5)
    block = 64
    N = n * block
    q = np.zeros((1, 1, N, D), np.float32)
    kk = np.zeros((1, 1, N, D), np.float32)
    for i in range(n):
        q[0, 0, i * block:(i + 1) * block, i % D] = 1 + i // D
        kk[0, 0, i * block:(i + 1) * block, :] = v[:, i]
    return torch.from_numpy(q), torch.from_numpy(kk)


@pytest.mark.parametrize("n,D,negative", [(64, 64, False), (64, 64, True), (512, 128, False), (512, 128, True)])
def test_select_rank_resolution_outside_tie_window(cuda, n, D, negative):
    budget = 0.3
    k = oracle.budget(n, budget)[0]
    q, kk = boundary_case(n, D, k, seed=n + D + int(negative), negative=negative)
    bm = run_select(q.to(cuda), kk.to(cuda), (), 64, budget)
    ref, tie = oracle_select(q, kk, (), 64, budget)
    assert tie.sum() == 0, "the construction must keep every row outside the near-tie window"
    assert compare_masks(bm, ref, tie) == 0


def random_layout(rng, block):
    """A random ordered segment list (every kind, lengths not block-aligned)."""
    kinds = ["text", "conditioning", "audio", "other", "image", "video", "padding"]
    segs, total = [], 0
    for _ in range(int(rng.integers(2, 9))):
        kind = kinds[int(rng.integers(0, len(kinds)))]
        n = int(rng.integers(1, 12)) * block + (int(rng.integers(0, block)) if rng.random() < 0.4 else 0)
        segs.append((kind, n))
        total += n
    pad = (-total) % block
    if pad:
        segs.append(("padding", pad))
        total += pad
    return segs, total


@pytest.mark.parametrize("seed", range(6))
def test_select_random_layouts(cuda, seed):
    # random packed layouts (segments not block-aligned, every token kind),
    # budgets and windows: masks bit-exact outside near ties
    rng = np.random.default_rng(1000 + seed)
    block = 64 if seed % 3 else 32
    segs, N = random_layout(rng, block)
    D = [32, 64, 128][seed % 3]
    budget = float(rng.choice([0.1, 0.25, 0.3, 0.5, 0.9]))
    window = int(rng.choice([0, 0, 64, 200, 512]))
    q, k, _ = workloads.small_case(B=1, H=2, N=N, D=D, block=block, dtype="bf16", seed=2000 + seed)
    bm = run_select(q.to(cuda), k.to(cuda), segs, block, budget, window)
    ref, tie = oracle_select(q, k, segs, block, budget, window)
    compare_masks(bm, ref, tie)


def test_select_and_forward_long_sequence(cuda):
    # 131072 tokens (2048 key blocks) on one head: the largest candidate count
    # through select and forward, forward checked on sampled rows
    from parity import upload_mask, assert_close
    N, D = 64 * 2048, 128
    q, k, v = workloads.small_case(B=1, H=1, N=N, D=D, seed=2100)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    bm = run_select(qd, kd, (), 64, 0.02)
    ref, tie = oracle_select(q, k, (), 64, 0.02)
    compare_masks(bm, ref, tie)
    out = hm.forward(qd, kd, vd, upload_mask(ref, cuda))
    torch.cuda.synchronize()
    rows = np.stack([np.zeros(48, int), np.zeros(48, int), np.random.default_rng(2101).integers(0, N, 48)], 1)
    refo = oracle.attention(to64(q), to64(k), to64(v), 64, ref, rows=rows)
    got = out.cpu()[rows[:, 0], rows[:, 1], rows[:, 2]].double().numpy()
    assert_close(got, refo, "bf16", "long sequence")


@pytest.mark.parametrize("D,nb,seed", [(32, 64, 60), (64, 64, 61), (128, 64, 62), (64, 256, 63), (128, 256, 64)])
def test_select_zero_mean_half_budget(cuda, D, nb, seed):
    """Zero-mean i.i.d. Q and K at a 50 % budget: every row's boundary sits at
    the median score, near zero, where an error proportional to the summed
    term magnitudes is largest against the score itself.  Many heads, masks
    bit-exact outside near-tie rows; the fused call too where it applies."""
    B, H = 1, 48 if nb == 64 else 12
    q, k, v = workloads.small_case(B=B, H=H, N=64 * nb, D=D, seed=seed)
    ref, tie = oracle_select(q, k, (), 64, 0.5)
    bm = run_select(q.to(cuda), k.to(cuda), (), 64, 0.5)
    compare_masks(bm, ref, tie)
    if D == 64 and nb <= 64:
        _out, bmf = hm.select_forward(q.to(cuda), k.to(cuda), v.to(cuda), hm.Layout(64, []), 0.5)
        torch.cuda.synchronize()
        compare_masks(bmf, ref, tie)


def cancellation_case(D, nb, H, seed):
    """bf16 Q/K whose block scores are exact small values reached through
    large cancelling terms.  Every query token is all ones; every token of
    key block j of head h is R_h + s_j.  R_h pairs +x with -x over randomly
    placed dimensions (so it sums to exactly 0): half the pairs big
    (2^18 .. 2^20), half fine-grained (1 + m 2^-7).  s_j writes j in two
    other dimensions as j // 64 and (j % 64) 2^-6, so block-mean scores
    are j / 64 exactly: distinct, 2^-6 apart, far outside the 1e-4 near-tie
    window.  A float32 sum of the pooled terms adds the fine values to
    partial sums near 2^20, whose spacing (2^-3 and up) is coarser than the
    gap between two candidates' scores."""
    rng = np.random.default_rng(seed)
    N = 64 * nb
    q = torch.ones((1, H, N, D), dtype=torch.bfloat16)
    kk = np.zeros((1, H, N, D), np.float32)
    for h in range(H):
        r = np.zeros(D, np.float64)
        perm = rng.permutation(D)          # random places for the pairs and the two signal dimensions
        sig_a, sig_b, pos = perm[0], perm[1], perm[2:]
        pairs = (D - 2) // 2
        for p in range(pairs):
            if p % 2 == 0:
                x = 2.0 ** rng.integers(18, 21) * (1 + rng.integers(0, 128) / 128.0)
            else:
                x = 1 + rng.integers(1, 128) / 128.0
            x *= 1 if rng.random() < 0.5 else -1
            r[pos[2 * p]] = x
            r[pos[2 * p + 1]] = -x
        for j in range(nb):
            row = r.copy()
            row[sig_a] = j // 64
            row[sig_b] = (j % 64) * 2.0 ** -6
            kk[0, h, j * 64:(j + 1) * 64, :] = row
    k = torch.from_numpy(kk).to(torch.bfloat16)
    assert torch.equal(k.float(), torch.from_numpy(kk)), "construction must be bf16-exact"
    return q, k


@pytest.mark.parametrize("D,nb", [(64, 64), (128, 64), (128, 512)])
def test_select_cancelling_scores(cuda, D, nb):
    """Scores reached through large cancelling terms (see cancellation_case):
    the ranking must follow the exact scores, so masks are bit-exact on every
    row (none is a near tie), for the selector and the fused call."""
    H = 8
    q, k = cancellation_case(D, nb, H, seed=70 + D + nb)
    budget = 0.5
    ref, tie = oracle_select(q, k, (), 64, budget)
    assert tie.sum() == 0
    bm = run_select(q.to(cuda), k.to(cuda), (), 64, budget)
    assert compare_masks(bm, ref, tie) == 0
    if D == 64 and nb <= 64:
        v = torch.zeros_like(q)
        _out, bmf = hm.select_forward(q.to(cuda), k.to(cuda), v.to(cuda), hm.Layout(64, []), budget)
        torch.cuda.synchronize()
        assert compare_masks(bmf, ref, tie) == 0


@pytest.mark.parametrize("D,nb,kind", [(64, 64, "zero_keys"), (128, 64, "equal_blocks"), (64, 256, "zero_keys"),
                                       (128, 512, "equal_blocks")])
def test_select_exact_ties_go_to_the_lower_block(cuda, D, nb, kind):
    """Every non-diagonal score of a row exactly equal (all keys zero, or
    every key block the same): the pages' rule sends ties to the lower block
    index, so the kept set is the diagonal plus the lowest k - 1 other
    candidates.  The oracle flags such rows as near ties, but both sides
    break exact ties the same way, so here every row is compared."""
    B, H = 1, 4
    q, k, _ = workloads.small_case(B=B, H=H, N=64 * nb, D=D, seed=80 + nb)
    if kind == "zero_keys":
        k = torch.zeros_like(k)
    else:
        k = k[:, :, :64].repeat(1, 1, nb, 1).contiguous()
    budget = 0.3
    ref, tie = oracle_select(q, k, (), 64, budget)
    assert tie.all()
    bm = run_select(q.to(cuda), k.to(cuda), (), 64, budget)
    got = download_mask(bm)[0]
    assert np.array_equal(got, ref)
    kk = oracle.budget(nb, budget)[0]
    for i in (0, nb // 2, nb - 1):
        expect = sorted({i} | set([j for j in range(nb) if j != i][:kk - 1]))
        assert np.nonzero(ref[0, 0, i])[0].tolist() == expect
    if D == 64 and nb <= 64:
        _out, bmf = hm.select_forward(q.to(cuda), k.to(cuda), torch.zeros_like(k).to(cuda), hm.Layout(64, []),
                                      budget)
        torch.cuda.synchronize()
        assert np.array_equal(download_mask(bmf)[0], ref)


@pytest.mark.parametrize("D,nb,budget", [(64, 256, 0.05), (128, 256, 0.3), (64, 512, 0.7), (128, 512, 0.3),
                                         (32, 512, 0.5)])
def test_select_scores_over_many_binades(cuda, D, nb, budget):
    """Key blocks scaled by 2^e (e from -12 to 12) with random signs, a few of
    them exact copies of another: each row's scores spread over many binades
    of both signs with exact ties among them, so the rank's ordering of float
    keys is exercised far from one scale.  Masks bit-exact outside the
    oracle's near-tie rows (selector paragraph: ranking by score, ties to the
    lower block)."""
    B, H = 1, 6
    q, k, _ = workloads.small_case(B=B, H=H, N=64 * nb, D=D, seed=90 + nb + D)
    rng = np.random.default_rng(91 + nb + D)
    scale = np.ldexp(1.0, rng.integers(-12, 13, size=(H, nb))) * rng.choice([-1.0, 1.0], size=(H, nb))
    kb = k.float().view(B, H, nb, 64, D) * torch.from_numpy(scale).float()[None, :, :, None, None]
    for dst, src in ((7, 3), (nb // 2, 3), (nb - 1, nb // 3)):
        kb[:, :, dst] = kb[:, :, src]
    k = kb.reshape(B, H, 64 * nb, D).to(k.dtype).contiguous()
    ref, tie = oracle_select(q, k, (), 64, budget)
    bm = run_select(q.to(cuda), k.to(cuda), (), 64, budget)
    compare_masks(bm, ref, tie)


HEADS_CASES = [
    # (name, B, H, Hkv, nb, D, dtype, block, segments, budget, window, head mask)
    ("sdxl_like", 2, 8, 8, 64, 64, "bf16", 64, (), 0.3, 0, (1, 0, 1, 1, 0, 0, 1, 0)),
    ("gqa_group_off", 1, 8, 2, 40, 128, "bf16", 64, (), 0.3, 0, (0, 0, 0, 0, 1, 0, 1, 1)),
    ("layout_window", 1, 4, 4, 50, 128, "bf16", 64,
     (("conditioning", 64), ("image", 64 * 45), ("padding", 64 * 4)), 0.3, 512, (0, 1, 1, 0)),
    ("dense_budget", 1, 4, 2, 20, 64, "bf16", 64, (("text", 100), ("image", 64 * 20 - 100)), 1.0, 0, (1, 0, 0, 1)),
    ("all_masked", 1, 3, 3, 16, 32, "fp32", 32, (), 0.4, 0, (0, 0, 0)),
    ("none_masked", 1, 3, 1, 16, 64, "bf16", 64, (), 0.4, 0, (1, 1, 1)),
    ("radix_rows", 1, 4, 4, 300, 64, "bf16", 64, (), 0.3, 0, (1, 0, 0, 1)),
    ("radix_512", 1, 2, 1, 512, 128, "bf16", 64, (), 0.3, 0, (0, 1)),
]


@pytest.mark.parametrize("case", HEADS_CASES, ids=[c[0] for c in HEADS_CASES])
def test_select_heads(cuda, case):
    """bsattn_select_heads: the rows of active heads are bit-identical to
    bsattn_select's (and so to the oracle outside near ties), every row of a
    masked head is empty, and attention under the same head mask gives the
    same output as after bsattn_select (haagenti_sparse crate docs: masked
    heads are skipped; SD.Next selector paragraph)."""
    name, B, H, Hkv, nb, D, dtype, block, segs, budget, window, hmask_t = case
    N = nb * block
    q, k, v = workloads.small_case(B=B, H=H, Hkv=Hkv, N=N, D=D, block=block, dtype=dtype, seed=120 + nb)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    hmask = np.array(hmask_t, np.uint8)
    hmd = torch.from_numpy(hmask).to(cuda)
    lay = hm.Layout(block, list(segs), window)
    full = hm.select(qd, kd, lay, budget)
    part = hm.select_heads(qd, kd, lay, budget, hmd)
    torch.cuda.synchronize()
    assert part.k == full.k and part.is_dense == full.is_dense
    mf, cf, idf = download_mask(full)
    mp, cp, idp = download_mask(part)
    on = hmask != 0
    assert np.array_equal(mp[:, on], mf[:, on])
    assert np.array_equal(cp[:, on], cf[:, on])
    for b in range(B):
        for h in np.nonzero(on)[0]:
            for i in range(nb):
                assert np.array_equal(idp[b, h, i, :cp[b, h, i]], idf[b, h, i, :cf[b, h, i]])
    assert not mp[:, ~on].any() and not cp[:, ~on].any()
    # against the oracle: masked heads' rows empty, the rest as selected
    ref, tie = oracle_select(q, k, segs, block, budget, window)
    ref = ref.copy()
    ref[:, ~on] = 0
    tie = tie.copy()
    tie[:, ~on] = 0
    compare_masks(part, ref, tie)
    # the forward under the same head mask does not see the difference
    o_full = hm.forward(qd, kd, vd, full, hmd)
    o_part = hm.forward(qd, kd, vd, part, hmd)
    torch.cuda.synchronize()
    assert torch.equal(o_full, o_part)
    # no head mask: exactly bsattn_select
    again = hm.select_heads(qd, kd, lay, budget, None)
    torch.cuda.synchronize()
    ma, ca, _ = download_mask(again)
    assert np.array_equal(ma, mf) and np.array_equal(ca, cf)
