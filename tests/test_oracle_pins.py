"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to the pages, to mathematics (closed forms,
brute force on tiny inputs, invariances) or to an independent library routine
(torch's float64 scaled_dot_product_attention, the reference the SD.Next
flex-consumer paragraph names for its tile-equivalence test).
"""
import itertools
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = line.split()
                vals[key] = float(val) if "." in val else int(val)
    return vals


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def sdpa64(q, k, v, scale=None):
    return F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                          torch.from_numpy(v), scale=scale).numpy()


@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2), (3, 1)])
def test_full_density_equals_sdpa(H, Hkv):
    B, N, D, block = 2, 96, 16, 32
    q, k, v = rnd((B, H, N, D), 1), rnd((B, Hkv, N, D), 2), rnd((B, Hkv, N, D), 3)
    nb = N // block
    out = oracle.attention(q, k, v, block, np.ones((nb, nb), np.uint8))
    rep = H // Hkv
    ref = sdpa64(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1))
    assert np.abs(out - ref).max() <= 1e-12


def test_explicit_scale_equals_sdpa_scale():
    q, k, v = rnd((1, 2, 64, 8), 4), rnd((1, 2, 64, 8), 5), rnd((1, 2, 64, 8), 6)
    out = oracle.attention(q, k, v, 32, np.ones((2, 2), np.uint8), scale=0.37)
    assert np.abs(out - sdpa64(q, k, v, scale=0.37)).max() <= 1e-12


def test_softmax_rows_sum_to_one():
    # with V = 1 every output element of a row is the sum of that row's
    # attention weights; empty rows give 0
    B, H, N, D, block = 1, 3, 128, 8, 32
    nb = N // block
    q, k = rnd((B, H, N, D), 7) * 3, rnd((B, H, N, D), 8) * 3
    v = np.ones((B, H, N, D))
    rng = np.random.default_rng(9)
    mask = (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)
    mask[0, 0, 1, :] = 0                        # one empty row
    out = oracle.attention(q, k, v, block, mask)
    rows_nonempty = mask.any(-1)                # [B,H,nb]
    for h in range(H):
        for i in range(nb):
            blk = out[0, h, i * block:(i + 1) * block]
            if rows_nonempty[0, h, i]:
                assert np.abs(blk - 1.0).max() <= 1e-12
            else:
                assert np.all(blk == 0.0)


def test_masked_heads_are_exactly_zero():
    q, k, v = rnd((2, 2, 64, 8), 10), rnd((2, 2, 64, 8), 11), rnd((2, 2, 64, 8), 12)
    out = oracle.attention(q, k, v, 32, np.ones((2, 2), np.uint8), head_mask=np.array([1, 0], np.uint8))
    assert np.all(out[:, 1] == 0.0)
    assert np.abs(out[:, 0] - sdpa64(q, k, v)[:, 0]).max() <= 1e-12


def gather_sdpa(q, k, v, block, mask2d):
    """Per query block: sdpa over only the kept key tiles (no -inf anywhere)."""
    B, H, N, D = q.shape
    nb = N // block
    out = np.zeros_like(q)
    for i in range(nb):
        cols = np.nonzero(mask2d[i])[0]
        if cols.size == 0:
            continue
        idx = np.concatenate([np.arange(j * block, (j + 1) * block) for j in cols])
        out[:, :, i * block:(i + 1) * block] = sdpa64(
            np.ascontiguousarray(q[:, :, i * block:(i + 1) * block]),
            np.ascontiguousarray(k[:, :, idx]), np.ascontiguousarray(v[:, :, idx]))
    return out


@pytest.mark.parametrize("nb", [2, 3])
def test_every_block_mask_matches_gathered_sdpa(nb):
    # brute force over all 2^(nb*nb) block masks: tile equivalence against
    # sdpa fed the same tiles
    block, D = 4, 8
    N = nb * block
    q, k, v = rnd((1, 2, N, D), 13), rnd((1, 2, N, D), 14), rnd((1, 2, N, D), 15)
    worst = 0.0
    for bits in range(1 << (nb * nb)):
        m = np.array([(bits >> s) & 1 for s in range(nb * nb)], np.uint8).reshape(nb, nb)
        got = oracle.attention(q, k, v, block, m)
        ref = gather_sdpa(q, k, v, block, m)
        worst = max(worst, float(np.abs(got - ref).max()))
    assert worst <= 1e-12


# ---- per-token key mask composed with the block mask (SD.Next sparse-stage
# paragraph: a masked_block backend takes the token mask and block mask together)

def test_key_mask_equals_sdpa_boolean_mask():
    B, H, N, D, block = 2, 3, 96, 8, 32
    q, k, v = rnd((B, H, N, D), 40), rnd((B, H, N, D), 41), rnd((B, H, N, D), 42)
    km = (np.random.default_rng(43).random((B, N)) < 0.7).astype(np.uint8)
    km[:, 0] = 1
    out = oracle.attention(q, k, v, block, np.ones((3, 3), np.uint8), key_mask=km)
    am = torch.from_numpy(km.astype(bool))[:, None, None, :]
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=am).numpy()
    assert np.abs(out - ref).max() <= 1e-12


def test_key_mask_and_block_mask_compose_as_gathered_sdpa():
    # each query block attends to the keys that are both in a kept block and
    # unmasked: gather exactly those and run sdpa on them
    B, H, N, D, block = 2, 2, 64, 8, 16
    nb = N // block
    q, k, v = rnd((B, H, N, D), 44), rnd((B, H, N, D), 45), rnd((B, H, N, D), 46)
    rng = np.random.default_rng(47)
    bm = (rng.random((nb, nb)) < 0.6).astype(np.uint8)
    np.fill_diagonal(bm, 1)
    km = (rng.random((B, N)) < 0.75).astype(np.uint8)
    km[:, ::block] = 1                      # every block keeps a live key
    out = oracle.attention(q, k, v, block, bm, key_mask=km)
    for b in range(B):
        for i in range(nb):
            keys = [j for j in range(N) if bm[i, j // block] and km[b, j]]
            ref = sdpa64(np.ascontiguousarray(q[b:b + 1, :, i * block:(i + 1) * block]),
                         np.ascontiguousarray(k[b:b + 1][:, :, keys]), np.ascontiguousarray(v[b:b + 1][:, :, keys]))
            assert np.abs(out[b:b + 1, :, i * block:(i + 1) * block] - ref).max() <= 1e-12


def test_masked_keys_never_reach_the_output():
    B, H, N, D, block = 1, 2, 64, 8, 32
    q, k, v = rnd((B, H, N, D), 48), rnd((B, H, N, D), 49), rnd((B, H, N, D), 50)
    km = np.ones((B, N), np.uint8)
    km[0, 5:40] = 0
    a = oracle.attention(q, k, v, block, np.ones((2, 2), np.uint8), key_mask=km)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 5:40] = 1e3 * rnd((B, H, 35, D), 51)
    v2[:, :, 5:40] = -7.0
    b2 = oracle.attention(q, k2, v2, block, np.ones((2, 2), np.uint8), key_mask=km)
    assert np.array_equal(a, b2)


def test_key_mask_of_whole_block_equals_block_mask_column():
    B, H, N, D, block = 1, 2, 96, 8, 32
    q, k, v = rnd((B, H, N, D), 52), rnd((B, H, N, D), 53), rnd((B, H, N, D), 54)
    km = np.ones((B, N), np.uint8)
    km[:, 32:64] = 0
    bm = np.ones((3, 3), np.uint8)
    bm[:, 1] = 0
    a = oracle.attention(q, k, v, block, np.ones((3, 3), np.uint8), key_mask=km)
    b = oracle.attention(q, k, v, block, bm)
    assert np.array_equal(a, b)


def test_rows_whose_kept_keys_are_all_masked_are_zero():
    B, H, N, D, block = 1, 1, 64, 8, 32
    q, k, v = rnd((B, H, N, D), 55), rnd((B, H, N, D), 56), rnd((B, H, N, D), 57)
    bm = np.array([[1, 0], [1, 1]], np.uint8)
    km = np.ones((B, N), np.uint8)
    km[:, :32] = 0                          # query block 0 keeps only block 0: all masked
    out = oracle.attention(q, k, v, block, bm, key_mask=km)
    assert np.all(out[:, :, :32] == 0.0)
    assert np.abs(out[:, :, 32:]).max() > 0


def test_sampled_rows_match_full_rows():
    q, k, v = rnd((2, 3, 96, 8), 16), rnd((2, 3, 96, 8), 17), rnd((2, 3, 96, 8), 18)
    rng = np.random.default_rng(19)
    mask = (rng.random((2, 3, 3, 3)) < 0.6).astype(np.uint8)
    full = oracle.attention(q, k, v, 32, mask)
    rows = np.array([[1, 2, 95], [0, 0, 0], [1, 1, 40], [0, 2, 63]])
    part = oracle.attention(q, k, v, 32, mask, rows=rows)
    for r, (b, h, t) in enumerate(rows):
        assert np.array_equal(part[r], full[b, h, t])


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def constructed_qk(M, block, noise_seed=0):
    """Q/K whose block means give scores exactly M[i, j] = <Qmean_i, Kmean_j>.

    Block i of Q is the unit vector e_i plus zero-mean integer noise; block j
    of K is column j of M plus zero-mean noise.  D = number of blocks.
    """
    nb = M.shape[0]
    D = nb
    rng = np.random.default_rng(noise_seed)
    q = np.zeros((1, 1, nb * block, D))
    k = np.zeros((1, 1, nb * block, D))
    for i in range(nb):
        for t in range(0, block, 2):
            z = rng.integers(-3, 4, size=D).astype(float)
            q[0, 0, i * block + t] = np.eye(D)[i] + z
            q[0, 0, i * block + t + 1] = np.eye(D)[i] - z
            z2 = rng.integers(-3, 4, size=D).astype(float)
            k[0, 0, i * block + t] = M[:, i] + z2
            k[0, 0, i * block + t + 1] = M[:, i] - z2
    return q, k


def brute_force_select_row(scores_row, i, cands, kk):
    """Max-sum k-subset of the candidates containing i; ties to the
    lexicographically smallest sorted index tuple."""
    others = [j for j in cands if j != i]
    best, best_set = None, None
    for comb in itertools.combinations(others, kk - 1):
        s = sum(scores_row[j] for j in comb)
        key = (-s, tuple(sorted(comb + (i,))))
        if best is None or key < best:
            best, best_set = key, set(comb) | {i}
    return best_set


@pytest.mark.parametrize("seed", range(4))
def test_selection_equals_brute_force_subsets(seed):
    nb, block = 6, 4
    rng = np.random.default_rng(100 + seed)
    M = rng.integers(-3, 4, size=(nb, nb)).astype(float)     # many exact ties, not symmetric
    q, k = constructed_qk(M, block, seed)
    for b in [0.2, 0.34, 0.5, 0.67, 0.84]:
        kk, dense = oracle.budget(nb, b)
        mask, _ = oracle.select(q, k, block, [], b)
        for i in range(nb):
            expect = brute_force_select_row(M[i], i, list(range(nb)), kk)
            got = set(np.nonzero(mask[0, 0, i])[0].tolist())
            assert got == expect, (b, i, M[i])


def test_scores_are_query_rows_against_key_columns():
    # a non-symmetric score matrix: row i must rank M[i, :], not M[:, i]
    M = np.array([[0, 5, 1, 2], [9, 0, 3, 1], [1, 8, 0, 7], [6, 2, 4, 0]], float)
    q, k = constructed_qk(M, 2)
    mask, _ = oracle.select(q, k, 2, [], 0.5)     # k = 2: diagonal + best other
    got = [set(np.nonzero(mask[0, 0, i])[0]) for i in range(4)]
    assert got == [{0, 1}, {0, 1}, {1, 2}, {0, 3}]


def test_near_tie_worked_example():
    # row 1 with other scores j0: 0.5, j2: 0.9, j3: 0.5
    M = np.zeros((4, 4))
    M[1] = [0.5, 0.0, 0.9, 0.5]
    M[0] = [0, 3, 2, 1]
    M[2] = [3, 2, 0, 1]
    M[3] = [3, 2, 1, 0]
    q, k = constructed_qk(M, 2)
    mask2, tie2 = oracle.select(q, k, 2, [], 0.5)    # k = 2
    assert set(np.nonzero(mask2[0, 0, 1])[0]) == {1, 2} and tie2[0, 0, 1] == 0
    mask3, tie3 = oracle.select(q, k, 2, [], 0.75)   # k = 3: tie between j0 and j3
    assert set(np.nonzero(mask3[0, 0, 1])[0]) == {0, 1, 2} and tie3[0, 0, 1] == 1


def test_selection_scale_and_permutation_invariance():
    rng = np.random.default_rng(20)
    q, k = rng.standard_normal((2, 3, 512, 16)), rng.standard_normal((2, 3, 512, 16))
    base, tie = oracle.select(q, k, 32, [], 0.3)
    assert np.array_equal(oracle.select(q * 4.0, k * 0.25, 32, [], 0.3)[0], base)
    perm = np.concatenate([rng.permutation(32) + 32 * i for i in range(16)])
    assert np.array_equal(oracle.select(q[:, :, perm], k[:, :, perm], 32, [], 0.3)[0], base)


def test_gqa_scoring_equals_key_expansion():
    rng = np.random.default_rng(21)
    q, k = rng.standard_normal((1, 4, 256, 16)), rng.standard_normal((1, 2, 256, 16))
    a, _ = oracle.select(q, k, 32, [], 0.5)
    b, _ = oracle.select(q, np.repeat(k, 2, axis=1), 32, [], 0.5)
    assert np.array_equal(a, b)


def test_diagonal_kept_and_rows_hold_exactly_k():
    rng = np.random.default_rng(22)
    q, k = rng.standard_normal((1, 2, 640, 16)), rng.standard_normal((1, 2, 640, 16))
    for b in [0.05, 0.3, 0.7]:
        kk, _ = oracle.budget(10, b)
        mask, _ = oracle.select(q, k, 64, [], b)
        assert np.all(mask[0, :, np.arange(10), np.arange(10)] == 1)
        assert np.all(mask.sum(-1) == kk)


def test_budget_fraction_of_candidates_keeps_that_many():
    """The budget is a fraction of the sparsifiable candidates (SD.Next
    selector paragraph), so the fraction k/n of n candidates keeps exactly
    k: for every 1 <= k <= n <= 512 with budget the double nearest k/n, and
    for two-decimal budgets d/100 whenever d n / 100 is whole (0.29 of 100
    candidates is 29, although 0.29 * 100 = 28.999999999999996 in doubles).
    A budget a hair below k/n keeps k - 1: the budget is never exceeded."""
    for n in range(1, 513):
        for k in range(1, n + 1):
            assert oracle.budget(n, k / n)[0] == k, (k, n)
            if k > 1:
                assert oracle.budget(n, (k - 1e-6) / n)[0] == k - 1, (k, n)
    for d in range(1, 100):
        for n in range(1, 2049):
            if d * n % 100 == 0:
                assert oracle.budget(n, d / 100)[0] == d * n // 100, (d, n)


def test_full_budget_reports_dense_layout_only_mask():
    rng = np.random.default_rng(23)
    segs = [("text", 64), ("padding", 64), ("image", 512)]
    q, k = rng.standard_normal((1, 1, 640, 8)), rng.standard_normal((1, 1, 640, 8))
    kk, dense = oracle.budget(8, 1.0)
    assert dense and kk == 8
    mask, _ = oracle.select(q, k, 64, segs, 1.0)
    cls = oracle.classes(segs, 640, 64)
    live = cls != oracle.DROPPED
    expect = np.outer(live, live).astype(np.uint8)
    assert np.array_equal(mask[0, 0], expect)


def test_window_matches_token_pair_brute_force():
    rng = np.random.default_rng(24)
    block, nb = 8, 10
    q, k = rng.standard_normal((1, 1, nb * block, 4)), rng.standard_normal((1, 1, nb * block, 4))
    for W in [1, 2, 15, 16, 17, 18, 40, 64]:
        mask, _ = oracle.select(q, k, block, [], 0.1, window_tokens=W)   # k = 1
        for i in range(nb):
            for j in range(nb):
                near = any(2 * abs(t - s) <= W for t in range(i * block, (i + 1) * block)
                           for s in range(j * block, (j + 1) * block))
                assert mask[0, 0, i, j] == (1 if (near or i == j) else 0), (W, i, j)


# --------------------------------------------------------------------------
# layout
# --------------------------------------------------------------------------

def test_joint_layout_reproduces_printed_264_and_6():
    g = read_golden("joint_2048_layout.txt")
    block = g["block_tokens"]
    segs = [("text", 128), ("padding", g["text_padded_tokens"] - 128), ("image", 128 * 128)]
    N = sum(n for _, n in segs)
    cls = oracle.classes(segs, N, block)
    assert cls.size == g["key_blocks_per_row"]
    rng = np.random.default_rng(25)
    q, k = rng.standard_normal((1, 1, N, 4)), rng.standard_normal((1, 1, N, 4))
    mask, _ = oracle.select(q, k, block, segs, 0.3)
    # same sequence with the padding taken for text, as before the live runs
    # were published: those blocks were pinned
    segs_before = [("text", g["text_padded_tokens"]), ("image", 128 * 128)]
    before, _ = oracle.select(q, k, block, segs_before, 0.3)
    for i in np.nonzero(cls != oracle.DROPPED)[0]:
        moved = (before[0, 0, i] == 1) & (mask[0, 0, i] == 0) & (cls == oracle.DROPPED)
        assert moved.sum() == g["dropped_blocks_per_row"]
        assert np.all(mask[0, 0, i, cls == oracle.DROPPED] == 0)
    assert np.all(mask[0, 0, cls == oracle.DROPPED] == 0)


def test_layout_classes_straddling_and_kinds():
    # block 4: tokens text [0,2) image [2,10) padding [10,14) image [14,20)
    # audio [20,24) video [24,28).  Block 0 straddles text/image and pins,
    # block 2 straddles image/padding and pins, block 3 straddles
    # padding/image and pins (padding inside a pinned tile does not drop it),
    # audio pins, whole image/video blocks are sparsifiable.
    segs = [("text", 2), ("image", 8), ("padding", 4), ("image", 6), ("audio", 4), ("video", 4)]
    cls = oracle.classes(segs, 28, 4)
    assert cls.tolist() == [1, 0, 1, 1, 0, 1, 0]
    assert oracle.classes([], 28, 4).tolist() == [0] * 7
    assert oracle.classes([("padding", 8), ("conditioning", 4), ("other", 4)], 16, 4).tolist() == [2, 2, 1, 1]
    assert oracle.classes([("image", 4), ("video", 4)], 8, 8).tolist() == [1]   # two segments: pins


def test_pinned_rows_and_columns_are_dense():
    rng = np.random.default_rng(26)
    segs = [("text", 128), ("padding", 128), ("image", 1024)]
    N, block = 1280, 64
    q, k = rng.standard_normal((1, 2, N, 8)), rng.standard_normal((1, 2, N, 8))
    mask, _ = oracle.select(q, k, block, segs, 0.2)
    cls = oracle.classes(segs, N, block)
    pinned, dropped = cls == oracle.PINNED, cls == oracle.DROPPED
    live = ~dropped
    for h in range(2):
        assert np.all(mask[0, h][np.ix_(pinned, live)] == 1)
        assert np.all(mask[0, h][np.ix_(live, pinned)] == 1)
        assert np.all(mask[0, h][dropped] == 0) and np.all(mask[0, h][:, dropped] == 0)


# --------------------------------------------------------------------------
# radial band
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 5, 8, 13])
def test_radial_closed_form_on_contiguous_candidates(n):
    for dens in [0.1, 0.25, 0.5, 0.77, 1.0]:
        kk, _ = oracle.budget(n, dens)
        m = oracle.radial(n * 16, 16, [], dens)
        for i in range(n):
            lo = min(max(i - kk // 2, 0), n - kk)
            expect = np.zeros(n, np.uint8)
            expect[lo:lo + kk] = 1
            assert np.array_equal(m[i], expect), (n, dens, i)


def test_radial_worked_examples():
    m = oracle.radial(8 * 64, 64, [], 0.5)
    assert np.nonzero(m[0])[0].tolist() == [0, 1, 2, 3]
    assert np.nonzero(m[5])[0].tolist() == [3, 4, 5, 6]
    assert np.nonzero(m[7])[0].tolist() == [4, 5, 6, 7]


def test_radial_honours_pins_and_matches_selector_count():
    segs = [("text", 128), ("padding", 384), ("video", 64 * 40)]
    N = 512 + 64 * 40
    m = oracle.radial(N, 64, segs, 0.3)
    cls = oracle.classes(segs, N, 64)
    live = cls != oracle.DROPPED
    assert np.all(m[np.ix_(live, cls == oracle.PINNED)] == 1)      # text columns in every live row
    rng = np.random.default_rng(27)
    q, k = rng.standard_normal((1, 1, N, 8)), rng.standard_normal((1, 1, N, 8))
    sel, _ = oracle.select(q, k, 64, segs, 0.3)
    assert np.array_equal(m.sum(-1), sel[0, 0].sum(-1))


def test_radial_non_contiguous_candidates_rank_definition():
    # candidates split by a pinned block: nearest by (|i-j|, j) across the gap
    segs = [("image", 64 * 3), ("text", 64), ("image", 64 * 4)]
    m = oracle.radial(64 * 8, 64, segs, 0.5)   # 7 candidates -> k = 3
    cands = [0, 1, 2, 4, 5, 6, 7]
    for i in cands:
        order = sorted(cands, key=lambda j: (abs(i - j), j))[:3]
        got = [j for j in np.nonzero(m[i])[0] if j in cands]
        assert sorted(got) == sorted(order)


# --------------------------------------------------------------------------
# head mask
# --------------------------------------------------------------------------

def test_head_mask_constants_from_the_crate():
    g = read_golden("haagenti_constants.txt")
    assert g["HEADS"] * g["LAYERS"] == g["HEAD_COMPUTATIONS"]
    imp = np.random.default_rng(28).random(g["HEADS"])
    m = oracle.head_mask(imp, g["DEFAULT_SPARSITY"], g["MIN_ACTIVE_HEADS"])
    assert m.sum() == 16
    assert oracle.head_mask(imp[:2], g["DEFAULT_SPARSITY"], g["MIN_ACTIVE_HEADS"]).sum() == 2
    assert oracle.head_mask(imp[:5], g["DEFAULT_SPARSITY"], g["MIN_ACTIVE_HEADS"]).sum() == 4
    assert oracle.head_mask(imp[:7], g["DEFAULT_SPARSITY"], g["MIN_ACTIVE_HEADS"]).sum() == 4
    assert oracle.head_mask(imp[:10], g["DEFAULT_SPARSITY"], g["MIN_ACTIVE_HEADS"]).sum() == 5


@pytest.mark.parametrize("H", [1, 3, 6, 8])
def test_head_mask_brute_force(H):
    rng = np.random.default_rng(29 + H)
    for trial in range(20):
        imp = rng.integers(0, 3, size=H).astype(float)   # ties
        for sp, mn in [(0.5, 4), (0.25, 1), (0.75, 2), (0.0, 0)]:
            n_act = min(H, max(mn, H - int(np.floor(sp * H))))
            best = None
            for comb in itertools.combinations(range(H), n_act):
                key = (-sum(imp[list(comb)]), comb)
                if best is None or key < best:
                    best = key
            expect = np.zeros(H, np.uint8)
            expect[list(best[1])] = 1
            assert np.array_equal(oracle.head_mask(imp, sp, mn), expect)


# --------------------------------------------------------------------------
# end-to-end properties named by the pages
# --------------------------------------------------------------------------

def test_selection_changes_the_output():
    # a selection that stopped changing the output would pass silently
    rng = np.random.default_rng(30)
    q, k, v = (rng.standard_normal((1, 2, 512, 16)) for _ in range(3))
    mask, _ = oracle.select(q, k, 64, [], 0.3)
    sparse = oracle.attention(q, k, v, 64, mask)
    dense = oracle.attention(q, k, v, 64, np.ones((8, 8), np.uint8))
    assert np.abs(sparse - dense).max() > 10 * 2e-2


def test_padding_contents_do_not_reach_live_rows():
    rng = np.random.default_rng(31)
    segs = [("text", 64), ("padding", 64), ("image", 512)]
    q, k, v = (rng.standard_normal((1, 1, 640, 8)) for _ in range(3))
    mask, _ = oracle.select(q, k, 64, segs, 0.5)
    out = oracle.attention(q, k, v, 64, mask)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[:, :, 64:128] = rng.standard_normal((1, 1, 64, 8)) * 50
    mask2, _ = oracle.select(q2, k2, 64, segs, 0.5)
    out2 = oracle.attention(q2, k2, v2, 64, mask2)
    assert np.array_equal(mask, mask2)
    live = np.r_[0:64, 128:640]
    assert np.array_equal(out[:, :, live], out2[:, :, live])
    assert np.all(out2[:, :, 64:128] == 0)


# --------------------------------------------------------------------------
# 8-bit float E4M3 (quantized consumer).  The pages name no format; the facts
# pinned here are those of the OCP E4M3 encoding the oracle states it follows:
# bias 7, 3 mantissa bits, subnormals below 2^-6, one NaN pattern per sign,
# largest finite 448, round to nearest with ties to even.
# --------------------------------------------------------------------------

def test_e4m3_decode_known_values():
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x38] == 1.0 and d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9 and d[0x08] == 2.0 ** -6
    assert d[0x40] == 2.0 and d[0x44] == 3.0 and d[0x48] == 4.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and np.isnan(d).sum() == 2
    assert d[0x00] == 0.0 and d[0x80] == 0.0 and np.signbit(d[0x80])
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # strictly increasing magnitudes
    assert np.array_equal(d[0x80:0xFF], -d[0x00:0x7F])    # sign symmetry


def test_e4m3_encode_round_trip_and_ties_to_even():
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in list(range(0x00, 0x7F)) + list(range(0x81, 0xFF)):
        assert oracle.e4m3_encode(d[c]) == c
    assert oracle.e4m3_encode(-0.0) == 0x80
    for c in range(0x00, 0x7E):
        lo, hi = d[c], d[c + 1]
        mid = (lo + hi) / 2
        assert oracle.e4m3_encode(mid) == (c if c % 2 == 0 else c + 1)     # halfway: even code
        assert oracle.e4m3_encode(np.nextafter(np.float32(mid), np.float32(0))) == c
        assert oracle.e4m3_encode(np.nextafter(np.float32(mid), np.float32(1e9))) == c + 1
    assert oracle.e4m3_encode(1000.0) == 0x7E and oracle.e4m3_encode(-1000.0) == 0xFE


def test_e4m3_quantize_scale_and_error_bound():
    x = rnd((2, 3, 64, 16), 60).astype(np.float32).astype(np.float64)
    x[1, 2] = 0.0                                          # an all-zero head
    codes, scale = oracle.quantize_e4m3(x)
    assert scale[1, 2] == 1.0 and np.all(codes[1, 2] == 0)
    deq = oracle.dequantize_e4m3(codes, scale)
    for b in range(2):
        for h in range(3):
            if b == 1 and h == 2:
                continue
            i = np.unravel_index(np.abs(x[b, h]).argmax(), x[b, h].shape)
            assert codes[b, h][i] in (0x7E, 0xFE)          # the largest magnitude maps to 448
            assert scale[b, h] == np.float32(np.float32(np.abs(x[b, h]).max()) / np.float32(448))
            # round to nearest: within half a step of the neighbouring codes
            s = float(scale[b, h])
            err = np.abs(deq[b, h] - x[b, h]) / s
            mag = np.abs(x[b, h]) / s
            step = np.where(mag < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3))
            assert np.all(err <= step / 2 * (1 + 1e-6) + 1e-12)
