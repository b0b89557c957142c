"""C-ABI boundary tests on the CPU: exports, host geometry, validation codes.

No kernel is launched here: every call either is host-only or fails
validation, which returns before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads
from head_masked_attention_amd import _binding as B_

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7f0000100000            # 16-byte aligned, never dereferenced


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bsattn.h")).read()
    return sorted(set(re.findall(r"\b(bsattn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B_.EXPORTS)


def test_status_strings(lib):
    for s in range(10):
        assert B_.status_string(s)
    assert B_.status_string(0) == "ok"


@pytest.mark.parametrize("w", list(workloads.ALL.values()), ids=lambda w: w.name)
def test_layout_classes_match_oracle_on_workloads(lib, w):
    lay = B_.Layout(w.block, list(w.segments), w.window_tokens)
    cls, n = B_.layout_classes(lay, w.N)
    ref = oracle.classes(list(w.segments), w.N, w.block)
    assert np.array_equal(cls, ref)
    assert n == int((ref == 0).sum())


def test_layout_classes_match_oracle_on_random_layouts(lib):
    rng = np.random.default_rng(0)
    kinds = list(B_.SEG_KINDS)
    for trial in range(300):
        block = int(rng.choice([32, 64]))
        nseg = int(rng.integers(1, 12))
        lens = rng.integers(1, 200, size=nseg)
        N = int(lens.sum())
        pad = (-N) % block
        lens[-1] += pad
        N += pad
        segs = [(kinds[int(rng.integers(len(kinds)))], int(x)) for x in lens]
        cls, n = B_.layout_classes(B_.Layout(block, segs), N)
        ref = oracle.classes(segs, N, block)
        assert np.array_equal(cls, ref), segs


def test_budget_rule_matches_oracle(lib):
    for n in [0, 1, 2, 7, 8, 63, 64, 256, 512, 2048]:
        for b in [1e-6, 0.01, 0.1, 0.2, 0.25, 0.3, 1 / 3, 0.5, 0.7, 0.99, 1.0, 1.5, 7.0]:
            assert B_.budget_k(n, b) == oracle.budget(n, b), (n, b)
    # the workloads' k values
    assert B_.budget_k(8, 0.5) == (4, False)
    assert B_.budget_k(64, 0.3)[0] == 19 and B_.budget_k(256, 0.3)[0] == 76
    assert B_.budget_k(512, 0.3)[0] == 153 and B_.budget_k(63, 0.3)[0] == 18


def test_budget_fraction_of_candidates_keeps_that_many(lib):
    """bsattn_budget_k: the fraction k/n of n candidates keeps exactly k
    (the double nearest k/n, and two-decimal budgets such as 0.29 of 100),
    and a budget a hair below it keeps k - 1."""
    for n in range(1, 257):
        for k in range(1, n + 1):
            assert B_.budget_k(n, k / n)[0] == k, (k, n)
            if k > 1:
                assert B_.budget_k(n, (k - 1e-6) / n)[0] == k - 1, (k, n)
    for d in range(1, 100):
        for n in (100, 200, 400, 800, 1500, 2000):
            if d * n % 100 == 0:
                assert B_.budget_k(n, d / 100)[0] == d * n // 100, (d, n)


def test_head_mask_matches_oracle(lib):
    rng = np.random.default_rng(1)
    for trial in range(200):
        H = int(rng.integers(1, 40))
        imp = rng.integers(0, 5, size=H).astype(float) if trial % 2 else rng.random(H)
        sp = float(rng.choice([0.0, 0.25, 0.5, 0.75, 1.0]))
        mn = int(rng.integers(0, 6))
        assert np.array_equal(B_.head_mask(imp, sp, mn), oracle.head_mask(imp, sp, mn))
    for layer in (0, 21, 42, 63):
        imp = workloads.head_importance(workloads.STACK, layer)
        m = B_.head_mask(imp)
        assert m.sum() == 16 and np.array_equal(m, oracle.head_mask(imp, 0.5, 4))


# ----- validation codes --------------------------------------------------------

def tensor(B=1, H=2, N=256, D=64, dtype=B_.BF16, data=FAKE, sn=None, sh=None, sb=None):
    sn = D if sn is None else sn
    sh = N * sn if sh is None else sh
    sb = H * sh if sb is None else sb
    return B_._Tensor(data, dtype, B, H, N, D, sb, sh, sn)


def bmask(B=1, H=2, nb=4, null=False):
    return B_._BlockMask(B, H, nb, nb, 0 if null else FAKE, FAKE, FAKE, -7, -7)


def layout(block=64, segs=(), window=0):
    lay, keep = B_.Layout(block, list(segs), window)._c()
    return lay, keep


def call_select(lib, q, k, lay, budget, out, ws=FAKE, ws_bytes=1 << 30):
    return lib.bsattn_select(ctypes.byref(q), ctypes.byref(k), ctypes.byref(lay), budget,
                             ctypes.byref(out), ws, ws_bytes, None)


def test_select_validation(lib):
    lay, _k = layout()
    q, k = tensor(), tensor()
    cases = [
        (dict(q=tensor(data=0)), 1),
        (dict(q=tensor(dtype=5)), 2),
        (dict(k=tensor(dtype=B_.F32)), 2),
        (dict(q=tensor(D=48)), 3),
        (dict(q=tensor(N=250, sn=64)), 3),
        (dict(k=tensor(H=3)), 3),
        (dict(q=tensor(data=FAKE + 2)), 4),
        (dict(q=tensor(sn=60)), 4),
        (dict(out=bmask(null=True)), 1),
        (dict(out=bmask(nb=5)), 3),
        (dict(out=bmask(H=1)), 3),
        (dict(budget=0.0), 6),
        (dict(budget=float("nan")), 6),
        (dict(budget=-1.0), 6),
        (dict(ws=0), 7),
        (dict(ws_bytes=100), 7),
        (dict(ws=FAKE + 16), 7),
    ]
    for over, code in cases:
        args = dict(q=q, k=k, lay=lay, budget=0.3, out=bmask(), ws=FAKE, ws_bytes=1 << 30)
        args.update(over)
        out = args["out"]
        st = call_select(lib, args["q"], args["k"], args["lay"], args["budget"], out,
                         args["ws"], args["ws_bytes"])
        assert st == code, (over, st)
        assert out.k == -7 and out.is_dense == -7          # untouched on error


def test_select_no_alloc_validation(lib):
    """bsattn_select_no_alloc: the validation codes of bsattn_select, and
    BSATTN_ERR_WORKSPACE when the pooled sums would not fit its scratch --
    all returned before any HIP call (so on the CPU too)."""
    lay, _k = layout()
    for over, code in [(dict(q=tensor(data=0)), 1), (dict(q=tensor(D=48)), 3), (dict(budget=0.0), 6),
                       (dict(out=bmask(nb=5)), 3)]:
        args = dict(q=tensor(), k=tensor(), budget=0.3, out=bmask())
        args.update(over)
        st = lib.bsattn_select_no_alloc(ctypes.byref(args["q"]), ctypes.byref(args["k"]), ctypes.byref(lay),
                                        args["budget"], ctypes.byref(args["out"]), None)
        assert st == code, (over, st)
        assert args["out"].k == -7
    # 64 heads x 1024 blocks x D 128: 128 MiB of pooled sums, over the 32 MiB scratch
    big = tensor(H=64, N=64 * 1024, D=128)
    out = bmask(H=64, nb=1024)
    assert B_.select_workspace_bytes(1, 64, 64, 64 * 1024, 64, 128) > 32 << 20
    st = lib.bsattn_select_no_alloc(ctypes.byref(big), ctypes.byref(big), ctypes.byref(lay), 0.3,
                                    ctypes.byref(out), None)
    assert st == 7 and out.k == -7


def test_select_layout_errors(lib):
    q, k = tensor(), tensor()
    for segs, code in [([("text", 100)], 5), ([("image", 128), ("text", 100)], 5),
                       ([("image", 256), ("padding", 0)], 5), ([(9, 256)], 5)]:
        lay, _k = layout(segs=segs)
        assert call_select(lib, q, k, lay, 0.3, bmask()) == code
    lay, _k = layout(block=48)
    assert call_select(lib, q, k, lay, 0.3, bmask()) == 3
    too_many = [("image", 8)] * 32 + [("text", 0)]
    lay, _k = layout(segs=too_many)
    assert call_select(lib, q, k, lay, 0.3, bmask()) == 5
    lay, _k = layout(window=-1)
    assert call_select(lib, q, k, lay, 0.3, bmask()) == 5


def test_select_unsupported_candidate_count(lib):
    N = 64 * 2100
    q, k = tensor(N=N, D=32), tensor(N=N, D=32)
    lay, _k = layout()
    assert call_select(lib, q, k, lay, 0.3, bmask(nb=2100)) == 9


def test_select_item_count_limit(lib):
    # the pool kernel indexes B * (H + Hkv) * n_cand items in 32 bits
    B, H, N = 1 << 20, 1024, 64 * 64
    q, k = tensor(B=B, H=H, N=N), tensor(B=B, H=H, N=N)
    lay, _k = layout()
    assert call_select(lib, q, k, lay, 0.3, bmask(B=B, H=H, nb=64)) == 3
    B = 1 << 8                                          # 2^8 * 2048 * 64 items pass; the 1 GiB workspace is too small
    q, k = tensor(B=B, H=H, N=N), tensor(B=B, H=H, N=N)
    assert call_select(lib, q, k, lay, 0.3, bmask(B=B, H=H, nb=64)) == 7


def test_select_forward_validation(lib):
    # the fused shape (bf16, D 64, block 64, no segments, <= 64 blocks) and one that runs the two calls
    lay, _k = layout()
    for N, D in ((64 * 16, 64), (64 * 16, 128)):
        q, k, v, out = tensor(N=N, D=D), tensor(N=N, D=D), tensor(N=N, D=D), tensor(N=N, D=D)
        call = lambda m, budget=0.3, ws=FAKE: lib.bsattn_select_forward(
            ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(lay), budget, None, 0.0,
            ctypes.byref(out), None if m is None else ctypes.byref(m), ws, 1 << 30, None)
        assert call(None) == 1                          # the mask is an output here: required
        assert call(bmask(nb=8)) == 3                   # wrong number of blocks
        assert call(bmask(nb=16), budget=0.0) == 6      # budget out of range
        assert call(bmask(nb=16), ws=None) == 7         # no workspace


def call_forward(lib, q, k, v, m, out, scale=0.0):
    return lib.bsattn_forward(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                              None if m is None else ctypes.byref(m), None, scale,
                              ctypes.byref(out), None)


def test_forward_validation(lib):
    cases = [
        (dict(q=tensor(data=0)), 1),
        (dict(v=tensor(dtype=B_.F32)), 2),
        (dict(out=tensor(dtype=B_.F32)), 2),
        (dict(k=tensor(N=128)), 3),
        (dict(v=tensor(H=1)), 3),
        (dict(out=tensor(D=32)), 3),
        (dict(m=bmask(nb=3)), 3),              # 256 / 3 not integral
        (dict(m=bmask(nb=16)), 3),             # block 16 unsupported
        (dict(m=bmask(B=2)), 3),
        (dict(m=B_._BlockMask(1, 2, 4, 4, FAKE, 0, FAKE, 0, 0)), 1),
        (dict(scale=float("inf")), 6),
        (dict(q=tensor(sn=72, sh=256 * 72 + 4)), 4),
        (dict(k=tensor(sn=1 << 24, sh=256 << 24)), 4),     # row pitch 32 MiB
    ]
    for over, code in cases:
        args = dict(q=tensor(), k=tensor(), v=tensor(), m=bmask(), out=tensor(), scale=0.0)
        args.update(over)
        st = call_forward(lib, args["q"], args["k"], args["v"], args["m"], args["out"], args["scale"])
        assert st == code, (over, st)


def test_forward_masked_validation(lib):
    def call(km, sb, **over):
        args = dict(q=tensor(), k=tensor(), v=tensor(), m=bmask(), out=tensor())
        args.update(over)
        return lib.bsattn_forward_masked(ctypes.byref(args["q"]), ctypes.byref(args["k"]),
                                         ctypes.byref(args["v"]), ctypes.byref(args["m"]), None, km, sb,
                                         0.0, ctypes.byref(args["out"]), None)
    assert call(FAKE, 100) == 4                # batch stride shorter than N = 256
    assert call(FAKE, -256) == 4
    assert call(FAKE, 256, q=tensor(data=0)) == 1      # tensor checks come first
    assert call(FAKE, 0, out=tensor(dtype=B_.F32)) == 2


def test_fp8_entry_points_validation(lib):
    f8 = lambda **kw: tensor(dtype=B_.FP8_E4M3, **kw)
    m = bmask()
    fwd8 = lambda q, k, v, out, scales=(FAKE, FAKE, FAKE): lib.bsattn_forward_fp8(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), scales[0], scales[1], scales[2], ctypes.byref(m),
        None, 0.0, ctypes.byref(out), None)
    assert fwd8(tensor(), f8(), f8(), tensor()) == 2              # bf16 q
    assert fwd8(f8(), f8(), f8(), tensor(dtype=B_.F32)) == 2     # out must be bf16
    assert fwd8(f8(), f8(), f8(), tensor(), scales=(None, FAKE, FAKE)) == 1
    assert fwd8(f8(D=32), f8(D=32), f8(D=32), tensor(D=32)) == 9  # no kernel for D = 32
    fwd8m = lambda km, sb, q=None: lib.bsattn_forward_fp8_masked(
        ctypes.byref(q or f8()), ctypes.byref(f8()), ctypes.byref(f8()), FAKE, FAKE, FAKE, ctypes.byref(m),
        None, km, sb, 0.0, ctypes.byref(tensor()), None)
    assert fwd8m(FAKE, 100) == 4                  # key-mask batch stride shorter than N = 256
    assert fwd8m(FAKE, -256) == 4
    assert fwd8m(FAKE, 256, q=tensor()) == 2      # tensor checks come first
    # the bf16/fp32 entry points refuse E4M3 codes
    assert call_forward(lib, f8(), f8(), f8(), m, tensor()) == 2
    x, y = tensor(), f8()
    assert lib.bsattn_quantize_fp8(ctypes.byref(x), ctypes.byref(y), FAKE, FAKE, 3, None) == 7   # scratch too small
    assert lib.bsattn_quantize_fp8(ctypes.byref(y), ctypes.byref(y), FAKE, FAKE, 64, None) == 2


def test_radial_and_density_validation(lib):
    lay, _k = layout()
    out = bmask()
    assert lib.bsattn_radial(ctypes.byref(lay), 0.0, ctypes.byref(out), None) == 6
    assert lib.bsattn_radial(None, 0.3, ctypes.byref(out), None) == 1
    bad = bmask(nb=4)
    bad.nkb = 5
    assert lib.bsattn_radial(ctypes.byref(lay), 0.3, ctypes.byref(bad), None) == 3
    d = ctypes.c_double()
    assert lib.bsattn_mask_density(None, None, ctypes.byref(d)) == 1
    z = bmask()
    z.B = 0
    assert lib.bsattn_mask_density(ctypes.byref(z), None, ctypes.byref(d)) == 3


def test_head_mask_validation(lib):
    imp = np.zeros(4)
    out = np.zeros(4, np.uint8)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.bsattn_head_mask(None, 4, 0.5, 4, p(out)) == 1
    assert lib.bsattn_head_mask(p(imp), 0, 0.5, 4, p(out)) == 3
    assert lib.bsattn_head_mask(p(imp), 4, 1.5, 4, p(out)) == 6
    assert lib.bsattn_head_mask(p(imp), 4, 0.5, -1, p(out)) == 6
    imp[2] = np.nan
    assert lib.bsattn_head_mask(p(imp), 4, 0.5, 4, p(out)) == 6


def test_workspace_bytes(lib):
    # per tensor: float32 hi and lo parts of the block sums ([heads][rows][D]
    # each) and one float norm bound per row; every part 256-byte aligned
    def a256(x):
        return 256 * ((x + 255) // 256)

    def expect(B, H, Hkv, rows, D):
        return 2 * (a256(B * H * rows * D * 4) + a256(B * Hkv * rows * D * 4)) + \
            a256(B * H * rows * 4) + a256(B * Hkv * rows * 4)
    assert B_.select_workspace_bytes(2, 10, 10, 4096, 64, 64) == expect(2, 10, 10, 64, 64)
    assert B_.select_workspace_bytes(2, 10, 10, 4096, 64, 64) == 2 * 2 * 2 * 10 * 64 * 64 * 4 + 2 * 2 * 10 * 64 * 4
    assert B_.select_workspace_bytes(1, 4, 2, 512, 32, 32) == expect(1, 4, 2, 16, 32)
    assert B_.select_workspace_bytes(1, 1, 1, 512, 48, 32) == 0


def test_empty_inputs_are_rejected_before_any_launch(lib):
    """A sequence, batch or head count of zero is a shape error (code 3) at
    every entry point, returned before anything is enqueued; the outputs are
    left untouched."""
    lay, _k = layout()
    for over in (dict(N=0), dict(B=0), dict(H=0)):
        q = tensor(**over)
        out = bmask()
        assert call_select(lib, q, tensor(), lay, 0.3, out) == 3, over
        assert call_select(lib, tensor(), q, lay, 0.3, out) == 3, over
        assert out.k == -7 and out.is_dense == -7
        assert call_forward(lib, q, tensor(), tensor(), bmask(), tensor()) == 3, over
        assert call_forward(lib, tensor(), tensor(), tensor(), bmask(), q) == 3, over
        assert lib.bsattn_select_forward(
            ctypes.byref(q), ctypes.byref(tensor()), ctypes.byref(tensor()), ctypes.byref(lay), 0.3, None, 0.0,
            ctypes.byref(tensor()), ctypes.byref(bmask()), FAKE, 1 << 30, None) == 3, over
    # a mask with no blocks
    assert call_forward(lib, tensor(), tensor(), tensor(), bmask(nb=0), tensor()) == 3
    out = bmask(nb=0)
    assert lib.bsattn_radial(ctypes.byref(lay), 0.3, ctypes.byref(out), None) == 3
    assert out.k == -7


def test_select_heads_validation(lib):
    """bsattn_select_heads validates as bsattn_select does (the head mask is a
    device pointer read by the kernels; NULL means every head)."""
    lay, _k = layout()
    call = lambda q, k, out, budget=0.3, ws=FAKE, ws_bytes=1 << 30, hmask=None: lib.bsattn_select_heads(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(lay), budget, hmask, ctypes.byref(out), ws, ws_bytes, None)
    for hmask in (None, FAKE):
        for over, code in ((dict(q=tensor(data=0)), 1), (dict(q=tensor(D=48)), 3), (dict(out=bmask(nb=5)), 3),
                           (dict(budget=0.0), 6), (dict(ws=0), 7), (dict(q=tensor(N=0)), 3)):
            args = dict(q=tensor(), k=tensor(), out=bmask(), budget=0.3, ws=FAKE)
            args.update(over)
            out = args["out"]
            assert call(args["q"], args["k"], out, args["budget"], args["ws"], hmask=hmask) == code, (over, hmask)
            assert out.k == -7 and out.is_dense == -7
