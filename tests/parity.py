"""Helpers shared by the GPU parity tests (comparison and marshalling only)."""
import numpy as np
import torch

BF16_MAX_ABS = 2e-2     # bf16 outputs: max abs error against the fp64 oracle
BF16_MEAN_ABS = 2e-3    # bf16 outputs: mean abs error
F32_MAX_ABS = 1e-5      # fp32 outputs: max abs error


def to64(t) -> np.ndarray:
    """Exact float64 copy of a (bf16 or fp32) tensor."""
    return t.detach().to("cpu").double().numpy()


def csr_from_mask(mask: np.ndarray):
    """count and ascending index lists of a 0/1 mask [..., nkb]."""
    m = mask.astype(bool)
    count = m.sum(-1).astype(np.int32)
    index = np.argsort(~m, axis=-1, kind="stable").astype(np.int32)
    return count, index


def upload_mask(mask: np.ndarray, device):
    """A BlockMask holding the oracle's mask, for feeding the GPU forward."""
    import head_masked_attention_amd as hm
    m = mask if mask.ndim == 4 else mask[None, None]
    count, index = csr_from_mask(m)
    return hm.BlockMask(torch.from_numpy(np.ascontiguousarray(m, dtype=np.uint8)).to(device),
                        torch.from_numpy(count).to(device), torch.from_numpy(index).to(device))


def download_mask(bm):
    return (bm.mask.cpu().numpy(), bm.count.cpu().numpy(), bm.index.cpu().numpy())


def assert_csr_consistent(mask, count, index):
    """count = row sums; the first count index entries = ascending kept columns."""
    assert np.array_equal(count, mask.sum(-1).astype(np.int32))
    flat_m = mask.reshape(-1, mask.shape[-1])
    flat_c = count.reshape(-1)
    flat_i = index.reshape(-1, index.shape[-1])
    for r in range(flat_m.shape[0]):
        expect = np.nonzero(flat_m[r])[0]
        assert np.array_equal(flat_i[r, :flat_c[r]], expect), f"row {r}"


def compare_masks(bm, oracle_mask, near_tie):
    """Bit-exact mask comparison outside the oracle's near-tie rows.

    Returns the number of excluded (near-tie) rows.  The CSR lists are checked
    for consistency with the GPU's own mask on every row.
    """
    m, c, i = download_mask(bm)
    assert m.shape == oracle_mask.shape
    assert set(np.unique(m).tolist()) <= {0, 1}
    assert_csr_consistent(m, c, i)
    keep = near_tie == 0
    diff = (m != oracle_mask).any(-1) & keep
    assert not diff.any(), f"{int(diff.sum())} rows differ, first at {np.argwhere(diff)[0].tolist()}"
    return int((~keep).sum())


def assert_close(out_gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    err = np.abs(out_gpu.astype(np.float64) - ref)
    if dtype == "fp32":
        assert err.max() <= F32_MAX_ABS, f"{what}: max abs {err.max():.3g}"
    else:
        assert err.max() <= BF16_MAX_ABS, f"{what}: max abs {err.max():.3g}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean abs {err.mean():.3g}"
    return float(err.max()), float(err.mean())


def sample_rows(B, H, nb, block, blocks_per_head, rows_per_block, seed):
    """(b, h, t) triples: the given query blocks of every (b, h), a few rows each."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(B):
        for h in range(H):
            for qb in blocks_per_head(b, h, rng):
                ts = rng.choice(block, size=min(rows_per_block, block), replace=False)
                out.extend((b, h, qb * block + int(t)) for t in ts)
    return np.array(out, dtype=np.int64)
