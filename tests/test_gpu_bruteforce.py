"""Every 3x3 block mask through the GPU forward, against the oracle.

The SD.Next commit page checks its consumer by tile equivalence against sdpa
fed the same tiles; here every one of the 512 block masks of a 3x3 grid runs
at once, one mask per head, under two head masks (all heads, and every other
head), and every output row is compared with the oracle's masked-dense
attention: bf16 with 64-token blocks at D 64 and 128 (the MFMA kernel), fp32
with 32-token blocks (the fp32 path).  Masked heads and rows whose mask row is
empty must be exactly zero.
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_close, to64, upload_mask

pytestmark = pytest.mark.gpu


def all_3x3_masks() -> np.ndarray:
    """[1, 512, 3, 3]: head h holds the mask whose bits are h (row-major)."""
    bits = (np.arange(512)[:, None] >> np.arange(9)[None, :]) & 1
    return bits.reshape(1, 512, 3, 3).astype(np.uint8)


@pytest.mark.parametrize("dtype,D,block", [("bf16", 64, 64), ("bf16", 128, 64), ("fp32", 32, 32)],
                         ids=["bf16_d64", "bf16_d128", "fp32_d32_block32"])
def test_every_3x3_mask(cuda, dtype, D, block):
    masks = all_3x3_masks()
    H, N = 512, 3 * block
    q, k, v = workloads.small_case(B=1, H=H, N=N, D=D, block=block, dtype=dtype, seed=51)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    bm = upload_mask(masks, cuda)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    empty = np.repeat(masks[0].sum(-1) == 0, block, axis=-1)          # [H, N]
    for hmask in (np.ones(H, np.uint8), (np.arange(H) % 2).astype(np.uint8)):
        out = hm.forward(qd, kd, vd, bm, torch.from_numpy(hmask).to(cuda))
        torch.cuda.synchronize()
        ref = oracle.attention(q64, k64, v64, block, masks, head_mask=hmask)
        got = to64(out)
        assert_close(got, ref, dtype, f"3x3 masks, {int(hmask.sum())} active heads")
        assert np.all(got[0, hmask == 0] == 0)
        assert np.all(got[0][empty] == 0)
