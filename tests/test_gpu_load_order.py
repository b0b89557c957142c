"""The library works when it is loaded before anything else touched HIP."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODE = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import head_masked_attention_amd as hm
hm.load_library()                      # before torch initialises the HIP runtime
import torch, workloads
q, k, v = workloads.small_case(B=1, H=2, N=64 * 8, D=64, seed=3, device="cuda")
bm = hm.select(q, k, hm.Layout(64, []), 0.5)
out = hm.forward(q, k, v, bm)
torch.cuda.synchronize()
assert int(bm.count.sum()) == 2 * 8 * 4
assert torch.isfinite(out.float()).all()
print("load-order ok")
"""


def test_library_loaded_before_torch(cuda):
    res = subprocess.run([sys.executable, "-c", CODE, ROOT], capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "load-order ok" in res.stdout
