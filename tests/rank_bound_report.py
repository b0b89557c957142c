"""How often the selector's float32 ranking needs its float64 band pass.

For each workload (a few heads of the large ones), computes the exact block
sums in float64, the scores of every sparsifiable row, and the selector's
certification margin at the budget boundary, M = 2 err + 2 T, with
err = (2 D + 16) 2^-24 |Q_i| max_j |K_j| and T = 2^(IB - 22) max(|a|, |b|)
the resolution of its 32-bit rank keys (IB index bits; 0 above 512
candidates, where the keys are 64-bit).  Prints the share of rows with a boundary gap below M
(they take the band pass), the smallest and median ratio gap / M, and the
oracle's near-tie share for comparison.

    python tests/rank_bound_report.py [workload ...]

A measurement of the inputs, run by hand; not collected by pytest.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def report(name, max_heads=4):
    w = workloads.ALL[name]
    q, k, _ = workloads.make_qkv(w)
    cls = oracle.classes(list(w.segments), w.N, w.block) if w.segments else np.zeros(w.nb, np.uint8)
    cand = np.nonzero(cls == oracle.SPARSE)[0]
    n = len(cand)
    kk = oracle.budget(n, w.budget)[0]
    npad = 64
    while npad < n:
        npad *= 2
    ib = int(np.log2(npad))
    tfac = 2.0 ** (ib - 22) if npad <= 512 else 0.0
    H = min(w.H, max_heads)
    ratios, near = [], 0
    for b in range(w.B):
        for h in range(H):
            qb = q[b, h].double().reshape(w.nb, w.block, w.D).sum(1).numpy()[cand]
            kb = k[b, h * w.kv_heads // w.H].double().reshape(w.nb, w.block, w.D).sum(1).numpy()[cand]
            S = qb @ kb.T
            qn = np.linalg.norm(qb, axis=1)
            kmax = np.linalg.norm(kb, axis=1).max()
            err = (2 * w.D + 16) * 2.0 ** -24 * qn * kmax
            for i in range(n):
                if kk < 2 or kk >= n:
                    continue
                o = np.sort(np.delete(S[i], i))[::-1]
                a, bb = o[kk - 2], o[kk - 1]
                M = 2 * err[i] + 2 * tfac * max(abs(a), abs(bb))
                ratios.append((a - bb) / M)
                near += abs(a - bb) <= 1e-4 * max(abs(a), abs(bb))
    r = np.array(ratios)
    print(f"{name}: heads {H} of {w.H}, rows {len(r)}, n_cand {n}, k {kk}: band pass {np.mean(r <= 1):.2%}, "
          f"gap/M min {r.min():.3g} median {np.median(r):.3g}; oracle near ties {near / len(r):.2%}", flush=True)


if __name__ == "__main__":
    for nm in sys.argv[1:] or ["sdxl_bf16", "joint_text_image_bf16", "video_radial_bf16", "head_masked_stack_bf16"]:
        report(nm)
