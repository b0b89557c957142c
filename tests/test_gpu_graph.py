"""Select + forward (and the fused select_forward) captured in a HIP graph: every replay equals the eager result.

The graph is replayed several times with eager work and synchronisations in
between, and each replay is compared bitwise with the eager step.
"""
import pytest
import torch

import head_masked_attention_amd as hm
import workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["sdxl_bf16", "tiny_fp32"])
def test_graph_replays_match_eager(cuda, name):
    w = workloads.ALL[name]
    q, k, v = (t.to(cuda) for t in workloads.make_qkv(w))
    layout = hm.Layout(w.block, list(w.segments), w.window_tokens)
    hmask = None if w.head_mask is None else torch.tensor(w.head_mask, dtype=torch.uint8, device=cuda)
    bm = hm.empty_block_mask(w.B, w.H, w.nb, cuda)
    ws = torch.empty(hm.select_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.block, w.D),
                     dtype=torch.uint8, device=cuda)
    out = torch.empty_like(q)
    # eager reference
    ref_bm = hm.select(q, k, layout, w.budget)
    ref = hm.forward(q, k, v, ref_bm, hmask)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(cuda)
    cap.wait_stream(torch.cuda.current_stream(cuda))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            hm.select(q, k, layout, w.budget, out=bm, workspace=ws, stream=cap)
            hm.forward(q, k, v, bm, hmask, out=out, stream=cap)
    torch.cuda.current_stream(cuda).wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        bm.mask.zero_()
        bm.count.zero_()
        junk = torch.randn(1024, 1024, device=cuda) @ torch.randn(1024, 1024, device=cuda)   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bm.mask, ref_bm.mask), rep
        assert torch.equal(bm.count, ref_bm.count), rep
        assert torch.equal(out, ref), rep
        del junk


def test_graph_replays_of_select_forward_match_eager(cuda):
    # bsattn_select_forward on the SDXL shape (the fused ranking) captured once
    # and replayed with eager work in between: every replay equals the eager call
    w = workloads.SDXL
    q, k, v = (t.to(cuda) for t in workloads.make_qkv(w))
    layout = hm.Layout(w.block, [], 0)
    bm = hm.empty_block_mask(w.B, w.H, w.nb, cuda)
    ws = torch.empty(hm.select_workspace_bytes(w.B, w.H, w.kv_heads, w.N, w.block, w.D),
                     dtype=torch.uint8, device=cuda)
    out = torch.empty_like(q)
    ref, ref_bm = hm.select_forward(q, k, v, layout, w.budget)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(cuda)
    cap.wait_stream(torch.cuda.current_stream(cuda))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            hm.select_forward(q, k, v, layout, w.budget, out=out, block_mask=bm, workspace=ws, stream=cap)
    torch.cuda.current_stream(cuda).wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        bm.mask.zero_()
        bm.count.zero_()
        junk = torch.randn(1024, 1024, device=cuda) @ torch.randn(1024, 1024, device=cuda)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bm.mask, ref_bm.mask), rep
        assert torch.equal(bm.count, ref_bm.count), rep
        assert torch.equal(out, ref), rep
        del junk
