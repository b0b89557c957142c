"""Calls on a stream other than torch's current one.

The binding allocates each call's temporaries (the selector workspace, the
block mask that sparse_attention builds, the fp8 quantiser's scratch) and
default outputs while `stream` is current, so the caching allocator ties
them to the stream the kernels run on: a temporary dropped on return is not
handed to other work until that stream has passed the kernels that use it.
"""
import numpy as np
import pytest
import torch

import head_masked_attention_amd as hm
import oracle
import workloads
from parity import assert_close, compare_masks, to64

pytestmark = pytest.mark.gpu


def _allocs_during(fn, device):
    """Run fn with the allocator's history on; return (result, alloc events)."""
    torch.cuda.synchronize()
    torch.cuda.memory._record_memory_history(max_entries=100000)
    try:
        res = fn()
        snap = torch.cuda.memory._snapshot()
    finally:
        torch.cuda.memory._record_memory_history(enabled=None)
    traces = snap["device_traces"][device.index]
    return res, [e for e in traces if e["action"] == "alloc"]


def test_temporaries_live_on_the_call_stream(lib, cuda):
    q, k, v = workloads.small_case(B=1, H=4, N=64 * 24, D=64, seed=21)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    side = torch.cuda.Stream(cuda)
    side.wait_stream(torch.cuda.current_stream(cuda))
    stage = hm.Stage(min_length=0, schedule=0.3)

    def calls():
        bm = hm.select(qd, kd, hm.Layout(64, []), 0.3, stream=side)
        o1 = hm.forward(qd, kd, vd, bm, stream=side)
        o2, bm2 = hm.select_forward(qd, kd, vd, hm.Layout(64, []), 0.3, stream=side)
        o3, _d = hm.sparse_attention(qd, kd, vd, stage, hm.Layout(64, []), stream=side)
        q8, qs = hm.quantize_fp8(qd, stream=side)
        rad = hm.radial(hm.Layout(64, []), qd.shape[2], 0.3, device=cuda, stream=side)
        return bm, o1, o2, bm2, o3, q8, qs, rad

    res, allocs = _allocs_during(calls, cuda)
    side.synchronize()
    assert len(allocs) >= 8, "the calls should have allocated their temporaries and outputs"
    streams = {e["stream"] for e in allocs}
    assert streams == {side.cuda_stream}, f"allocations on streams {streams}, call stream {side.cuda_stream}"
    stage.close()


def test_side_stream_behind_long_work_with_current_stream_churn(lib, cuda):
    """select + forward on a side stream that is held behind a long kernel,
    while the current stream allocates and fills buffers of the same sizes:
    the masks equal the oracle's and the output is within the bf16 bar."""
    B, H, nb, D = 1, 6, 32, 64
    q, k, v = workloads.small_case(B=B, H=H, N=64 * nb, D=D, seed=22)
    qd, kd, vd = q.to(cuda), k.to(cuda), v.to(cuda)
    cur = torch.cuda.current_stream(cuda)
    side = torch.cuda.Stream(cuda)
    side.wait_stream(cur)
    need = hm.select_workspace_bytes(B, H, H, 64 * nb, 64, D)
    with torch.cuda.stream(side):
        a = torch.rand(2048, 2048, device=cuda)
        for _ in range(40):
            a = torch.tanh(a @ a)
    bm = hm.select(qd, kd, hm.Layout(64, []), 0.3, stream=side)
    out = hm.forward(qd, kd, vd, bm, stream=side)
    junk = []
    for _ in range(6):
        junk.append(torch.full((need,), 0x7F, dtype=torch.uint8, device=cuda))
        junk.append(torch.zeros((B, H, nb), dtype=torch.int32, device=cuda))
        junk.append(torch.full((B, H, nb, nb), 1, dtype=torch.uint8, device=cuda))
    torch.cuda.synchronize()
    ref_mask, tie = oracle.select(to64(q), to64(k), 64, [], 0.3)
    compare_masks(bm, ref_mask, tie)
    ref = oracle.attention(to64(q), to64(k), to64(v), 64, bm.mask.cpu().numpy())
    assert_close(out.float().cpu().numpy(), ref, "bf16", "side-stream forward")
    del junk, a


def test_concurrent_host_threads(cuda):
    """Four host threads, each with its own stream and inputs, call select,
    forward, select_forward, select_heads and the fp8 pair at once (ctypes releases the
    interpreter lock, so the library's entry points run concurrently).  Every
    result equals the same calls made one after another on one thread."""
    import threading
    cases = []
    for i in range(4):
        D = 64 if i % 2 == 0 else 128
        q, k, v = workloads.small_case(B=1, H=4, Hkv=2, N=64 * (10 + 3 * i), D=D, seed=300 + i)
        cases.append((q.to(cuda), k.to(cuda), v.to(cuda)))
    lay = hm.Layout(64, [])
    hmd = torch.tensor([1, 0, 0, 1], dtype=torch.uint8, device=cuda)

    def work(qd, kd, vd, stream):
        bm = hm.select(qd, kd, lay, 0.3, stream=stream)
        out = hm.forward(qd, kd, vd, bm, stream=stream)
        out_f, bm_f = hm.select_forward(qd, kd, vd, lay, 0.3, stream=stream)
        bm_h = hm.select_heads(qd, kd, lay, 0.3, hmd, stream=stream)
        q8, qs = hm.quantize_fp8(qd, stream=stream)
        k8, ks = hm.quantize_fp8(kd, stream=stream)
        v8, vs = hm.quantize_fp8(vd, stream=stream)
        out8 = hm.forward_fp8(q8, k8, v8, qs, ks, vs, bm, stream=stream)
        return bm.mask, out, bm_f.mask, out_f, out8, bm_h.mask, bm_h.count

    serial = [work(*c, torch.cuda.current_stream(cuda)) for c in cases]
    torch.cuda.synchronize()
    serial = [[t.clone() for t in r] for r in serial]
    results = [None] * len(cases)
    errors = []
    streams = [torch.cuda.Stream(cuda) for _ in cases]

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    results[i] = work(*cases[i], streams[i])
        except Exception as e:       # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for want, got in zip(serial, results):
        for a, b in zip(want, got):
            assert torch.equal(a, b)
