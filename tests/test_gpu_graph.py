"""The whole step captured in a HIP graph (torch.cuda.graph on the library's
stream argument): the library launches kernels only, with no allocation,
copy, fill or host synchronisation, so one step records as a graph. Each of
several replays, with eager work and synchronisation between them, must
equal the eager step bit for bit. The step runs with and without the run
table that the Top-k writes for the reduce."""
import numpy as np
import pytest
import torch

import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import assert_bits_equal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("table", [False, True])
def test_step_replays_in_a_graph(dev, table):
    w = W.workload(4, N=500009, P=8)
    P, N, k, B = w.P, w.N, w.k, w.q4_bucket
    g = W.gradients(w, 0, device=dev)
    r0 = (W.gradients(w, 1, device=dev) * 0.25).contiguous()
    off = [p * k for p in range(P + 1)]
    r = torch.empty_like(r0)
    ws = torch.empty(sg.topk_ef_workspace_bytes(P, N, k), dtype=torch.uint8, device=dev)
    idx = torch.empty((P, k), dtype=torch.int32, device=dev)
    val = torch.empty((P, k), dtype=torch.float32, device=dev)
    codes = torch.empty((P, (k + 1) // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((P, (k + B - 1) // B), dtype=torch.float32, device=dev)
    deq = torch.empty((P, k), dtype=torch.float32, device=dev)
    T = sg.dense_threshold(w.delta, N)
    ri = torch.empty(max(1, min(N, T - 1)), dtype=torch.int32, device=dev)
    rv = torch.empty(N, dtype=torch.float32, device=dev)
    res = torch.zeros(16, dtype=torch.uint8, device=dev)
    wsr = torch.empty(sg.sparse_reduce_workspace_bytes(P, N, P * k), dtype=torch.uint8, device=dev)
    tab = torch.zeros(sg.run_table_shape(P, N), dtype=torch.int32, device=dev) if table else None

    def step():
        sg.topk_ef(g, r, k, out_idx=idx, out_val=val, workspace=ws, runs=tab)
        sg.q4(val, B, 5, 1, codes=codes, scales=scales)
        sg.dq4(codes, scales, k, B, out=deq)
        sg.sparse_reduce(off, idx.view(-1), deq.view(-1), N, w.delta, out_idx=ri, out_val=rv, result=res,
                         workspace=wsr, runs=tab)

    def outputs():
        K, dense, flags = sg.ReduceOutput(res, ri, rv, N).read()
        assert flags == 0
        return [r.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy(), codes.cpu().numpy(),
                scales.cpu().numpy(), np.array([K, int(dense)]), ri[:K].cpu().numpy(), rv[:K].cpu().numpy()]

    r.copy_(r0)
    step()
    torch.cuda.synchronize()
    eager = outputs()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r.copy_(r0)
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        r.copy_(r0)
        idx.zero_()
        rv.zero_()
        res.zero_()
        if table:
            tab.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"graph replay {rep}", flush=True)
        for a, b in zip(eager, outputs()):
            assert_bits_equal(a, b, f"replay {rep}")
        (g * 0.5).sum().item()  # unrelated eager work between replays
