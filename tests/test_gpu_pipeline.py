"""GPU parity of the whole hot path, step by step against the oracle:
error-feedback Top-k -> (4-bit quantize -> dequantize) -> sparse reduce,
with the residual carried between steps."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import assert_bits_equal, reduce_tolerance

pytestmark = pytest.mark.gpu


def _pipeline(w, dev, seed=20240601):
    r_o = np.zeros((w.P, w.N), np.float32)
    rd = torch.zeros((w.P, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(sg.topk_ef_workspace_bytes(w.P, w.N, w.k), dtype=torch.uint8, device=dev)
    off = [p * w.k for p in range(w.P + 1)]
    dense_steps = []
    for step in range(w.steps):
        g = W.gradients(w, step).numpy()
        oi, ov, r_o = oracle.topk_ef(g, r_o, w.k)
        gi, gv = sg.topk_ef(torch.from_numpy(g).to(dev), rd, w.k, workspace=ws)
        if w.q4_bucket:
            oc, osc = oracle.q4(ov, w.q4_bucket, seed, step)
            ov = oracle.dq4(oc, osc, w.k, w.q4_bucket)
            gc, gsc = sg.q4(gv, w.q4_bucket, seed, step)
            gv = sg.dq4(gc, gsc, w.k, w.q4_bucket)
            assert_bits_equal(gc.cpu().numpy(), oc, f"codes step {step}")
        assert_bits_equal(gi.cpu().numpy().view(np.uint32), oi, f"idx step {step}")
        assert_bits_equal(gv.cpu().numpy(), ov, f"values step {step}")
        K, dense, ri, rv = oracle.reduce(np.array(off, np.uint64), oi.ravel(), ov.ravel(), w.N, w.delta)
        out = sg.sparse_reduce(off, gi.reshape(-1), gv.reshape(-1), w.N, w.delta)
        gK, gdense, flags, gri, grv = out.host()
        assert flags == 0 and gK == K and gdense == dense
        if not dense:
            np.testing.assert_array_equal(gri.numpy().astype(np.uint32), ri)
        assert np.max(np.abs(grv.numpy().astype(np.float64) - rv)) <= reduce_tolerance(w.P, ov)
        dense_steps.append(dense)
    assert_bits_equal(rd.cpu().numpy(), r_o, "final residual")
    return dense_steps


def test_pipeline_workload0(dev):
    assert _pipeline(W.workload(0), dev) == [False]


def test_pipeline_resnet20_crosses_dense(dev):
    dense = _pipeline(W.workload(1), dev)
    assert dense[0] is False and dense[-1] is True


def test_pipeline_wideresnet_reduced_n(dev):
    """The wide-ResNet workload (0.5% per node, q4 in buckets of 512, two
    error-feedback steps, delta 0.3) at N = 2^20 so that the oracle keeps up."""
    w = W.workload(4, N=1 << 20)
    _pipeline(w, dev)


def test_pipeline_laplace_reduced_n(dev):
    w = W.workload(2, N=1 << 20, steps=3)
    _pipeline(w, dev)
