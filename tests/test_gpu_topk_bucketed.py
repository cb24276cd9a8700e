"""GPU parity: sparcml_topk_ef_bucketed against the oracle, bit for bit
(index rows, values, residual), over every supported bucket size, partial
buckets, ties, k at and beyond the bucket size, and the wide-ResNet-sized
gradient with 16 of every 512 kept."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import assert_bits_equal

pytestmark = pytest.mark.gpu


def _run(g, r, bucket, kb, dev):
    gd = torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(dev)
    rd = torch.from_numpy(np.ascontiguousarray(r, np.float32)).to(dev)
    idx, val = sg.topk_ef_bucketed(gd, rd, bucket, kb)
    torch.cuda.synchronize()
    return idx.cpu().numpy().view(np.uint32), val.cpu().numpy(), rd.cpu().numpy()


def _check(g, r, bucket, kb, dev):
    oi, ov, orr = oracle.topk_ef_bucketed(g, r, bucket, kb)
    gi, gv, grr = _run(g, r, bucket, kb, dev)
    assert gi.shape == oi.shape
    assert_bits_equal(gi, oi, "idx")
    assert_bits_equal(gv, ov, "val")
    assert_bits_equal(grr, orr, "residual")


@pytest.mark.parametrize("bucket", [64, 128, 256, 512, 1024])
@pytest.mark.parametrize("P,N,kb", [(1, 1, 1), (2, 100, 3), (3, 5000, 16), (2, 4097, 8), (4, 3333, 0),
                                    (2, 2500, 5000), (5, 65536, 16)])
def test_bucketed_shapes(dev, bucket, P, N, kb):
    rng = np.random.default_rng(P * 100003 + N + bucket + kb)
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.5).astype(np.float32)
    print(f"bucketed P={P} N={N} bucket={bucket} kb={kb}", flush=True)
    _check(g, r, bucket, kb, dev)


@pytest.mark.parametrize("bucket", [64, 128, 512])
def test_bucketed_ties_zeros_and_subnormals(dev, bucket):
    rng = np.random.default_rng(bucket)
    P, N = 4, 6000
    g = (rng.integers(-3, 4, size=(P, N)) * 0.25).astype(np.float32)  # heavy ties
    g[1] = 0.0                                                          # all zero: lowest indices
    g[2] = (rng.integers(-4, 5, size=N) * np.float32(1e-45)).astype(np.float32)
    g[2, ::7] = -0.0
    r = np.zeros_like(g)
    _check(g, r, bucket, 16, dev)
    _check(g, r, bucket, 63, dev)


def test_bucketed_error_feedback_steps(dev):
    """Five steps with the residual carried on the device."""
    rng = np.random.default_rng(77)
    P, N, bucket, kb = 3, 20000, 512, 16
    rd = torch.zeros((P, N), dtype=torch.float32, device=dev)
    r_o = np.zeros((P, N), np.float32)
    for step in range(5):
        g = rng.laplace(0, 1e-3, (P, N)).astype(np.float32)
        oi, ov, r_o = oracle.topk_ef_bucketed(g, r_o, bucket, kb)
        gi, gv = sg.topk_ef_bucketed(torch.from_numpy(g).to(dev), rd, bucket, kb)
        torch.cuda.synchronize()
        assert_bits_equal(gi.cpu().numpy().view(np.uint32), oi, f"idx step {step}")
        assert_bits_equal(gv.cpu().numpy(), ov, f"val step {step}")
        assert_bits_equal(rd.cpu().numpy(), r_o, f"residual step {step}")


@pytest.mark.parametrize("bucket,kb", [(512, 16), (128, 4), (64, 2)])
def test_bucketed_wideresnet_size_sampled_nodes(dev, bucket, kb):
    """P = 64, N = 2^27, one in 32 kept: oracle on two nodes, properties on all."""
    w = W.workload(4)
    P, N = w.P, w.N
    print(f"bucketed wide-ResNet size bucket={bucket} kb={kb}", flush=True)
    g = W.gradients(w, 0, device=dev)
    r = torch.zeros_like(g)
    idx, val = sg.topk_ef_bucketed(g, r, bucket, kb)
    torch.cuda.synchronize()
    K = sg.topk_bucketed_count(N, bucket, kb)
    assert idx.shape == (P, K) and K == N // bucket * kb
    for p in (0, P - 1):
        gp = g[p:p + 1].cpu().numpy()
        oi, ov, orr = oracle.topk_ef_bucketed(gp, np.zeros_like(gp), bucket, kb)
        assert_bits_equal(idx[p:p + 1].cpu().numpy().view(np.uint32), oi, f"idx node {p}")
        assert_bits_equal(val[p:p + 1].cpu().numpy(), ov, f"val node {p}")
        assert_bits_equal(r[p:p + 1].cpu().numpy(), orr, f"residual node {p}")
    il = idx.to(torch.int64) & 0xFFFFFFFF
    assert bool((il[:, 1:] > il[:, :-1]).all())
    assert bool(((il // bucket).view(P, -1, kb) == torch.arange(N // bucket, device=dev).view(1, -1, 1)).all())
    recon = r.clone()
    recon.scatter_add_(1, il, val)
    assert torch.equal(recon, g)
