"""GPU parity: sparcml_q4 / sparcml_dq4 against the oracle, bit for bit
(codes from the same Philox-4x32-10 stream, scales, dequantized values)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from tests.gpu_util import assert_bits_equal

pytestmark = pytest.mark.gpu


def _check(v, bucket, seed, step, dev):
    n = v.shape[1]
    oc, os_ = oracle.q4(v, bucket, seed, step)
    vd = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    gc, gs = sg.q4(vd, bucket, seed, step)
    gd = sg.dq4(gc, gs, n, bucket)
    torch.cuda.synchronize()
    assert_bits_equal(gs.cpu().numpy(), os_, "scales")
    assert_bits_equal(gc.cpu().numpy(), oc, "codes")
    od = oracle.dq4(oc, os_, n, bucket)
    assert_bits_equal(gd.cpu().numpy(), od, "dq4")


@pytest.mark.parametrize("P,n,bucket", [
    (1, 1, 8), (3, 7, 8), (2, 512, 512), (4, 1000, 512), (5, 1311, 512), (2, 4097, 64),
    (3, 10485, 512), (2, 3000, 1024), (1, 10000, 2048), (7, 513, 8), (64, 1677, 512),
])
def test_q4_shapes(dev, P, n, bucket):
    rng = np.random.default_rng(P * 7919 + n + bucket)
    v = (rng.standard_normal((P, n)) * 1e-3).astype(np.float32)
    print(f"q4 P={P} n={n} bucket={bucket}", flush=True)
    _check(v, bucket, seed=0xDEADBEEF12345678 + n, step=n % 5, dev=dev)


def test_q4_zero_buckets_and_extremes(dev):
    v = np.zeros((3, 2000), np.float32)
    v[0, :512] = np.linspace(-3, 3, 512).astype(np.float32)
    v[1, 7] = -0.0
    v[1, 600] = 5.0
    v[2, :] = -1.0  # every value at the scale
    _check(v, 512, seed=77, step=0, dev=dev)


def test_q4_laplace_values(dev):
    rng = np.random.default_rng(3)
    v = rng.laplace(0, 1e-3, size=(16, 20000)).astype(np.float32)
    for step in range(3):
        _check(v, 512, seed=2 ** 63 + 11, step=step, dev=dev)


def test_q4_wideresnet_full_size(dev):
    """All 64 nodes of 671088 sent values in buckets of 512 (the wide-ResNet
    workload's quantizer) against the oracle, every code."""
    P, n = 64, 671088
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    vd = torch.randn((P, n), generator=g, device=dev) * 1e-3
    codes, scales = sg.q4(vd, 512, 987654321, 1)
    torch.cuda.synchronize()
    v = vd.cpu().numpy()
    oc, os_ = oracle.q4(v, 512, 987654321, 1)
    assert_bits_equal(scales.cpu().numpy(), os_, "scales")
    assert_bits_equal(codes.cpu().numpy(), oc, "codes")
