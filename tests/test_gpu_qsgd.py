"""GPU parity for the b-bit (2, 4, 8) quantizer, the quantization of a dense
reduction result and the reduction of quantized contributions, against the
oracle: codes, scales and dequantized values bit for bit; reductions with
the same K, dense decision and index list, sums within 1e-6 * P * max|v|."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import assert_bits_equal, reduce_tolerance

pytestmark = pytest.mark.gpu


def _check_qsgd(v, bits, bucket, seed, step, node0, dev):
    n = v.shape[1]
    oc, os_ = oracle.qsgd(v, bits, bucket, seed, step, node0=node0)
    vd = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    gc, gs = sg.qsgd(vd, bits, bucket, seed, step, node0=node0)
    gd = sg.dqsgd(gc, gs, n, bits, bucket)
    torch.cuda.synchronize()
    assert_bits_equal(gs.cpu().numpy(), os_, "scales")
    assert_bits_equal(gc.cpu().numpy(), oc, "codes")
    assert_bits_equal(gd.cpu().numpy(), oracle.dqsgd(oc, os_, n, bits, bucket), "dequantized")


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("P,n,bucket,node0", [
    (1, 1, 8, 0), (3, 7, 8, 5), (2, 13, 8, 0), (4, 1000, 512, 0), (5, 1311, 512, 9), (2, 4097, 64, 0),
    (3, 10485, 1024, 1), (7, 513, 8, 0), (64, 1677, 512, 0),
])
def test_qsgd_shapes(dev, bits, P, n, bucket, node0):
    rng = np.random.default_rng(P * 7919 + n + bucket + bits)
    v = (rng.standard_normal((P, n)) * 1e-3).astype(np.float32)
    print(f"qsgd bits={bits} P={P} n={n} bucket={bucket} node0={node0}", flush=True)
    _check_qsgd(v, bits, bucket, seed=0x0123456789ABCDEF + n, step=n % 7, node0=node0, dev=dev)


@pytest.mark.parametrize("bits", [2, 8])
def test_qsgd_zero_buckets_and_extremes(dev, bits):
    v = np.zeros((2, 1500), np.float32)
    v[0, :512] = np.linspace(-3, 3, 512).astype(np.float32)
    v[1, 7] = -0.0
    v[1, 1000] = 2.0
    _check_qsgd(v, bits, 512, seed=3, step=1, node0=0, dev=dev)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_qsgd_ratio_edge_cases(dev, bits):
    """Buckets whose ratios |v| / scale are hard for the quotient: tiny and
    denormal values beside a normal scale, buckets of denormals only, scales
    near the top of the range, values on and one ulp off every level
    boundary, and random significands over wide exponent ranges."""
    rng = np.random.default_rng(bits)
    B = 512
    rows = []
    r = np.zeros(8 * B, np.float32)
    r[0:B] = np.float32(1.0)
    r[1:B:3] = np.float32(2.0 ** -120)  # ratios below 2^-100 take the division
    r[2:B:3] = np.float32(1e-45)        # smallest denormal
    r[B:2 * B] = (rng.standard_normal(B) * 1e-39).astype(np.float32)  # denormals only
    r[2 * B:3 * B] = (rng.standard_normal(B) * 1e37).astype(np.float32)
    r[2 * B] = np.float32(3.0e38)
    s = (1 << (bits - 1)) - 1
    sc = np.float32(0.7311)
    lv = np.arange(B) % (s + 1)
    on = (np.float64(sc) * lv / s).astype(np.float32)
    r[3 * B:4 * B] = on
    r[3 * B] = sc
    r[4 * B:5 * B] = np.nextafter(on, np.float32(0))
    r[4 * B] = sc
    r[5 * B:6 * B] = np.nextafter(on, np.float32(1))
    r[5 * B] = np.float32(1.0)
    r[6 * B:8 * B] = (rng.standard_normal(2 * B) * np.exp2(rng.integers(-40, 40, 2 * B))).astype(np.float32)
    rows.append(r)
    rows.append(-r)
    v = np.stack(rows)
    print(f"qsgd ratio edges bits={bits}", flush=True)
    for step in range(3):
        _check_qsgd(v, bits, B, seed=0x5EED + step, step=step, node0=3, dev=dev)


def test_q4_is_qsgd_4(dev):
    rng = np.random.default_rng(8)
    v = torch.from_numpy(rng.standard_normal((3, 2049)).astype(np.float32)).to(dev)
    a = sg.q4(v, 512, 77, 2)
    b = sg.qsgd(v, 4, 512, 77, 2)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _ragged_quantized(rng, P, N, nnz_max, bits, bucket, seed, step):
    """Per node: sorted unique indices, N(0,1) values, quantized by the oracle
    as node p; codes and scales concatenated node after node."""
    idx_parts, code_parts, scale_parts, deq_parts = [], [], [], []
    for p in range(P):
        n = int(rng.integers(0, nnz_max + 1))
        ids = np.sort(rng.choice(N, size=min(n, N), replace=False)).astype(np.uint32)
        vals = rng.standard_normal((1, ids.size)).astype(np.float32)
        c, s = oracle.qsgd(vals, bits, bucket, seed, step, node0=p)
        idx_parts.append(ids)
        code_parts.append(c[0])
        scale_parts.append(s[0])
        deq_parts.append(oracle.dqsgd(c, s, ids.size, bits, bucket)[0])
    off = np.zeros(P + 1, np.uint64)
    off[1:] = np.cumsum([a.size for a in idx_parts])
    cat = lambda parts, dt: np.concatenate(parts).astype(dt) if parts else np.zeros(0, dt)
    return off, cat(idx_parts, np.uint32), cat(code_parts, np.uint8), cat(scale_parts, np.float32), \
        cat(deq_parts, np.float32)


def _run_fused(off, idx, codes, scales, bits, bucket, N, delta, dev, hint=0):
    it = torch.from_numpy(idx.view(np.int32)).to(dev)
    ct = torch.from_numpy(codes).to(dev)
    st = torch.from_numpy(scales).to(dev)
    out = sg.sparse_reduce_qsgd([int(x) for x in off], it, ct, st, bits, bucket, N, delta, expected_nnz_hint=hint)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("P,N,nnz,bucket,delta", [
    (1, 100, 30, 8, 0.5), (3, 8191, 501, 8, 0.25), (5, 30000, 4001, 512, 0.25), (8, 30000, 9000, 64, 0.25),
    (16, 100003, 2003, 512, 0.05), (200, 30000, 150, 32, 0.25), (300, 20000, 77, 16, 0.3),
])
def test_reduce_qsgd_matches_oracle(dev, bits, P, N, nnz, bucket, delta):
    rng = np.random.default_rng(P * 31 + N + nnz + bits)
    off, idx, codes, scales, deq = _ragged_quantized(rng, P, N, nnz, bits, bucket, seed=99, step=4)
    print(f"reduce_qsgd bits={bits} P={P} N={N} pairs={idx.size} bucket={bucket} delta={delta}", flush=True)
    K, dense, oi, ov = oracle.reduce(off, idx, deq, N, delta)
    for hint in (0, 1, N):  # both algorithms
        gK, gdense, flags, gi, gv = _run_fused(off, idx, codes, scales, bits, bucket, N, delta, dev, hint).host()
        assert flags == 0 and gK == K and gdense == dense, (gK, K, gdense, dense)
        if not dense:
            np.testing.assert_array_equal(gi.numpy().astype(np.uint32), oi)
        err = np.max(np.abs(gv.numpy().astype(np.float64) - ov)) if ov.size else 0.0
        assert err <= reduce_tolerance(P, deq), err


def test_reduce_qsgd_equals_unfused_wideresnet_shape(dev):
    """wide-ResNet shape (P = 64, N = 2^27, k = 0.5%, 4-bit, buckets of 512):
    fused against the oracle, and bit for bit against sparcml_sparse_reduce
    over the same dequantized values."""
    w = W.workload(4)
    P, N, k = w.P, w.N, w.k
    rng = np.random.default_rng(44)
    idx = np.empty((P, k), np.uint32)
    for p in range(P):
        cand = np.unique(rng.integers(0, N, size=int(k * 1.02)))
        while cand.size < k:
            cand = np.unique(np.concatenate([cand, rng.integers(0, N, size=k)]))
        idx[p] = np.sort(rng.choice(cand, size=k, replace=False))
    vals = (rng.standard_normal((P, k)) * 1e-3).astype(np.float32)
    codes, scales = oracle.qsgd(vals, 4, 512, 1234, 1)
    deq = oracle.dqsgd(codes, scales, k, 4, 512)
    off = np.arange(P + 1, dtype=np.uint64) * k
    K, dense, oi, ov = oracle.reduce(off, idx.reshape(-1), deq.reshape(-1), N, w.delta)
    fused = _run_fused(off, idx.reshape(-1), codes.reshape(-1), scales.reshape(-1), 4, 512, N, w.delta, dev)
    gK, gdense, flags, gi, gv = fused.host()
    assert flags == 0 and gK == K and gdense == dense
    np.testing.assert_array_equal(gi.numpy().astype(np.uint32), oi)
    assert np.max(np.abs(gv.numpy().astype(np.float64) - ov)) <= reduce_tolerance(P, deq)
    it = torch.from_numpy(idx.reshape(-1).view(np.int32)).to(dev)
    plain = sg.sparse_reduce([int(x) for x in off], it, torch.from_numpy(deq.reshape(-1)).to(dev), N, w.delta)
    torch.cuda.synchronize()
    pK, pdense, _, pi, pv = plain.host()
    assert pK == gK and pdense == gdense
    assert torch.equal(pi, gi)
    assert_bits_equal(pv.numpy(), gv.numpy(), "fused vs unfused")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dense_result_quantized_only_when_dense(dev, bits):
    rng = np.random.default_rng(50 + bits)
    P, N = 6, 20000
    parts = [np.sort(rng.choice(N, size=4000, replace=False)).astype(np.uint32) for _ in range(P)]
    idx = np.concatenate(parts)
    val = rng.standard_normal(idx.size).astype(np.float32)
    off = np.arange(P + 1, dtype=np.uint64) * 4000
    it = torch.from_numpy(idx.view(np.int32)).to(dev)
    vt = torch.from_numpy(val).to(dev)
    bucket, seed, step, node = 1024, 0xABCDEF, 3, 2
    nb = (N + bucket - 1) // bucket
    # dense (K ~ 14000 >= T = 5000): codes and scales follow the oracle's quantizer on the dense sum
    out = sg.sparse_reduce([int(x) for x in off], it, vt, N, 0.25)
    codes = torch.full((sg.qsgd_row_bytes(bits, N),), 0xAB, dtype=torch.uint8, device=dev)
    scales = torch.full((nb,), -1.0, dtype=torch.float32, device=dev)
    sg.qsgd_dense_result(out, bits, bucket, seed, step, node, codes=codes, scales=scales)
    torch.cuda.synchronize()
    K, dense, flags = out.read()
    assert dense and flags == 0
    dense_val = out.out_val[:N].cpu().numpy()
    K_o, dense_o, _, ov = oracle.reduce(off, idx, val, N, 0.25)
    assert dense_o and K_o == K
    assert np.max(np.abs(dense_val.astype(np.float64) - ov)) <= reduce_tolerance(P, val)
    oc, os_ = oracle.qsgd(dense_val[None, :], bits, bucket, seed, step, node0=node)
    assert_bits_equal(codes.cpu().numpy(), oc[0], "dense codes")
    assert_bits_equal(scales.cpu().numpy(), os_[0], "dense scales")
    # sparse (K < T = 19000): nothing written
    out2 = sg.sparse_reduce([int(x) for x in off], it, vt, N, 0.95)
    codes2 = torch.full_like(codes, 0xAB)
    scales2 = torch.full_like(scales, -1.0)
    sg.qsgd_dense_result(out2, bits, bucket, seed, step, node, codes=codes2, scales=scales2)
    torch.cuda.synchronize()
    assert not out2.read()[1]
    assert bool((codes2 == 0xAB).all()) and bool((scales2 == -1.0).all())


def test_reduce_qsgd_invalid_input_sets_flags(dev):
    """Descending and out-of-range indices set the flags; the code and scale
    loads stay inside each node's rows even with a run table left over from
    an earlier call in the same workspace."""
    P, N, bits, bucket = 3, 300000, 4, 64
    ws = torch.empty(sg.sparse_reduce_workspace_bytes(P, N, 60000), dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(61)
    off, idx, codes, scales, _ = _ragged_quantized(rng, P, N, 20000, bits, bucket, seed=1, step=0)
    it = torch.from_numpy(idx.view(np.int32)).to(dev)
    out = sg.sparse_reduce_qsgd([int(x) for x in off], it, torch.from_numpy(codes).to(dev),
                                torch.from_numpy(scales).to(dev), bits, bucket, N, 0.25, workspace=ws)
    torch.cuda.synchronize()
    assert out.read()[2] == 0
    parts = [np.array([100000, 50000, 10], np.uint32), np.array([5, N + 3], np.uint32), np.array([7, 8], np.uint32)]
    c_parts, s_parts = [], []
    for p, ids in enumerate(parts):
        c, s = oracle.qsgd(np.ones((1, ids.size), np.float32), bits, bucket, 2, 0, node0=p)
        c_parts.append(c[0])
        s_parts.append(s[0])
    bad_off = [0, 3, 5, 7]
    bad_idx = torch.from_numpy(np.concatenate(parts).view(np.int32)).to(dev)
    bc = torch.from_numpy(np.concatenate(c_parts)).to(dev)
    bs = torch.from_numpy(np.concatenate(s_parts)).to(dev)
    for hint in (1, N):
        out = sg.sparse_reduce_qsgd(bad_off, bad_idx, bc, bs, bits, bucket, N, 0.25, expected_nnz_hint=hint,
                                    workspace=ws)
        torch.cuda.synchronize()
        flags = out.read()[2]
        assert flags & sg.FLAG_NOT_ASCENDING and flags & sg.FLAG_INDEX_RANGE, flags


def test_qsgd_max_nodes(dev):
    rng = np.random.default_rng(15)
    v = rng.standard_normal((65535, 9)).astype(np.float32)
    _check_qsgd(v, 4, 8, seed=5, step=1, node0=0, dev=dev)
