"""GPU parity: sparcml_sparse_reduce against the oracle. Union size K, the
dense decision and the index list must match exactly; sums within
1e-6 * P * max|v| (the oracle sums in fp64 and rounds once; so does the GPU,
in another order)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import reduce_tolerance

pytestmark = pytest.mark.gpu


def _gpu_reduce(off, idx, val, N, delta, dev, hint=0):
    it = torch.from_numpy(np.ascontiguousarray(idx, np.uint32).view(np.int32)).to(dev)
    vt = torch.from_numpy(np.ascontiguousarray(val, np.float32)).to(dev)
    out = sg.sparse_reduce([int(x) for x in off], it, vt, N, delta, expected_nnz_hint=hint)
    torch.cuda.synchronize()
    return out.host()


def _check(off, idx, val, N, delta, dev, hint=0, P=None):
    P = P if P is not None else len(off) - 1
    K, dense, oi, ov = oracle.reduce(off, idx, val, N, delta)
    gK, gdense, flags, gi, gv = _gpu_reduce(off, idx, val, N, delta, dev, hint)
    assert flags == 0
    assert gK == K and gdense == dense, (gK, K, gdense, dense)
    gv = gv.numpy()
    if not dense:
        np.testing.assert_array_equal(gi.numpy().astype(np.uint32), oi)
    tol = reduce_tolerance(P, val)
    err = np.max(np.abs(gv.astype(np.float64) - ov)) if ov.size else 0.0
    assert err <= tol, (err, tol)
    return K, dense


def _random_sparse(rng, P, N, nnz_max):
    parts, vals = [], []
    for _ in range(P):
        n = int(rng.integers(0, nnz_max + 1))
        ids = np.sort(rng.choice(N, size=min(n, N), replace=False)).astype(np.uint32)
        parts.append(ids)
        vals.append(rng.standard_normal(ids.size).astype(np.float32))
    off = np.zeros(P + 1, np.uint64)
    off[1:] = np.cumsum([a.size for a in parts])
    return off, np.concatenate(parts), np.concatenate(vals)


@pytest.mark.parametrize("P,N,nnz,delta", [
    (1, 1, 1, 0.25), (1, 100, 30, 0.5), (3, 8191, 500, 0.25), (4, 8192, 3000, 0.25),
    (5, 8193, 2000, 0.3), (8, 30000, 4000, 0.25), (8, 30000, 9000, 0.25), (16, 100003, 2000, 0.05),
    (2, 1 << 20, 5000, 0.3), (64, 65536, 800, 0.25), (65, 70001, 700, 0.25), (200, 70000, 300, 0.25),
    (256, 40000, 100, 0.3), (257, 20000, 60, 0.3),
])
@pytest.mark.parametrize("hint", ["estimate", "count_first", "dense_first"])
def test_reduce_random(dev, P, N, nnz, delta, hint):
    rng = np.random.default_rng(P * 31 + N + nnz)
    off, idx, val = _random_sparse(rng, P, N, nnz)
    h = {"estimate": 0, "count_first": 1, "dense_first": N}[hint]
    print(f"reduce P={P} N={N} nnz<={nnz} delta={delta} hint={hint}", flush=True)
    _check(off, idx, val, N, delta, dev, hint=h)


@pytest.mark.parametrize("N,delta", [(100000, 0.25), (99999, 0.3), (65536, 0.3), (10007, 0.5)])
@pytest.mark.parametrize("hint", ["count_first", "dense_first"])
def test_switch_exactly_at_threshold(dev, N, delta, hint):
    T = math.ceil(delta * N)
    rng = np.random.default_rng(N)
    for K_target, want_dense in [(T - 1, False), (T, True), (T + 1, True)]:
        ids = np.sort(rng.choice(N, K_target, replace=False)).astype(np.uint32)
        a, b, c = ids[: 2 * K_target // 3], ids[K_target // 3:], ids[::5]
        idx = np.concatenate([a, b, c]).astype(np.uint32)
        val = rng.standard_normal(idx.size).astype(np.float32)
        off = np.array([0, a.size, a.size + b.size, idx.size], np.uint64)
        K, dense = _check(off, idx, val, N, delta, dev, hint={"count_first": 1, "dense_first": N}[hint])
        assert K == K_target and dense == want_dense


def test_full_overlap_and_disjoint(dev):
    rng = np.random.default_rng(8)
    P, N, k = 16, 200000, 3000
    ids = np.sort(rng.choice(N, k, replace=False)).astype(np.uint32)
    idx = np.tile(ids, P)
    val = rng.standard_normal(P * k).astype(np.float32)
    off = np.arange(P + 1, dtype=np.uint64) * k
    K, dense = _check(off, idx, val, N, 0.25, dev)
    assert K == k
    perm = rng.permutation(N)[: P * k]
    idx = np.concatenate([np.sort(perm[p * k:(p + 1) * k]) for p in range(P)]).astype(np.uint32)
    K, dense = _check(off, idx, val, N, 0.5, dev)
    assert K == P * k


def test_empty_and_edge_delta(dev):
    off = np.zeros(5, np.uint64)
    e_i, e_v = np.zeros(0, np.uint32), np.zeros(0, np.float32)
    assert _check(off, e_i, e_v, 50000, 0.25, dev) == (0, False)
    assert _check(off, e_i, e_v, 50000, 0.0, dev) == (0, True)
    rng = np.random.default_rng(1)
    off, idx, val = _random_sparse(rng, 3, 20000, 5000)
    _check(off, idx, val, 20000, -2.0, dev)   # always dense
    _check(off, idx, val, 20000, 7.0, dev)    # never dense


def test_segment_boundary_indices(dev):
    N = 3 * 8192 + 5
    idx = np.array([0, 8191, 8192, 16383, 16384, 24575, 24576, N - 1], np.uint32)
    val = np.arange(1, 9, dtype=np.float32)
    off = np.array([0, 4, 8, 8], np.uint64)
    idx2 = np.concatenate([idx[:4], idx[::2]])
    val2 = np.concatenate([val[:4], val[::2]])
    off2 = np.array([0, 4, 8], np.uint64)
    _check(off, idx, val, N, 0.5, dev)
    _check(off2, idx2, val2, N, 0.5, dev)
    _check(off2, idx2, val2, N, 0.0001, dev)


def test_segment_boundary_indices_4096(dev):
    """Indices on both sides of every 4096-index segment edge, from several
    nodes, with a ragged last segment."""
    N = 5 * 4096 + 77
    edges = [0, 4095, 4096, 8191, 8192, 12287, 12288, 16383, 16384, 20479, 20480, N - 1]
    idx = np.array(edges, np.uint32)
    parts = [idx, idx[1::2], idx[::3], np.zeros(0, np.uint32), idx[-2:]]
    off = np.zeros(len(parts) + 1, np.uint64)
    off[1:] = np.cumsum([a.size for a in parts])
    cat = np.concatenate(parts)
    val = np.arange(1, cat.size + 1, dtype=np.float32)
    _check(off, cat, val, N, 0.5, dev)
    _check(off, cat, val, N, 0.0001, dev)


def test_many_segments_scan_rounds(dev):
    """More than 32768 segments (the count scan takes two rounds, the second
    ragged) in both the sparse and the dense result."""
    N = 4096 * 40001 + 123
    rng = np.random.default_rng(21)
    off, idx, val = _random_sparse(rng, 3, N, 60000)
    idx[-1] = N - 1 if idx.size and off[-1] - off[-2] > 0 and idx[-1] < N - 1 else idx[-1]
    _check(off, idx, val, N, 0.25, dev)
    _check(off, idx, val, N, 0.0, dev)


def test_max_nodes(dev):
    rng = np.random.default_rng(2)
    off, idx, val = _random_sparse(rng, 1024, 50000, 40)
    _check(off, idx, val, 50000, 0.25, dev)
    _check(off, idx, val, 50000, 0.25, dev, hint=50000)


def test_invalid_input_sets_flags(dev):
    N = 10000
    # node 0 not ascending, node 1 has an index >= N
    idx = np.array([5, 3, 9, 1, 2, N + 7], np.uint32)
    val = np.ones(6, np.float32)
    off = [0, 3, 6]
    for hint in (1, N):
        _, _, flags, _, _ = _gpu_reduce(off, idx, val, N, 0.25, dev, hint)
        assert flags & sg.FLAG_NOT_ASCENDING
        assert flags & sg.FLAG_INDEX_RANGE
    # a valid call afterwards with the same workspace size is clean
    _, _, flags, _, _ = _gpu_reduce([0, 2], np.array([1, 4], np.uint32), np.ones(2, np.float32), N, 0.25, dev)
    assert flags == 0


def test_zipf_workload_full_size(dev):
    """Already-sparse URL-style input: N = 2^22, P = 32, 65536 Zipf(1.1) indices per node."""
    w = W.workload(3)
    off, idx, val = W.zipf_sparse(w)
    K, dense = _check(off, idx, val, w.N, w.delta, dev)
    assert not dense and 0.1 * w.N < K < 0.3 * w.N


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_unaligned_index_array(dev, shift):
    """Pair arrays that start 4, 8 or 12 bytes past a 16-byte boundary (views
    into a larger buffer): the bounds pass reads indices in aligned quads, with
    partial quads at both ends of the array and at node edges."""
    rng = np.random.default_rng(40 + shift)
    N, delta = 70001, 0.25
    off, idx, val = _random_sparse(rng, 7, N, 9000)
    K, dense, oi, ov = oracle.reduce(off, idx, val, N, delta)
    n = idx.size
    bi = torch.zeros(n + 8, dtype=torch.int32, device=dev)
    bv = torch.zeros(n + 8, dtype=torch.float32, device=dev)
    bi[shift:shift + n] = torch.from_numpy(idx.view(np.int32)).to(dev)
    bv[shift:shift + n] = torch.from_numpy(val).to(dev)
    it, vt = bi[shift:shift + n], bv[shift:shift + n]
    assert it.data_ptr() % 16 == 4 * shift
    for hint in (1, N):
        gK, gdense, flags, gi, gv = sg.sparse_reduce([int(x) for x in off], it, vt, N, delta,
                                                     expected_nnz_hint=hint).host()
        assert flags == 0 and gK == K and gdense == dense
        if not dense:
            np.testing.assert_array_equal(gi.numpy().astype(np.uint32), oi)
        assert np.max(np.abs(gv.numpy().astype(np.float64) - ov)) <= reduce_tolerance(7, val)


def test_wideresnet_size_dense_result(dev):
    """Full wide-ResNet size (P = 64, N = 2^27, 671088 pairs per node) with
    delta = 0.25, where the union (about 0.274 N) passes T: the dense result
    of both the dense-first and the count-first path against the oracle."""
    w = W.workload(4)
    P, N, k, delta = w.P, w.N, w.k, 0.25
    rng = np.random.default_rng(45)
    idx = np.empty((P, k), np.uint32)
    for p in range(P):
        cand = np.unique(rng.integers(0, N, size=int(k * 1.02)))
        while cand.size < k:
            cand = np.unique(np.concatenate([cand, rng.integers(0, N, size=k)]))
        idx[p] = np.sort(rng.choice(cand, size=k, replace=False))
    val = (rng.standard_normal((P, k)) * 1e-3).astype(np.float32)
    off = np.arange(P + 1, dtype=np.uint64) * k
    K, dense, _, ov = oracle.reduce(off, idx.reshape(-1), val.reshape(-1), N, delta)
    assert dense and K >= sg.dense_threshold(delta, N)
    tol = reduce_tolerance(P, val)
    for hint in (0, 1):  # the estimate (dense-first here), then count-first
        print(f"wide-ResNet dense result hint={hint}", flush=True)
        gK, gdense, flags, _, gv = _gpu_reduce(off, idx.reshape(-1), val.reshape(-1), N, delta, dev, hint)
        assert flags == 0 and gK == K and gdense
        assert np.max(np.abs(gv.numpy().astype(np.float64) - ov)) <= tol


def test_reduce_deterministic(dev):
    rng = np.random.default_rng(21)
    off, idx, val = _random_sparse(rng, 32, 1 << 18, 20000)
    a = _gpu_reduce(off, idx, val, 1 << 18, 0.25, dev)
    b = _gpu_reduce(off, idx, val, 1 << 18, 0.25, dev)
    assert a[0] == b[0]
    assert torch.equal(a[3], b[3])
    assert torch.equal(a[4].view(torch.int32), b[4].view(torch.int32))


def _sparse_sorted(rng, P, N, nnz):
    """P nodes of nnz sorted distinct indices below N (drawn with repeats,
    deduplicated, topped up), N(0,1) values."""
    parts = []
    for _ in range(P):
        cand = np.unique(rng.integers(0, N, size=int(nnz * 1.05) + 8))
        while cand.size < nnz:
            cand = np.unique(np.concatenate([cand, rng.integers(0, N, size=nnz)]))
        parts.append(np.sort(rng.choice(cand, size=nnz, replace=False)).astype(np.uint32))
    off = np.arange(P + 1, dtype=np.uint64) * nnz
    return off, np.concatenate(parts), rng.standard_normal(P * nnz).astype(np.float32)


@pytest.mark.parametrize("P,N,nnz", [
    (64, 1 << 24, 16384),   # 4096 segments of 256 pairs: writer groups of 4, count groups of 8; writers scan
    (8, 1 << 26, 262144),   # 16384 segments of 128 pairs: 4096 writer groups, the decide pass scans
    (3, 1 << 25, 700000),   # long runs of few nodes (about 340 pairs per group): groups of 4 for both
    (300, 1 << 24, 3000),   # more than 256 nodes (run tables for 1024) in writer groups of 4
    (5, 1 << 26, 300),      # very sparse: consecutive indices of a node about 54 segments apart
    (64, (1 << 24) + 5 * 4096 + 7, 16384),  # ragged ends: last writer group 2 of 4 segments, last count
                                            # group 6 of 8, last segment 7 indices
])
@pytest.mark.parametrize("delta", [0.3, 0.01])
def test_multi_segment_groups(dev, P, N, nnz, delta):
    """Few pairs per 4096-index segment: the count pass takes groups of
    several segments and the rank-order writer groups of up to four, whose
    union ranks span the group. Both thresholds (at delta = 0.01 the result
    is dense but for the very sparse case), each result written by both
    writers (hint 1: rank order, N: the tile)."""
    rng = np.random.default_rng(P + nnz)
    off, idx, val = _sparse_sorted(rng, P, N, nnz)
    print(f"multi-segment P={P} N={N} nnz={nnz} delta={delta}", flush=True)
    for hint in (1, N):
        _check(off, idx, val, N, delta, dev, hint=hint)


@pytest.mark.parametrize("bits", [4, 8])
def test_multi_segment_groups_quantized(dev, bits):
    """The same grouping with 4- and 8-bit codes dequantized on load (pairs
    one per lane), against the oracle on the dequantized values."""
    rng = np.random.default_rng(60 + bits)
    P, N, nnz, bucket = 64, 1 << 24, 16384, 512
    off, idx, val = _sparse_sorted(rng, P, N, nnz)
    codes, scales = oracle.qsgd(val.reshape(P, nnz), bits, bucket, 77, 2)
    deq = oracle.dqsgd(codes, scales, nnz, bits, bucket).reshape(-1)
    K, dense, oi, ov = oracle.reduce(off, idx, deq, N, 0.3)
    out = sg.sparse_reduce_qsgd([int(x) for x in off], torch.from_numpy(idx.view(np.int32)).to(dev),
                                torch.from_numpy(codes.reshape(-1)).to(dev),
                                torch.from_numpy(scales.reshape(-1)).to(dev), bits, bucket, N, 0.3,
                                expected_nnz_hint=1)
    torch.cuda.synchronize()
    gK, gdense, flags, gi, gv = out.host()
    assert flags == 0 and gK == K and gdense == dense and not dense
    np.testing.assert_array_equal(gi.numpy().astype(np.uint32), oi)
    assert np.max(np.abs(gv.numpy().astype(np.float64) - ov)) <= reduce_tolerance(P, deq)


def test_multi_segment_groups_unaligned(dev):
    """Writer groups of four segments over pair arrays 8 bytes past a 16-byte
    boundary (pairs one per lane in the writer, partial quads in the bounds
    pass)."""
    rng = np.random.default_rng(61)
    P, N, nnz = 64, 1 << 24, 16384
    off, idx, val = _sparse_sorted(rng, P, N, nnz)
    K, dense, oi, ov = oracle.reduce(off, idx, val, N, 0.3)
    n = idx.size
    bi = torch.zeros(n + 8, dtype=torch.int32, device=dev)
    bv = torch.zeros(n + 8, dtype=torch.float32, device=dev)
    bi[2:2 + n] = torch.from_numpy(idx.view(np.int32)).to(dev)
    bv[2:2 + n] = torch.from_numpy(val).to(dev)
    gK, gdense, flags, gi, gv = sg.sparse_reduce([int(x) for x in off], bi[2:2 + n], bv[2:2 + n], N, 0.3,
                                                 expected_nnz_hint=1).host()
    assert flags == 0 and gK == K and gdense == dense and not dense
    np.testing.assert_array_equal(gi.numpy().astype(np.uint32), oi)
    assert np.max(np.abs(gv.numpy().astype(np.float64) - ov)) <= reduce_tolerance(P, val)


@pytest.mark.parametrize("hint", [0, 1])
def test_clustered_indices_take_several_rank_windows(dev, hint):
    """Indices crowded into the first few segments while the uniform estimate
    expects about 64 per segment: the rank writer sized by the estimate (the
    smaller slot count) meets unions of about 4000 per segment and takes
    several windows over the group's pairs."""
    rng = np.random.default_rng(77 + hint)
    P, N = 8, 1 << 22
    parts, vals = [], []
    for _ in range(P):
        ids = np.sort(rng.choice(4 * 4096, size=8192, replace=False)).astype(np.uint32)
        parts.append(ids)
        vals.append(rng.standard_normal(ids.size).astype(np.float32))
    off = np.arange(P + 1, dtype=np.uint64) * 8192
    K, dense = _check(off, np.concatenate(parts), np.concatenate(vals), N, 0.25, dev, hint=hint)
    assert not dense and K > 3 * 4096
