"""Pins for the oracle's sparse reduction with the dense switch (CPU only).

SparCML §5.1 (sparse streams, dense past delta), §5.2 (sum, neutral element
0), §5.3 (dense when K >= delta; overlap extremes), §5.3.1 (full overlap
keeps k items) and Appendix B (K is the union size; the union bound is tight
for disjoint sets, which reduces the problem to an allgather).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_sparse(rng, P, N, max_nnz, dup_ok=False):
    idx_parts, val_parts = [], []
    for _ in range(P):
        n = int(rng.integers(0, max_nnz + 1))
        ids = np.sort(rng.choice(N, size=min(n, N), replace=False)).astype(np.uint32)
        idx_parts.append(ids)
        val_parts.append(rng.standard_normal(ids.size).astype(np.float32))
    off = np.zeros(P + 1, np.uint64)
    off[1:] = np.cumsum([a.size for a in idx_parts])
    return off, np.concatenate(idx_parts), np.concatenate(val_parts)


def _check(res, ref, rtol_abs):
    K, dense, oi, ov = res
    bK, bdense, bi, bv = ref
    assert K == bK and dense == bdense
    np.testing.assert_array_equal(oi, bi)
    # oracle rounds an fp64 sum once; bincount sums in fp64 too (possibly in another order)
    np.testing.assert_allclose(ov, bv, rtol=0, atol=rtol_abs)


@pytest.mark.parametrize("seed", range(12))
def test_reduce_matches_bincount_unique(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 9))
    N = int(rng.integers(1, 300))
    off, idx, val = _random_sparse(rng, P, N, max_nnz=N)
    delta = float(rng.choice([0.0, 0.1, 0.25, 0.5, 0.9, 1.0, 1.5]))
    res = oracle.reduce(off, idx, val, N, delta)
    ref = brute.reduce(off, idx, val, N, delta)
    _check(res, ref, 1e-6)


def test_full_overlap_keeps_k_items():
    rng = np.random.default_rng(1)
    P, N, k = 8, 1000, 50
    ids = np.sort(rng.choice(N, k, replace=False)).astype(np.uint32)
    idx = np.tile(ids, P)
    val = rng.standard_normal(P * k).astype(np.float32)
    off = np.arange(P + 1, dtype=np.uint64) * k
    K, dense, oi, ov = oracle.reduce(off, idx, val, N, 0.25)
    assert K == k and not dense
    np.testing.assert_array_equal(oi, ids)
    np.testing.assert_allclose(ov, val.reshape(P, k).astype(np.float64).sum(0), atol=1e-6)


def test_disjoint_sets_reduce_to_allgather():
    rng = np.random.default_rng(2)
    P, N, k = 6, 600, 40
    perm = rng.permutation(N)[: P * k]
    parts = [np.sort(perm[p * k:(p + 1) * k]) for p in range(P)]
    idx = np.concatenate(parts).astype(np.uint32)
    val = rng.standard_normal(P * k).astype(np.float32)
    off = np.arange(P + 1, dtype=np.uint64) * k
    K, dense, oi, ov = oracle.reduce(off, idx, val, N, 0.9)
    assert K == P * k and not dense
    order = np.argsort(idx, kind="stable")
    np.testing.assert_array_equal(oi, idx[order])  # sorted concatenation
    np.testing.assert_array_equal(ov, val[order])  # single contributions: exact


@pytest.mark.parametrize("N,delta", [(1000, 0.25), (999, 0.3), (4096, 0.3), (77, 0.5)])
def test_switch_exactly_at_threshold(N, delta):
    T = math.ceil(delta * N)
    rng = np.random.default_rng(N)
    for K_target, want_dense in [(T - 1, False), (T, True), (T + 1, True)]:
        ids = np.sort(rng.choice(N, K_target, replace=False)).astype(np.uint32)
        # split the union over 3 nodes with some overlap
        a = ids[: 2 * K_target // 3]
        b = ids[K_target // 3:]
        c = ids[::5]
        idx = np.concatenate([a, b, c]).astype(np.uint32)
        val = rng.standard_normal(idx.size).astype(np.float32)
        off = np.array([0, a.size, a.size + b.size, idx.size], np.uint64)
        K, dense, oi, ov = oracle.reduce(off, idx, val, N, delta)
        assert K == K_target
        assert dense == want_dense


def test_delta_edges_and_empty():
    off = np.zeros(4, np.uint64)
    K, dense, oi, ov = oracle.reduce(off, np.zeros(0, np.uint32), np.zeros(0, np.float32), 10, 0.25)
    assert K == 0 and not dense and oi.size == 0
    K, dense, oi, ov = oracle.reduce(off, np.zeros(0, np.uint32), np.zeros(0, np.float32), 10, 0.0)
    assert K == 0 and dense and np.all(ov == 0)
    K, dense, oi, ov = oracle.reduce(off, np.zeros(0, np.uint32), np.zeros(0, np.float32), 10, -1.0)
    assert dense


def test_cancelling_sum_still_counts():
    off = np.array([0, 1, 2], np.uint64)
    idx = np.array([3, 3], np.uint32)
    val = np.array([1.5, -1.5], np.float32)
    K, dense, oi, ov = oracle.reduce(off, idx, val, 8, 0.5)
    assert K == 1 and not dense
    np.testing.assert_array_equal(oi, [3])
    assert ov[0] == 0.0


def test_out_of_range_index_rejected():
    off = np.array([0, 1], np.uint64)
    with pytest.raises(ValueError):
        oracle.reduce(off, np.array([8], np.uint32), np.array([1.0], np.float32), 8, 0.5)


def test_fp64_accumulation_rounds_once():
    # 1 + 2^-24 + 2^-24: sequential fp32 would give 1.0; fp64 gives 1 + 2^-23 exactly
    off = np.array([0, 1, 2, 3], np.uint64)
    idx = np.array([0, 0, 0], np.uint32)
    val = np.array([1.0, 2.0 ** -24, 2.0 ** -24], np.float32)
    K, dense, oi, ov = oracle.reduce(off, idx, val, 4, 0.5)
    assert ov[0] == np.float32(1.0 + 2.0 ** -23)


def test_golden_reduce_hand_examples():
    with open(os.path.join(GOLDEN, "reduce_hand.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    off = np.array(inp["offsets"], np.uint64)
    idx = np.array(inp["idx"], np.uint32)
    val = np.array(inp["val"], np.float32)
    for c in g["cases"]:
        K, dense, oi, ov = oracle.reduce(off, idx, val, inp["N"], c["delta"])
        assert K == c["K"] and dense == c["dense"], c["name"]
        if not dense:
            np.testing.assert_array_equal(oi, c["idx"], err_msg=c["name"])
        np.testing.assert_array_equal(ov, np.array(c["val"], np.float32), err_msg=c["name"])
