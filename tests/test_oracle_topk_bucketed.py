"""Pins for the oracle's bucketed error-feedback Top-k (CPU only).

SparCML §8.3 keeps k entries out of every 512 (16/512, 8/512); §2.2 and §4
give the selection by magnitude and the residual. Pinned by a numpy lexsort
brute force per bucket, by the one-bucket case that is the (separately
pinned) whole-vector Top-k, and by the exact error-feedback identity.
"""
import numpy as np
import pytest

import oracle
from tests import brute


@pytest.mark.parametrize("P,N,bucket,kb", [
    (1, 1, 64, 1), (2, 64, 64, 3), (3, 100, 64, 5), (2, 1000, 128, 16), (4, 513, 512, 16), (2, 777, 256, 0),
    (3, 300, 64, 64), (2, 300, 64, 70), (5, 2048, 1024, 33),
])
def test_bucketed_matches_brute_force(P, N, bucket, kb):
    rng = np.random.default_rng(P * 1000 + N + bucket + kb)
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.3).astype(np.float32)
    oi, ov, orr = oracle.topk_ef_bucketed(g, r, bucket, kb)
    bi, bv, br = brute.topk_ef_bucketed(g, r, bucket, kb)
    assert oi.shape == (P, oracle.bucketed_count(N, bucket, kb))
    np.testing.assert_array_equal(oi, bi)
    np.testing.assert_array_equal(ov.view(np.uint32), bv.view(np.uint32))
    np.testing.assert_array_equal(orr.view(np.uint32), br.view(np.uint32))


def test_bucketed_ties_take_lowest_indices():
    g = np.full((2, 256), 0.5, np.float32)
    g[1, ::2] = -0.5
    oi, _, _ = oracle.topk_ef_bucketed(g, np.zeros_like(g), 64, 10)
    want = np.concatenate([np.arange(lo, lo + 10) for lo in range(0, 256, 64)])
    np.testing.assert_array_equal(oi[0], want)
    np.testing.assert_array_equal(oi[1], want)


@pytest.mark.parametrize("N,kb", [(100, 7), (4096, 40), (777, 777)])
def test_one_bucket_is_whole_vector_topk(N, kb):
    rng = np.random.default_rng(N)
    g = rng.standard_normal((3, N)).astype(np.float32)
    r = rng.standard_normal((3, N)).astype(np.float32)
    bi, bv, br = oracle.topk_ef_bucketed(g, r, 1 << 20, kb)
    ti, tv, tr = oracle.topk_ef(g, r, min(kb, N))
    np.testing.assert_array_equal(bi, ti)
    np.testing.assert_array_equal(bv.view(np.uint32), tv.view(np.uint32))
    np.testing.assert_array_equal(br.view(np.uint32), tr.view(np.uint32))


def test_counts_and_ef_identity():
    rng = np.random.default_rng(3)
    P, N, bucket, kb = 3, 5000, 512, 16
    g = rng.laplace(0, 1e-3, (P, N)).astype(np.float32)
    r = rng.laplace(0, 1e-3, (P, N)).astype(np.float32)
    oi, ov, orr = oracle.topk_ef_bucketed(g, r, bucket, kb)
    assert oracle.bucketed_count(N, bucket, kb) == 9 * 16 + min(16, 5000 - 9 * 512)
    assert oracle.bucketed_count(0, bucket, kb) == 0
    assert oracle.bucketed_count(130, 64, 100) == 130  # every position of every bucket
    a = (g + r).astype(np.float32)
    recon = orr.copy()
    for p in range(P):
        assert np.all(np.diff(oi[p].astype(np.int64)) > 0)
        recon[p, oi[p]] += ov[p]
        for lo in range(0, N, bucket):  # per bucket: exactly min(kb, len) kept
            assert np.sum((oi[p] >= lo) & (oi[p] < lo + bucket)) == min(kb, N - lo)
    assert np.array_equal(recon, a)
