"""Pins for the oracle's per-layer error-feedback Top-k (CPU only).

SparCML §8.4 sparsifies layer by layer; §2.2 and §4 give the selection by
magnitude and the residual. Pinned by a numpy lexsort brute force per layer,
by the one-layer case that is the (separately pinned) whole-vector Top-k, and
by the exact error-feedback identity.
"""
import numpy as np
import pytest

import oracle
from tests import brute


def _layers(rng, N, nl):
    cuts = np.sort(rng.choice(np.arange(1, N), size=nl - 1, replace=False)) if nl > 1 else np.zeros(0, int)
    return np.concatenate([[0], cuts, [N]]).astype(np.uint64)


@pytest.mark.parametrize("P,N,nl", [(1, 1, 1), (2, 50, 3), (3, 700, 7), (2, 5000, 12), (4, 999, 40)])
def test_layers_match_brute_force(P, N, nl):
    rng = np.random.default_rng(P * 100 + N + nl)
    off = _layers(rng, N, nl)
    sizes = np.diff(off.astype(np.int64))
    ks = np.array([rng.integers(0, s + 1) for s in sizes], np.uint64)
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.3).astype(np.float32)
    oi, ov, orr = oracle.topk_ef_layers(g, r, off, ks)
    bi, bv, br = brute.topk_ef_layers(g, r, off, ks)
    np.testing.assert_array_equal(oi, bi)
    np.testing.assert_array_equal(ov.view(np.uint32), bv.view(np.uint32))
    np.testing.assert_array_equal(orr.view(np.uint32), br.view(np.uint32))


def test_empty_layers_and_ties():
    g = np.full((2, 300), 0.5, np.float32)
    g[1, ::3] = -0.5
    off = np.array([0, 0, 100, 100, 300], np.uint64)  # two empty layers
    ks = np.array([0, 10, 0, 7], np.uint64)
    oi, _, _ = oracle.topk_ef_layers(g, np.zeros_like(g), off, ks)
    want = np.concatenate([np.arange(0, 10), np.arange(100, 107)])
    np.testing.assert_array_equal(oi[0], want)
    np.testing.assert_array_equal(oi[1], want)


@pytest.mark.parametrize("N,k", [(100, 7), (4096, 40), (777, 0), (50, 50)])
def test_one_layer_is_whole_vector_topk(N, k):
    rng = np.random.default_rng(N + k)
    g = rng.standard_normal((3, N)).astype(np.float32)
    r = rng.standard_normal((3, N)).astype(np.float32)
    li, lv, lr = oracle.topk_ef_layers(g, r, [0, N], [k])
    ti, tv, tr = oracle.topk_ef(g, r, k)
    np.testing.assert_array_equal(li, ti)
    np.testing.assert_array_equal(lv.view(np.uint32), tv.view(np.uint32))
    np.testing.assert_array_equal(lr.view(np.uint32), tr.view(np.uint32))


def test_ef_identity_and_counts():
    rng = np.random.default_rng(9)
    P, N = 3, 20000
    off = np.array([0, 100, 5100, 5164, 20000], np.uint64)
    ks = np.array([1, 50, 64, 150], np.uint64)
    g = rng.laplace(0, 1e-3, (P, N)).astype(np.float32)
    r = rng.laplace(0, 1e-3, (P, N)).astype(np.float32)
    oi, ov, orr = oracle.topk_ef_layers(g, r, off, ks)
    assert oi.shape == (P, int(ks.sum()))
    recon = orr.copy()
    for p in range(P):
        assert np.all(np.diff(oi[p].astype(np.int64)) > 0)
        for l in range(4):
            assert np.sum((oi[p] >= off[l]) & (oi[p] < off[l + 1])) == ks[l]
        recon[p, oi[p]] += ov[p]
    assert np.array_equal(recon, (g + r).astype(np.float32))
