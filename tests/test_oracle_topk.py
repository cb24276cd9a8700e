"""Pins for the oracle's error-feedback Top-k (CPU only).

SparCML §2.2 (Top-k with residual accumulation) and §4 (residual carried
forward): the oracle is checked against numpy brute force, the pairwise
characterisation of the selected set, closed-form special cases and the exact
error-feedback identity.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, P, N, kind):
    if kind == "normal":
        return rng.standard_normal((P, N)).astype(np.float32)
    if kind == "ties":  # few distinct magnitudes, both signs, many ties
        return (rng.integers(-3, 4, size=(P, N)) * 0.5).astype(np.float32)
    if kind == "tiny":  # subnormals and zeros of both signs
        v = rng.integers(-4, 5, size=(P, N)).astype(np.float32) * np.float32(1e-45)
        v[rng.random((P, N)) < 0.2] = -0.0
        return v
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "ties", "tiny"])
@pytest.mark.parametrize("N", [1, 2, 7, 33, 64])
def test_topk_matches_bruteforce_all_k(kind, N):
    rng = np.random.default_rng(N * 31 + len(kind))
    P = 3
    g = _rand(rng, P, N, kind)
    r = _rand(rng, P, N, kind)
    for k in range(0, N + 1):
        oi, ov, orr = oracle.topk_ef(g, r, k)
        bi, bv, br = brute.topk_ef(g, r, k)
        np.testing.assert_array_equal(oi, bi)
        np.testing.assert_array_equal(ov.view(np.uint32), bv.view(np.uint32))
        np.testing.assert_array_equal(orr.view(np.uint32), br.view(np.uint32))


@pytest.mark.parametrize("seed", range(6))
def test_topk_characterisation(seed):
    rng = np.random.default_rng(seed)
    P, N = 5, 48
    g = _rand(rng, P, N, "ties" if seed % 2 else "normal")
    r = _rand(rng, P, N, "normal")
    k = int(rng.integers(0, N + 1))
    oi, ov, orr = oracle.topk_ef(g, r, k)
    a = (g + r).astype(np.float32)
    for p in range(P):
        assert brute.characterise(a[p], oi[p], k)
        assert np.all(np.diff(oi[p].astype(np.int64)) > 0)


def test_all_equal_keys_take_lowest_indices():
    P, N, k = 2, 50, 17
    g = np.full((P, N), 0.75, np.float32)
    g[1, ::2] = -0.75  # same magnitude, mixed sign
    r = np.zeros_like(g)
    oi, ov, orr = oracle.topk_ef(g, r, k)
    for p in range(P):
        np.testing.assert_array_equal(oi[p], np.arange(k))
        np.testing.assert_array_equal(ov[p], g[p, :k])


def test_k_zero_and_k_n():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((3, 40)).astype(np.float32)
    r = rng.standard_normal((3, 40)).astype(np.float32)
    a = (g + r).astype(np.float32)
    oi, ov, orr = oracle.topk_ef(g, r, 0)
    assert oi.shape == (3, 0)
    np.testing.assert_array_equal(orr.view(np.uint32), a.view(np.uint32))
    oi, ov, orr = oracle.topk_ef(g, r, 40)
    np.testing.assert_array_equal(oi, np.tile(np.arange(40), (3, 1)))
    np.testing.assert_array_equal(ov, a)
    assert np.all(orr.view(np.uint32) == 0)  # +0.0 everywhere


@pytest.mark.parametrize("seed", range(4))
def test_error_feedback_identity(seed):
    """r_new + scatter(out_val) == fl32(g + r_old) exactly, over several steps."""
    rng = np.random.default_rng(100 + seed)
    P, N, k = 4, 1000, 37
    r = np.zeros((P, N), np.float32)
    for step in range(5):
        g = rng.standard_normal((P, N)).astype(np.float32) * np.float32(10.0 ** -seed)
        a = (g + r).astype(np.float32)
        oi, ov, r_new = oracle.topk_ef(g, r, k)
        recon = r_new.copy()
        for p in range(P):
            assert np.all(r_new[p, oi[p]].view(np.uint32) == 0)
            recon[p, oi[p]] += ov[p]
        assert np.array_equal(recon, a)  # value equality: -0 + +0 = +0
        assert oi.shape == (P, k)
        r = r_new


def test_negative_zero_key_ties_positive_zero():
    g = np.array([[0.0, -0.0, 0.0, -0.0]], np.float32)
    r = np.zeros_like(g)
    oi, ov, orr = oracle.topk_ef(g, r, 2)
    np.testing.assert_array_equal(oi[0], [0, 1])


def test_golden_topk_hand_examples():
    with open(os.path.join(GOLDEN, "topk_ef_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        g = np.array(c["grad"], np.float32)
        r = np.array(c["residual"], np.float32)
        oi, ov, orr = oracle.topk_ef(g, r, c["k"])
        np.testing.assert_array_equal(oi, np.array(c["idx"], np.uint32), err_msg=c["name"])
        np.testing.assert_array_equal(ov, np.array(c["val"], np.float32), err_msg=c["name"])
        np.testing.assert_array_equal(orr, np.array(c["residual_new"], np.float32), err_msg=c["name"])
