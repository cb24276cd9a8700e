"""Pins for the oracle's run table (CPU only).

SparCML §5.3.2: the split phase gives each owner one range of indices and
every node hands it the part of its sorted pairs that falls there. The run
table records, per node and range, where that part starts.
"""
import numpy as np
import pytest

import oracle


def _sorted_nodes(rng, P, N, max_nnz):
    parts = []
    for _ in range(P):
        n = int(rng.integers(0, min(max_nnz, N) + 1))
        parts.append(np.sort(rng.choice(N, size=n, replace=False)).astype(np.uint32))
    off = np.zeros(P + 1, np.uint64)
    off[1:] = np.cumsum([a.size for a in parts])
    return off, (np.concatenate(parts) if parts else np.zeros(0, np.uint32))


def _brute(off, idx, N, seg):
    """Every entry counted directly: node p's pairs below s * seg, after its offset."""
    P = off.size - 1
    S = -(-N // seg)
    out = np.zeros((P, S + 1), np.int64)
    for p in range(P):
        mine = [int(i) for i in idx[int(off[p]):int(off[p + 1])]]
        for s in range(S + 1):
            out[p, s] = int(off[p]) + sum(1 for i in mine if i < s * seg)
    return out


@pytest.mark.parametrize("seed", range(10))
def test_run_table_matches_brute_force_count(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 7))
    seg = int(rng.choice([1, 3, 8, 64]))
    N = int(rng.integers(1, 400))
    off, idx = _sorted_nodes(rng, P, N, max_nnz=N)
    got = oracle.run_table(off, idx, N, seg)
    np.testing.assert_array_equal(got.astype(np.int64), _brute(off, idx, N, seg))


def test_run_table_ends_and_membership():
    rng = np.random.default_rng(5)
    P, N, seg = 9, 100_003, 4096  # N not a multiple of the range size
    off, idx = _sorted_nodes(rng, P, N, max_nnz=3000)
    runs = oracle.run_table(off, idx, N, seg).astype(np.int64)
    S = -(-N // seg)
    assert runs.shape == (P, S + 1)
    np.testing.assert_array_equal(runs[:, 0], off[:-1].astype(np.int64))
    np.testing.assert_array_equal(runs[:, S], off[1:].astype(np.int64))
    assert np.all(np.diff(runs, axis=1) >= 0)
    for p in range(P):
        for s in range(S):
            part = idx[runs[p, s]:runs[p, s + 1]].astype(np.int64)
            assert np.all((part >= s * seg) & (part < (s + 1) * seg))


def test_run_table_edges_of_ranges():
    # indices right at and right below each range start
    N, seg = 5 * 4096, 4096
    a = np.array([0, 4095, 4096, 8191, 12288, 20479], np.uint32)
    b = np.zeros(0, np.uint32)  # an empty node
    c = np.array([20479], np.uint32)  # only the last index
    idx = np.concatenate([a, b, c])
    off = np.array([0, a.size, a.size, a.size + 1], np.uint64)
    runs = oracle.run_table(off, idx, N, seg).astype(np.int64)
    np.testing.assert_array_equal(runs[0], [0, 2, 4, 4, 5, 6])
    np.testing.assert_array_equal(runs[1], [6, 6, 6, 6, 6, 6])
    np.testing.assert_array_equal(runs[2], [6, 6, 6, 6, 6, 7])


def test_run_table_rejects_index_out_of_range():
    with pytest.raises(ValueError):
        oracle.run_table(np.array([0, 2], np.uint64), np.array([1, 4096], np.uint32), 4096)
