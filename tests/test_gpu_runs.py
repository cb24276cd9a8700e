"""GPU parity of the run-table calls.

sparcml_topk_ef_runs: the Top-k output and the run table of that output, bit
for bit against the oracle (oracle.topk_ef, then oracle.run_table of its
output), on the candidate pipeline, its exact rescan, the one-workgroup row
path, k = 0 and very sparse nodes whose runs span many segments.

sparcml_sparse_reduce_runs: the reduction with a given table equals the plain
reduction bit for bit (same count pass and writer) and the oracle within
1e-6 * P * max|v|; tables that do not fit the pairs set SPARCML_FLAG_RUN_TABLE.
SparCML §5.3.2 (index ranges of the split phase), §5.3 and App. B.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import assert_bits_equal, reduce_tolerance

pytestmark = pytest.mark.gpu

FLAG_RUN_TABLE = 4


def _topk_runs(g, r, k, dev):
    P, N = g.shape
    gd = torch.from_numpy(np.ascontiguousarray(g)).to(dev)
    rd = torch.from_numpy(np.ascontiguousarray(r)).to(dev)
    runs = torch.full(sg.run_table_shape(P, N), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(sg.topk_ef_workspace_bytes(P, N, k), 1), dtype=torch.uint8, device=dev)
    idx, val = sg.topk_ef(gd, rd, k, workspace=ws, runs=runs)
    torch.cuda.synchronize()
    paths = sg.topk_ef_paths(ws, P).cpu().numpy()
    return (idx.cpu().numpy().view(np.uint32), val.cpu().numpy(), rd.cpu().numpy(),
            runs.cpu().numpy().view(np.uint32), paths)


def _check_topk_runs(g, r, k, dev, expect_path=None):
    P, N = g.shape
    oi, ov, orr = oracle.topk_ef(g, r, k)
    o_runs = oracle.run_table(np.arange(P + 1, dtype=np.uint64) * k, oi.reshape(-1), N)
    gi, gv, grr, g_runs, paths = _topk_runs(g, r, k, dev)
    assert_bits_equal(gi, oi, "idx")
    assert_bits_equal(gv, ov, "val")
    assert_bits_equal(grr, orr, "residual")
    assert_bits_equal(g_runs, o_runs, "run table")
    assert np.all(paths[1] == 0), "consistency flag"
    if expect_path is not None and k > 0:
        assert np.all(paths[0] == expect_path), paths[0]


@pytest.mark.parametrize("P,N,k,path", [
    (4, 1 << 20, 10486, 0),      # candidate pipeline
    (3, 300007, 3000, None),     # N not a multiple of the segment
    (5, 65536, 655, 2),          # one workgroup per node, table from the output
    (3, 100003, 0, 2),           # row path, nothing selected
    (2, 1 << 19, 0, None),       # pipeline shape, nothing selected: every run empty
    (2, 1 << 20, 2, None),       # two pairs per node: runs spanning hundreds of segments
    (2, 4096 * 40, 4096 * 40, None),  # every element selected
])
def test_topk_runs_match_oracle(dev, P, N, k, path):
    rng = np.random.default_rng(P * 7919 + N + k)
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.3).astype(np.float32)
    print(f"topk runs P={P} N={N} k={k}", flush=True)
    _check_topk_runs(g, r, k, dev, expect_path=path)


def test_topk_runs_rescan_path(dev):
    """Tie-heavy rows overflow the candidate list: the exact rescan emits the
    pairs and the table, its candidates being every position of the row."""
    P, N, k = 3, 1 << 20, 777
    g = np.full((P, N), 0.5, np.float32)
    g[1, ::3] = -0.5
    g[2, 840000:] = 0.25
    _check_topk_runs(g, np.zeros_like(g), k, dev, expect_path=1)


def test_topk_runs_concentrated_selection(dev):
    """All selected positions of a node inside one stretch: the first and the
    last candidate write long spans of the table."""
    P, N, k = 2, 1 << 21, 5000
    rng = np.random.default_rng(3)
    g = (rng.standard_normal((P, N)) * 1e-3).astype(np.float32)
    g[0, 1_000_000:1_020_000] *= 1000.0
    g[1, N - 9000:] *= 1000.0
    _check_topk_runs(g, np.zeros_like(g), k, dev)


def _sorted_nodes(rng, P, N, nnz_max):
    parts, vals = [], []
    for _ in range(P):
        n = int(rng.integers(0, nnz_max + 1))
        ids = np.sort(rng.choice(N, size=min(n, N), replace=False)).astype(np.uint32)
        parts.append(ids)
        vals.append(rng.standard_normal(ids.size).astype(np.float32))
    off = np.zeros(P + 1, np.uint64)
    off[1:] = np.cumsum([a.size for a in parts])
    return off, np.concatenate(parts), np.concatenate(vals)


def _reduce_pair(off, idx, val, runs, N, delta, dev, hint):
    it = torch.from_numpy(np.ascontiguousarray(idx, np.uint32).view(np.int32)).to(dev)
    vt = torch.from_numpy(np.ascontiguousarray(val, np.float32)).to(dev)
    rt = torch.from_numpy(np.ascontiguousarray(runs, np.uint32).view(np.int32)).to(dev)
    o = [int(x) for x in off]
    a = sg.sparse_reduce(o, it, vt, N, delta, expected_nnz_hint=hint).host()
    b = sg.sparse_reduce(o, it, vt, N, delta, expected_nnz_hint=hint, runs=rt).host()
    return a, b


@pytest.mark.parametrize("P,N,nnz,delta", [
    (1, 1, 1, 0.25), (3, 8193, 2000, 0.3), (8, 30000, 9000, 0.25), (16, 100003, 2000, 0.05),
    (64, 65536, 800, 0.25), (200, 70000, 300, 0.25), (300, 20000, 60, 0.3), (4, 1 << 20, 20000, 0.3),
])
@pytest.mark.parametrize("hint", [0, 1, "dense"])
def test_reduce_runs_equals_reduce_and_oracle(dev, P, N, nnz, delta, hint):
    rng = np.random.default_rng(P * 131 + N + nnz)
    off, idx, val = _sorted_nodes(rng, P, N, nnz)
    runs = oracle.run_table(off, idx, N)
    h = N if hint == "dense" else hint
    print(f"reduce runs P={P} N={N} hint={hint}", flush=True)
    a, b = _reduce_pair(off, idx, val, runs, N, delta, dev, h)
    K, dense, oi, ov = oracle.reduce(off, idx, val, N, delta)
    assert a[2] == 0 and b[2] == 0, (a[2], b[2])
    assert (b[0], b[1]) == (K, dense) and (a[0], a[1]) == (K, dense)
    assert torch.equal(a[3], b[3])
    assert_bits_equal(b[4].numpy(), a[4].numpy(), "sums with and without the table")
    if not dense:
        np.testing.assert_array_equal(b[3].numpy().astype(np.uint32), oi)
    err = np.max(np.abs(b[4].numpy().astype(np.float64) - ov)) if ov.size else 0.0
    assert err <= reduce_tolerance(P, val), err


def test_reduce_runs_after_topk_resnet20_five_steps(dev):
    """The ResNet20-sized workload's five error-feedback steps, sparse to
    dense: Top-k with the table, the reduce with it, each step against the
    oracle's Top-k and reduce."""
    w = W.workload(1)
    P, N, k = w.P, w.N, w.k
    r = torch.zeros((P, N), dtype=torch.float32, device=dev)
    runs = torch.empty(sg.run_table_shape(P, N), dtype=torch.int32, device=dev)
    r_o = np.zeros((P, N), np.float32)
    off = [p * k for p in range(P + 1)]
    seen_dense = set()
    for step in range(w.steps):
        g = W.gradients(w, step, device=dev)
        idx, val = sg.topk_ef(g, r, k, runs=runs)
        out = sg.sparse_reduce(off, idx.view(-1), val.view(-1), N, w.delta, runs=runs).host()
        oi, ov, r_o = oracle.topk_ef(g.cpu().numpy(), r_o, k)
        K, dense, ri, rv = oracle.reduce(np.array(off, np.uint64), oi.reshape(-1), ov.reshape(-1), N, w.delta)
        assert out[2] == 0 and out[0] == K and out[1] == dense, (step, out[:3], K, dense)
        if not dense:
            np.testing.assert_array_equal(out[3].numpy().astype(np.uint32), ri)
        assert np.max(np.abs(out[4].numpy().astype(np.float64) - rv)) <= reduce_tolerance(P, ov)
        seen_dense.add(dense)
    assert seen_dense == {False, True}  # the workload crosses the switch


def test_reduce_runs_tables_that_do_not_fit_set_flag(dev):
    N = 3 * 4096
    idx = np.array([5, 4100, 9000, 1, 2, 3], np.uint32)
    val = np.ones(6, np.float32)
    off = np.array([0, 3, 6], np.uint64)
    good = oracle.run_table(off, idx, N)  # [[0, 1, 2, 3], [3, 6, 6, 6]]
    bad_tables = []
    t = good.copy(); t[0, 1] = 2; bad_tables.append(t)   # 4100 placed in segment 0
    t = good.copy(); t[0, 0] = 1; bad_tables.append(t)   # the first entry is not the node's offset
    t = good.copy(); t[1, 3] = 5; bad_tables.append(t)   # the last entry is not the node's end
    t = good.copy(); t[0, 1] = 3; t[0, 2] = 2; bad_tables.append(t)   # entries out of order
    t = good.copy(); t[1, 1] = 7; bad_tables.append(t)   # an entry past the node's pairs
    for i, t in enumerate(bad_tables):
        for hint in (1, N):
            _, b = _reduce_pair(off, idx, val, t, N, 0.25, dev, hint)
            assert b[2] & FLAG_RUN_TABLE, (i, hint, b[2])
    # an index >= N in a run of the last segment
    idx2 = np.array([5, N + 3], np.uint32)
    off2 = np.array([0, 2], np.uint64)
    t2 = np.array([[0, 1, 1, 2]], np.uint32)
    _, b = _reduce_pair(off2, idx2, np.ones(2, np.float32), t2, N, 0.25, dev, 1)
    assert b[2] & sg.FLAG_INDEX_RANGE
    # the right table afterwards: clean
    a, b = _reduce_pair(off, idx, val, good, N, 0.25, dev, 1)
    assert a[2] == 0 and b[2] == 0 and a[0] == b[0] == 6


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("P,N,nnz,bucket,delta", [
    (3, 8191, 501, 8, 0.25), (8, 30000, 9000, 64, 0.25), (16, 100003, 2003, 512, 0.05), (300, 20000, 77, 16, 0.3),
])
@pytest.mark.parametrize("shift", [0, 1])
def test_reduce_qsgd_runs_equals_plain_and_oracle(dev, bits, P, N, nnz, bucket, delta, shift):
    """Quantized contributions with the run table: the same result as
    sparcml_sparse_reduce_qsgd (bit for bit) and the oracle's reduce of the
    dequantized values. shift = 1 places the indices 4 bytes and the codes 1
    byte past an aligned start (pair-by-pair loads instead of quads)."""
    rng = np.random.default_rng(P * 17 + N + nnz + bits)
    parts, cparts, sparts, dparts = [], [], [], []
    for p in range(P):
        n = int(rng.integers(0, nnz + 1))
        ids = np.sort(rng.choice(N, size=min(n, N), replace=False)).astype(np.uint32)
        vals = rng.standard_normal((1, ids.size)).astype(np.float32)
        c, s = oracle.qsgd(vals, bits, bucket, 7, 3, node0=p)
        parts.append(ids)
        cparts.append(c[0])
        sparts.append(s[0])
        dparts.append(oracle.dqsgd(c, s, ids.size, bits, bucket)[0])
    off = np.zeros(P + 1, np.uint64)
    off[1:] = np.cumsum([a.size for a in parts])
    idx, codes = np.concatenate(parts), np.concatenate(cparts).astype(np.uint8)
    scales, deq = np.concatenate(sparts).astype(np.float32), np.concatenate(dparts).astype(np.float32)
    runs = oracle.run_table(off, idx, N)
    bi = torch.zeros(idx.size + 8, dtype=torch.int32, device=dev)
    bc = torch.zeros(codes.size + 8, dtype=torch.uint8, device=dev)
    bi[shift:shift + idx.size] = torch.from_numpy(idx.view(np.int32)).to(dev)
    bc[shift:shift + codes.size] = torch.from_numpy(codes).to(dev)
    it, ct = bi[shift:shift + idx.size], bc[shift:shift + codes.size]
    st = torch.from_numpy(scales).to(dev)
    rt = torch.from_numpy(runs.view(np.int32)).to(dev)
    o = [int(x) for x in off]
    K, dense, oi, ov = oracle.reduce(off, idx, deq, N, delta)
    print(f"reduce_qsgd runs bits={bits} P={P} N={N} shift={shift}", flush=True)
    for hint in (0, 1, N):
        a = sg.sparse_reduce_qsgd(o, it, ct, st, bits, bucket, N, delta, expected_nnz_hint=hint).host()
        b = sg.sparse_reduce_qsgd(o, it, ct, st, bits, bucket, N, delta, expected_nnz_hint=hint, runs=rt).host()
        assert a[2] == 0 and b[2] == 0 and (a[0], a[1]) == (K, dense) == (b[0], b[1])
        assert torch.equal(a[3], b[3])
        assert_bits_equal(b[4].numpy(), a[4].numpy(), "quantized sums with and without the table")
        if not dense:
            np.testing.assert_array_equal(b[3].numpy().astype(np.uint32), oi)
        err = np.max(np.abs(b[4].numpy().astype(np.float64) - ov)) if ov.size else 0.0
        assert err <= reduce_tolerance(P, deq), err


@pytest.mark.parametrize("P,N,nnz,delta", [
    (3, 8193, 2000, 0.3), (16, 100003, 2000, 0.05), (300, 20000, 60, 0.3), (8, 1 << 24, 3000, 0.25),
    (8, 1 << 25, 3000, 0.25), (64, 1 << 20, 3000, 0.3),
])
@pytest.mark.parametrize("table", [False, True])
@pytest.mark.parametrize("hint", [0, 1, "dense"])
def test_reduce_in_two_phases_equals_one_call(dev, P, N, nnz, delta, table, hint):
    """sparcml_sparse_reduce_union, other work on the stream, then
    sparcml_sparse_reduce_sums: the one-call result bit for bit (with the
    decide pass where there are more than 4096 writer groups, N = 2^25, and
    writers that add up the counts themselves otherwise, 4096 of them at
    N = 2^24), and the oracle's."""
    rng = np.random.default_rng(P * 7 + N + nnz)
    off, idx, val = _sorted_nodes(rng, P, N, nnz)
    runs = oracle.run_table(off, idx, N)
    it = torch.from_numpy(idx.view(np.int32)).to(dev)
    vt = torch.from_numpy(val).to(dev)
    rt = torch.from_numpy(runs.view(np.int32)).to(dev) if table else None
    o = [int(x) for x in off]
    h = N if hint == "dense" else hint
    print(f"two phases P={P} N={N} table={table} hint={hint}", flush=True)
    one = sg.sparse_reduce(o, it, vt, N, delta, expected_nnz_hint=h, runs=rt).host()
    u = sg.sparse_reduce_union(o, it, N, delta, runs=rt, expected_nnz_hint=h)
    junk = torch.randn(1 << 20, device=dev)  # unrelated work between the phases
    junk.mul_(2.0).sum().item()
    two = sg.sparse_reduce_sums(u, vt).host()
    assert one[:3] == two[:3] and one[2] == 0
    assert torch.equal(one[3], two[3])
    assert_bits_equal(two[4].numpy(), one[4].numpy(), "two phases")
    K, dense, oi, ov = oracle.reduce(off, idx, val, N, delta)
    assert (two[0], two[1]) == (K, dense)
    if not dense:
        np.testing.assert_array_equal(two[3].numpy().astype(np.uint32), oi)
    err = np.max(np.abs(two[4].numpy().astype(np.float64) - ov)) if ov.size else 0.0
    assert err <= reduce_tolerance(P, val), err
