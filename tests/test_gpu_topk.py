"""GPU parity: sparcml_topk_ef against the oracle, bit for bit (index sets,
values, residual), over ragged shapes, ties, both internal paths, the
ResNet20-sized five-step error-feedback run and the LSTM/ASR-sized gradient."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import assert_bits_equal, run_topk

pytestmark = pytest.mark.gpu


def _check(g, r, k, dev, expect_path=None):
    oi, ov, orr = oracle.topk_ef(g, r, k)
    gi, gv, grr, paths = run_topk(g, r, k, dev)
    assert_bits_equal(gi, oi, "idx")
    assert_bits_equal(gv, ov, "val")
    assert_bits_equal(grr, orr, "residual")
    assert np.all(paths[1] == 0), "consistency flag"
    if expect_path is not None and k > 0:
        assert np.all(paths[0] == expect_path), paths[0]
    return paths


@pytest.mark.parametrize("P,N,k", [
    (1, 1, 1), (1, 1, 0), (3, 7, 3), (2, 100, 10), (4, 8191, 100), (4, 8193, 4000),
    (5, 65537, 655), (3, 32769, 330), (2, 100003, 1), (2, 100003, 100003), (7, 20000, 0),
    (6, 30001, 29999), (9, 123457, 6172), (2, 131072, 1310), (3, 131076, 1310), (2, 131068, 131068), (5, 4, 2), (3, 65536, 655),
    (2, 131072, 0), (4, 12, 12), (7, 3, 2), (5, 6, 5), (3, 131071, 1310), (6, 9, 4),
])
def test_topk_random_shapes(dev, P, N, k):
    rng = np.random.default_rng(P * 1000003 + N + k)
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.5).astype(np.float32)
    print(f"topk P={P} N={N} k={k}", flush=True)
    paths = _check(g, r, k, dev)
    if N <= sg.TOPK_ROW_MAX and P * N <= sg.TOPK_ROW_TOTAL_MAX:  # short rows: one workgroup per node
        assert np.all(paths[0] == 2), paths[0]
    elif k > 0:
        assert np.all(paths[0] <= 1), paths[0]


def test_topk_ties_take_lowest_indices_rescan_path(dev):
    P, N, k = 3, 1 << 20, 777
    g = np.full((P, N), 0.5, np.float32)
    g[1, ::3] = -0.5
    g[2, 840000:] = 0.25  # 840000 ties: still more than the list holds (256 regions of 1287 slots)
    r = np.zeros_like(g)
    _check(g, r, k, dev, expect_path=1)  # far more candidates than the list holds


def test_topk_ties_mixed_with_distinct(dev):
    rng = np.random.default_rng(5)
    P, N, k = 4, 70000, 3000
    g = (rng.integers(-20, 21, size=(P, N)) * 0.125).astype(np.float32)
    r = np.zeros_like(g)
    _check(g, r, k, dev)


@pytest.mark.parametrize("N", [65536, 65533, 70001])
@pytest.mark.parametrize("cut", [0, -5])
def test_topk_row_ties_at_the_boundary(dev, N, cut):
    """One-workgroup rows with 41 value levels, every node a permutation of the
    same multiset: k ends exactly at a level (every key equal to the k-th
    largest is taken, many of them) or five short of it (only the lowest
    indices among them). Rows of 65536 or fewer elements are held in
    registers; 65533 leaves every row but the first unaligned."""
    rng = np.random.default_rng(N + 17)
    P = 4
    base = (rng.integers(-20, 21, size=N) * 0.125).astype(np.float32)
    g = np.stack([rng.permutation(base) for _ in range(P)])
    r = np.zeros_like(g)
    k = int(np.count_nonzero(np.abs(base) >= 1.5)) + cut
    print(f"topk row ties N={N} k={k}", flush=True)
    _check(g, r, k, dev, expect_path=2)


@pytest.mark.parametrize("N", [65536, 65531])
def test_topk_row_crowded_first_digit(dev, N):
    """Every key of a register-held row in one bin of the first 11-bit digit
    (values in [1, 1.125)): both refining passes see the whole row, and the
    histogram's atomics all land on a few bins."""
    rng = np.random.default_rng(N)
    P, k = 3, 655
    g = (1.0 + rng.random((P, N)) * 0.125).astype(np.float32)
    g[:, ::7] *= -1.0
    r = np.zeros_like(g)
    _check(g, r, k, dev, expect_path=2)


def test_topk_sample_underestimate_takes_rescan_path(dev):
    """Large values placed exactly on the sampled chunks make the predicted
    threshold too high: fewer than k candidates, exact rescan."""
    P, N, k = 2, 1 << 20, 60000
    rng = np.random.default_rng(9)
    g = (rng.standard_normal((P, N)) * 1e-3).astype(np.float32)
    for c in range(1024):  # the 1024 sampled chunks of 64 elements, c * ((N - 64) // 1023) on
        s = c * ((N - 64) // 1023)
        g[:, s:s + 64] = (10.0 + rng.random((P, 64))).astype(np.float32)
    r = np.zeros_like(g)
    _check(g, r, k, dev, expect_path=1)


def test_topk_skewed_quarter(dev):
    """One quarter of each node at 1000 times the scale of the rest: every
    selected element lies in it, the sample's estimate comes from the chunks
    that fall in it, and the result is exact on the candidate path."""
    P, N = 2, 1 << 22
    k = N // 200
    rng = np.random.default_rng(22)
    g = rng.standard_normal((P, N)).astype(np.float32)
    g[:, :N // 4] *= 1000.0
    r = (rng.standard_normal((P, N)) * 1e-2).astype(np.float32)
    _check(g, r, k, dev, expect_path=0)


def test_topk_normal_data_takes_candidate_path(dev):
    rng = np.random.default_rng(10)
    P, N = 4, 1 << 20
    k = N // 100
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = np.zeros_like(g)
    _check(g, r, k, dev, expect_path=0)


def test_topk_crowded_stretch_stays_on_candidate_path(dev):
    """Candidates crowded into one stretch of a long node (2^18 elements at 100
    times the scale of the other 2^23): the tiles of the stretch feed many
    counter regions, so the node keeps the candidate path."""
    rng = np.random.default_rng(14)
    P, N = 2, 1 << 23
    k = N // 200
    g = (rng.standard_normal((P, N)) * 1e-3).astype(np.float32)
    g[:, 3_000_000:3_000_000 + (1 << 18)] *= 100.0
    r = np.zeros_like(g)
    _check(g, r, k, dev, expect_path=0)


def test_topk_subnormal_and_signed_zero(dev):
    rng = np.random.default_rng(12)
    P, N, k = 3, 40000, 900
    g = (rng.integers(-5, 6, size=(P, N)).astype(np.float32) * np.float32(1e-45))
    g[rng.random((P, N)) < 0.3] = -0.0
    r = (rng.integers(-2, 3, size=(P, N)).astype(np.float32) * np.float32(1e-45))
    _check(g, r, k, dev)


def test_topk_workload0(dev):
    w = W.workload(0)
    g = W.gradients(w, 0).numpy()
    _check(g, np.zeros_like(g), w.k, dev)


def test_topk_resnet20_five_steps_carry_residual(dev):
    w = W.workload(1)
    r_o = np.zeros((w.P, w.N), np.float32)
    rd = torch.zeros((w.P, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(sg.topk_ef_workspace_bytes(w.P, w.N, w.k), dtype=torch.uint8, device=dev)
    for step in range(w.steps):
        g = W.gradients(w, step).numpy()
        oi, ov, r_o = oracle.topk_ef(g, r_o, w.k)
        gi, gv = sg.topk_ef(torch.from_numpy(g).to(dev), rd, w.k, workspace=ws)
        assert_bits_equal(gi.cpu().numpy().view(np.uint32), oi, f"idx step {step}")
        assert_bits_equal(gv.cpu().numpy(), ov, f"val step {step}")
        assert_bits_equal(rd.cpu().numpy(), r_o, f"residual step {step}")


def test_topk_deterministic(dev):
    rng = np.random.default_rng(13)
    g = rng.standard_normal((4, 300000)).astype(np.float32)
    r = rng.standard_normal((4, 300000)).astype(np.float32)
    a = run_topk(g, r, 3000, dev)
    b = run_topk(g, r, 3000, dev)
    for x, y in zip(a[:3], b[:3]):
        assert_bits_equal(x, y, "repeat")


def test_topk_laplace_full_size_sampled_nodes(dev):
    """LSTM/ASR-sized gradient (N = 2^26, P = 8) in the bench's launch
    configuration: oracle on two nodes, properties on all."""
    w = W.workload(2)
    g = W.gradients(w, 0, device=dev)
    r = (W.gradients(w, 1, device=dev) * 0.5).contiguous()
    r_old = r.clone()
    idx, val = sg.topk_ef(g, r, w.k)
    torch.cuda.synchronize()
    for p in (0, w.P - 1):
        oi, ov, orr = oracle.topk_ef(g[p:p + 1].cpu().numpy(), r_old[p:p + 1].cpu().numpy(), w.k)
        assert_bits_equal(idx[p:p + 1].cpu().numpy().view(np.uint32), oi, f"idx node {p}")
        assert_bits_equal(val[p:p + 1].cpu().numpy(), ov, f"val node {p}")
        assert_bits_equal(r[p:p + 1].cpu().numpy(), orr, f"residual node {p}")
    # all nodes: ascending unique indices, EF identity exactly
    il = idx.to(torch.int64) & 0xFFFFFFFF
    assert bool((il[:, 1:] > il[:, :-1]).all())
    a = g + r_old
    recon = r.clone()
    recon.scatter_add_(1, il, val)
    assert torch.equal(recon, a)
    assert bool((torch.gather(r, 1, il) == 0).all())
    # every unselected magnitude is <= every selected one
    min_sel = val.abs().min(dim=1).values
    unsel_max = r.abs().max(dim=1).values
    assert bool((unsel_max <= min_sel).all())


def test_topk_max_nodes(dev):
    """65535 nodes (the largest second launch dimension) of 5 elements."""
    rng = np.random.default_rng(14)
    P, N, k = 65535, 5, 2
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = np.zeros_like(g)
    _check(g, r, k, dev)


def test_topk_wideresnet_full_size_two_ef_steps(dev):
    """The wide-ResNet-sized call as the bench makes it: P = 64 nodes of
    N = 2^27, k = 0.5% (671 088), two error-feedback steps with the residual
    carried on the device. Nodes 0 and 63 bit for bit against the oracle's
    own residual chain, with the 4-bit codes of their sent values and the run
    table rows of their output (sparcml_topk_ef_runs); on all 64 nodes the
    exact EF identity, strictly ascending indices and no unselected magnitude
    above a selected one. The reduce of the last step's pairs with that table,
    in one call and in two phases, equals the reduce that finds the runs
    itself, bit for bit."""
    w = W.workload(4)
    P, N, k, B = w.P, w.N, w.k, w.q4_bucket
    seed = 987654321
    r = torch.zeros((P, N), dtype=torch.float32, device=dev)
    ws = torch.empty(sg.topk_ef_workspace_bytes(P, N, k), dtype=torch.uint8, device=dev)
    idx = torch.empty((P, k), dtype=torch.int32, device=dev)
    val = torch.empty((P, k), dtype=torch.float32, device=dev)
    runs = torch.empty(sg.run_table_shape(P, N), dtype=torch.int32, device=dev)
    sample = (0, P - 1)
    r_o = {p: np.zeros((1, N), np.float32) for p in sample}
    for step in range(2):
        print(f"wide-ResNet Top-k step {step}", flush=True)
        g = W.gradients(w, step, device=dev)
        r_old = r.clone()
        sg.topk_ef(g, r, k, out_idx=idx, out_val=val, workspace=ws, runs=runs)
        codes, scales = sg.q4(val, B, seed, step)
        torch.cuda.synchronize()
        paths = sg.topk_ef_paths(ws, P).cpu().numpy()
        assert np.all(paths[1] == 0), "consistency flag"
        assert np.all(paths[0] <= 1), paths[0]  # the candidate pipeline (or its exact rescan)
        for p in sample:
            oi, ov, orr = oracle.topk_ef(g[p:p + 1].cpu().numpy(), r_o[p], k)
            assert_bits_equal(idx[p:p + 1].cpu().numpy().view(np.uint32), oi, f"idx node {p} step {step}")
            assert_bits_equal(val[p:p + 1].cpu().numpy(), ov, f"val node {p} step {step}")
            assert_bits_equal(r[p:p + 1].cpu().numpy(), orr, f"residual node {p} step {step}")
            # node p's table row: the oracle's table of its own k pairs, positions counted from p * k
            o_runs = oracle.run_table(np.array([0, k], np.uint64), oi.reshape(-1), N) + np.uint32(p * k)
            assert_bits_equal(runs[p:p + 1].cpu().numpy().view(np.uint32), o_runs, f"run table node {p} step {step}")
            oc, osc = oracle.qsgd(ov, 4, B, seed, step, node0=p)
            assert_bits_equal(codes[p:p + 1].cpu().numpy(), oc, f"q4 codes node {p} step {step}")
            assert_bits_equal(scales[p:p + 1].cpu().numpy(), osc, f"q4 scales node {p} step {step}")
            r_o[p] = orr
        for c0 in range(0, P, 8):  # properties on every node, 8 nodes at a time
            c = slice(c0, c0 + 8)
            il = idx[c].to(torch.int64) & 0xFFFFFFFF
            assert bool((il[:, 1:] > il[:, :-1]).all()), f"ascending, nodes {c0}.."
            a = g[c] + r_old[c]
            recon = r[c].clone()
            assert bool((torch.gather(recon, 1, il) == 0).all()), f"sent positions zeroed, nodes {c0}.."
            recon.scatter_add_(1, il, val[c])
            assert torch.equal(recon, a), f"EF identity, nodes {c0}.."
            min_sel = val[c].abs().min(dim=1).values
            unsel_max = r[c].abs().max(dim=1).values
            assert bool((unsel_max <= min_sel).all()), f"magnitude split, nodes {c0}.."
            del il, a, recon
        del g, r_old, codes, scales
        torch.cuda.empty_cache()
    off = [p * k for p in range(P + 1)]
    plain = sg.sparse_reduce(off, idx.view(-1), val.view(-1), N, w.delta)
    K, dense, flags = plain.read()
    assert flags == 0
    n = N if dense else K
    with_runs = sg.sparse_reduce(off, idx.view(-1), val.view(-1), N, w.delta, runs=runs)
    # and in two phases with the table, the union before other work on the stream
    u = sg.sparse_reduce_union(off, idx.view(-1), N, w.delta, runs=runs)
    sg.q4(val, B, seed, 5)
    phased = sg.sparse_reduce_sums(u, val.view(-1))
    for other in (with_runs, phased):
        assert (K, dense, flags) == other.read()
        assert torch.equal(plain.out_val[:n].view(torch.int32), other.out_val[:n].view(torch.int32))
        if not dense:
            assert torch.equal(plain.out_idx[:K], other.out_idx[:K])


@pytest.mark.parametrize("scale", [64.0, 1 << 16])
def test_topk_ties_around_the_threshold_on_the_candidate_path(dev, scale):
    """Values on a grid of 1/scale: at 1/64 every chunk of candidates holds
    far more keys sharing T*'s upper 21 bits than the 32 last-digit slots
    the last histogram pass keeps (the count pass then counts those chunks),
    at 2^-16 only a few (the scan finishes the counts from the slots). Both
    against the oracle, on the candidate path."""
    rng = np.random.default_rng(int(scale))
    P, N, k = 3, 1 << 20, 10486
    g = (np.round(rng.standard_normal((P, N)) * scale) / scale).astype(np.float32)
    r = np.zeros_like(g)
    _check(g, r, k, dev)


def test_topk_some_chunks_past_their_digit_slots(dev):
    """Ties at T* = 1.0 clustered in one stretch of a node (one chunk of
    candidates holds thousands of them, the others none), spread thinly over
    another node (every chunk within its digit slots), and both at once on a
    third: the count pass counts only the crowded chunks and the scan
    finishes the rest from their slots, against the oracle."""
    rng = np.random.default_rng(29)
    P, N, k = 3, 1 << 20, 10486
    g = (rng.uniform(-0.9, 0.9, size=(P, N))).astype(np.float32)
    for p in range(P):
        g[p, rng.choice(N, 10000, replace=False)] = 2.0  # above T*
    g[0, 500000:503000] = 1.0
    g[1, np.arange(600) * 1747 + 11] = 1.0
    g[2, 200000:201000] = -1.0
    g[2, 700000:701000] = 1.0
    g[2, np.arange(300) * 3001 + 5] = 1.0
    r = np.zeros_like(g)
    print("topk ties clustered and spread at T*", flush=True)
    _check(g, r, k, dev)
