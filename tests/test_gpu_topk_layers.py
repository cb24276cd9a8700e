"""GPU parity: sparcml_topk_ef_layers against the oracle, bit for bit (index
rows, values, residual): random layer cuts with empty, sub-tile and
misaligned layers, k = 0 and k = n layers, a row forced onto the exact
rescan path, several error-feedback steps, and a full-size layer list."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import assert_bits_equal

pytestmark = pytest.mark.gpu


def _run(g, r, off, ks, dev):
    gd = torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(dev)
    rd = torch.from_numpy(np.ascontiguousarray(r, np.float32)).to(dev)
    P, N = g.shape
    ws = torch.empty(max(1, sg.topk_ef_layers_workspace_bytes(P, N, off, ks)), dtype=torch.uint8, device=dev)
    idx, val = sg.topk_ef_layers(gd, rd, off, ks, workspace=ws)
    torch.cuda.synchronize()
    rows = P * len(ks)
    paths = ws[: 8 * rows].view(torch.int32).view(2, rows).cpu().numpy()
    return idx.cpu().numpy().view(np.uint32), val.cpu().numpy(), rd.cpu().numpy(), paths


def _check(g, r, off, ks, dev, expect_rescan_rows=None):
    oi, ov, orr = oracle.topk_ef_layers(g, r, off, ks)
    gi, gv, grr, paths = _run(g, r, off, ks, dev)
    assert_bits_equal(gi, oi, "idx")
    assert_bits_equal(gv, ov, "val")
    assert_bits_equal(grr, orr, "residual")
    assert np.all(paths[1] == 0), "consistency flag"
    if expect_rescan_rows is not None:
        assert set(np.nonzero(paths[0] == 1)[0].tolist()) == set(expect_rescan_rows), paths[0]
    short = np.max(np.diff(np.asarray(off, np.int64))) <= sg.TOPK_ROW_MAX
    if short and g.size <= sg.TOPK_ROW_TOTAL_MAX:  # only short layers, small call: one workgroup per row
        assert np.all(paths[0] == 2), paths[0]
    return paths


def _random_layers(rng, N, nl):
    cuts = np.sort(rng.integers(0, N + 1, size=nl - 1))  # repeats make empty layers
    return np.concatenate([[0], cuts, [N]]).astype(np.uint64)


@pytest.mark.parametrize("P,N,nl", [(1, 1, 1), (2, 100, 3), (3, 5003, 9), (4, 70001, 17), (2, 300000, 40),
                                    (7, 20000, 200), (64, 4099, 5)])
def test_layers_random(dev, P, N, nl):
    rng = np.random.default_rng(P * 1009 + N + nl)
    off = _random_layers(rng, N, nl)
    sizes = np.diff(off.astype(np.int64))
    ks = np.array([0 if s == 0 else rng.integers(0, s + 1) for s in sizes], np.uint64)
    nz = np.nonzero(sizes)[0]
    if nz.size:
        ks[nz[0]] = sizes[nz[0]]  # one layer kept whole
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.5).astype(np.float32)
    print(f"layers P={P} N={N} nl={nl} K={int(ks.sum())}", flush=True)
    _check(g, r, off, ks, dev)


@pytest.mark.parametrize("P,N,nl", [(2, 100, 3), (3, 5003, 9), (4, 70001, 17), (7, 20000, 200)])
def test_layers_random_with_a_long_layer(dev, P, N, nl):
    """The random short layers of test_layers_random followed by one layer
    longer than the one-workgroup limit, which sends every row through the
    candidate pipeline."""
    rng = np.random.default_rng(P * 1013 + N + nl)
    long = sg.TOPK_ROW_MAX + 5
    off = np.concatenate([_random_layers(rng, N, nl), [N + long]]).astype(np.uint64)
    sizes = np.diff(off.astype(np.int64))
    ks = np.array([0 if s == 0 else rng.integers(0, s + 1) for s in sizes], np.uint64)
    ks[-1] = long // 50
    N += long
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.5).astype(np.float32)
    print(f"layers + long layer P={P} N={N} nl={nl + 1}", flush=True)
    paths = _check(g, r, off, ks, dev)
    assert np.all(paths[0] <= 1), paths[0]


def test_layers_prediction_size_classes(dev):
    """Layers on both sides of each prediction size class: whole-row
    candidates (<= 16384), samples held by 256-thread blocks (<= 16384
    keys, n < 257 * 4096) and by 1024-thread blocks (up to 65536 keys), at
    1%, with line-misaligned starts; every row stays on the candidate path."""
    sizes = [16384, 16385, 777, 1048575, 1052672, 1052671 + 4096, 4194305, 123457]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.uint64)
    ks = np.array([max(1, s // 100) for s in sizes], np.uint64)
    P, N = 3, int(off[-1])
    rng = np.random.default_rng(2718)
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.5).astype(np.float32)
    print(f"layers size classes P={P} N={N}", flush=True)
    _check(g, r, off, ks, dev, expect_rescan_rows=[])


def test_layers_one_layer_equals_whole_vector(dev):
    rng = np.random.default_rng(3)
    P, N, k = 4, 300001, 3000
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = rng.standard_normal((P, N)).astype(np.float32)
    li, lv, lr, _ = _run(g, r, [0, N], [k], dev)
    gd = torch.from_numpy(g).to(dev)
    rd = torch.from_numpy(r).to(dev)
    ti, tv = sg.topk_ef(gd, rd, k)
    torch.cuda.synchronize()
    assert_bits_equal(li, ti.cpu().numpy().view(np.uint32), "idx")
    assert_bits_equal(lv, tv.cpu().numpy(), "val")
    assert_bits_equal(lr, rd.cpu().numpy(), "residual")


def test_layers_short_rows_with_ties(dev):
    """Short layers of 41 value levels: ties at the k-th largest key in most
    rows, partly or wholly taken, on the one-workgroup row path."""
    rng = np.random.default_rng(11)
    P, N = 3, 200003
    off = np.array([0, 5, 65541, 65542, 130000, 170001, N], np.uint64)
    sizes = np.diff(off.astype(np.int64))
    ks = np.array([2, 3000, 1, 65536 // 8, 4000, 555], np.uint64)
    assert np.all(ks <= sizes)
    g = (rng.integers(-20, 21, size=(P, N)) * 0.125).astype(np.float32)
    r = np.zeros_like(g)
    _check(g, r, off, ks, dev)


def test_layers_rows_longer_than_registers(dev):
    """A per-layer call whose longest layer (100003 elements) is beyond what a
    workgroup holds in registers but within the one-workgroup row limit: every
    row streams its passes from memory, unaligned layers included."""
    rng = np.random.default_rng(12)
    P, N = 2, 200001
    off = np.array([0, 100003, 100004, 165000, N], np.uint64)
    ks = np.array([1000, 1, 650, 350], np.uint64)
    g = rng.standard_normal((P, N)).astype(np.float32)
    r = (rng.standard_normal((P, N)) * 0.5).astype(np.float32)
    assert np.max(np.diff(off.astype(np.int64))) > 65536
    _check(g, r, off, ks, dev)


def test_layers_rescan_row(dev):
    """A large layer of equal values far exceeds its candidate capacity: that
    row alone takes the exact rescan path."""
    rng = np.random.default_rng(4)
    P, N = 2, 400000
    off = np.array([0, 1000, 301000, N], np.uint64)
    ks = np.array([10, 777, 900], np.uint64)
    g = rng.standard_normal((P, N)).astype(np.float32)
    g[1, 1000:301000] = 0.5  # 300000 ties in node 1, layer 1 (row 4)
    r = np.zeros_like(g)
    _check(g, r, off, ks, dev, expect_rescan_rows=[4])


def test_layers_error_feedback_steps(dev):
    rng = np.random.default_rng(5)
    P, N = 3, 150000
    off = W.layer_offsets(N, 30, seed=7)
    ks = W.layer_ks(off, 1, 100)
    rd = torch.zeros((P, N), dtype=torch.float32, device=dev)
    r_o = np.zeros((P, N), np.float32)
    for step in range(4):
        g = rng.laplace(0, 1e-3, (P, N)).astype(np.float32)
        oi, ov, r_o = oracle.topk_ef_layers(g, r_o, off, ks)
        gi, gv = sg.topk_ef_layers(torch.from_numpy(g).to(dev), rd, off, ks)
        torch.cuda.synchronize()
        assert_bits_equal(gi.cpu().numpy().view(np.uint32), oi, f"idx step {step}")
        assert_bits_equal(gv.cpu().numpy(), ov, f"val step {step}")
        assert_bits_equal(rd.cpu().numpy(), r_o, f"residual step {step}")


def test_layers_full_size_sampled_nodes(dev):
    """P = 64, N = 2^27 cut into 160 layers, 1% of every layer: oracle on two
    nodes, properties on all."""
    w = W.workload(4)
    P, N = w.P, w.N
    off = W.layer_offsets(N, 160)
    ks = W.layer_ks(off, 1, 100)
    g = W.gradients(w, 0, device=dev)
    r = torch.zeros_like(g)
    idx, val = sg.topk_ef_layers(g, r, off, ks)
    torch.cuda.synchronize()
    for p in (0, P - 1):
        gp = g[p:p + 1].cpu().numpy()
        oi, ov, orr = oracle.topk_ef_layers(gp, np.zeros_like(gp), off, ks)
        assert_bits_equal(idx[p:p + 1].cpu().numpy().view(np.uint32), oi, f"idx node {p}")
        assert_bits_equal(val[p:p + 1].cpu().numpy(), ov, f"val node {p}")
        assert_bits_equal(r[p:p + 1].cpu().numpy(), orr, f"residual node {p}")
    il = idx.to(torch.int64) & 0xFFFFFFFF
    assert bool((il[:, 1:] > il[:, :-1]).all())
    recon = r.clone()
    recon.scatter_add_(1, il, val)
    assert torch.equal(recon, g)
