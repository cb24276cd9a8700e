"""The allocation-free reduce (sparcml_sparse_reduce_noalloc) through the C
ABI, against sparcml_sparse_reduce with a torch-allocated workspace on the
same inputs: identical K, dense flag, input flags, indices and values, over
calls in a row on the one static scratch, each later call smaller than the
first (a stale larger table in the scratch must not leak into it)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gradient_reduction_amd as sg
from tests.gpu_util import assert_bits_equal, reduce_tolerance

pytestmark = pytest.mark.gpu


def _inputs(P, N, nnz, seed):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.sort(rng.choice(N, size=nnz, replace=False)) for _ in range(P)]).astype(np.uint32)
    val = rng.standard_normal(P * nnz).astype(np.float32)
    off = [p * nnz for p in range(P + 1)]
    return off, idx, val


def _call_both(off, idx, val, N, delta, dev):
    ii = torch.from_numpy(idx.view(np.int32)).to(dev)
    vv = torch.from_numpy(val).to(dev)
    T = sg.dense_threshold(delta, N)
    cap = max(1, min(N, T - 1))
    # outputs of the allocation-free call are allocated here, by the caller
    a_idx = torch.full((cap,), -1, dtype=torch.int32, device=dev)
    a_val = torch.full((N,), float("nan"), dtype=torch.float32, device=dev)
    a_res = torch.zeros(16, dtype=torch.uint8, device=dev)
    ref = sg.sparse_reduce(off, ii, vv, N, delta)
    got = sg.sparse_reduce_noalloc(off, ii, vv, N, delta, a_idx, a_val, a_res)
    torch.cuda.synchronize()
    return ref.host(), got.host()


SEQUENCES = {
    # (P, N, nnz per node, delta, seed, dense result expected); the union
    # fraction of N is from the uniform model 1 - (1 - nnz/N)^P
    "sparse_dense_sparse": [(64, 1 << 22, 20000, 0.5, 11, False),   # 0.26 of N
                            (8, 1 << 18, 20000, 0.25, 12, True),    # 0.47
                            (5, 100003, 777, 0.3, 13, False)],      # 0.04, ragged last segment
    "dense_sparse_dense": [(64, 1 << 22, 20000, 0.25, 21, True),    # 0.26
                           (16, 1 << 20, 3000, 0.3, 22, False),     # 0.04
                           (3, 70001, 40000, 0.1, 23, True)],       # 0.92, ragged
}


@pytest.mark.parametrize("order", sorted(SEQUENCES))
def test_noalloc_matches_workspace_call_on_calls_in_a_row(dev, order):
    cases = SEQUENCES[order]
    first_pairs = cases[0][0] * cases[0][2]
    for P, N, nnz, delta, seed, want_dense in cases:
        assert P * nnz <= first_pairs  # every later call is smaller than the first
        print(f"noalloc P={P} N={N} nnz={nnz} delta={delta}", flush=True)
        off, idx, val = _inputs(P, N, nnz, seed)
        (K0, d0, f0, i0, v0), (K1, d1, f1, i1, v1) = _call_both(off, idx, val, N, delta, dev)
        assert (K1, d1, f1) == (K0, d0, f0)
        assert f1 == 0 and d1 == want_dense
        assert_bits_equal(i1.numpy(), i0.numpy(), "idx")
        assert_bits_equal(v1.numpy(), v0.numpy(), "val")
        # and the oracle, to the reduce's tolerance
        oK, od, oi, ov = oracle.reduce(np.array(off, np.uint64), idx, val, N, delta)
        assert (oK, od) == (K1, d1)
        if not od:
            assert_bits_equal(i1.numpy().astype(np.uint32), oi, "idx vs oracle")
        assert np.max(np.abs(v1.numpy().astype(np.float64) - ov)) <= reduce_tolerance(P, val)


def test_noalloc_flags_bad_input_and_recovers(dev):
    """An out-of-range index sets the range flag; the next call on the same
    scratch, with valid input, is clean and exact."""
    P, N, nnz = 4, 50000, 300
    off, idx, val = _inputs(P, N, nnz, 31)
    bad = idx.copy()
    bad[5] = N + 3
    bad[4] = min(bad[4], N - 1)
    ii = torch.from_numpy(bad.view(np.int32)).to(dev)
    vv = torch.from_numpy(val).to(dev)
    T = sg.dense_threshold(0.3, N)
    o_idx = torch.empty(max(1, min(N, T - 1)), dtype=torch.int32, device=dev)
    o_val = torch.empty(N, dtype=torch.float32, device=dev)
    res = torch.zeros(16, dtype=torch.uint8, device=dev)
    out = sg.sparse_reduce_noalloc(off, ii, vv, N, 0.3, o_idx, o_val, res)
    torch.cuda.synchronize()
    assert out.read()[2] & sg.FLAG_INDEX_RANGE
    (K0, d0, f0, i0, v0), (K1, d1, f1, i1, v1) = _call_both(off, idx, val, N, 0.3, dev)
    assert (K1, d1, f1) == (K0, d0, 0)
    assert_bits_equal(i1.numpy(), i0.numpy(), "idx")
    assert_bits_equal(v1.numpy(), v0.numpy(), "val")


def test_noalloc_rejects_oversize_without_launch(dev):
    P, N = 1024, 1 << 27
    off = [0] * (P + 1)
    z = torch.zeros(1, dtype=torch.int32, device=dev)
    zf = torch.zeros(1, dtype=torch.float32, device=dev)
    with pytest.raises(sg.SparcmlError) as e:
        sg.sparse_reduce_noalloc(off, z, zf, N, 0.3, z, zf, torch.zeros(16, dtype=torch.uint8, device=dev))
    assert e.value.status == sg.ERR_SCRATCH_LIMIT
