"""The measurement entry points (include/sparcml_bench.h) on the GPU: each
gives the same results as the call of the same name, bit for bit, and the
events it attaches to the kernel dispatches give an op span that contains its
dominant kernel's own duration."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_gradient_reduction_amd as sg
from sparse_gradient_reduction_amd import workloads as W
from tests.gpu_util import assert_bits_equal

pytestmark = pytest.mark.gpu

hip = ctypes.CDLL("libamdhip64.so")
hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
hip.hipEventDestroy.argtypes = [ctypes.c_void_p]


def _event():
    e = ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(e)) == 0
    return e.value


def _ms(a, b):
    out = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
    return out.value


def _events(op_stop=True, kernel=True):
    return sg.BenchEvents(_event(), _event() if op_stop else None, _event() if kernel else None,
                          _event() if kernel else None)


@pytest.mark.parametrize("P,N,k", [(8, 1 << 20, 5243), (4, 4096, 41), (16, 1 << 18, 0)])
def test_bench_topk_matches_plain_call(P, N, k):
    """Whole-vector pipeline, the one-workgroup row path, and k = 0 (the
    stream kernel is the op's last kernel)."""
    dev = torch.device("cuda:0")
    g = torch.from_numpy(np.random.default_rng(P + N + k).standard_normal((P, N), dtype=np.float32)).to(dev)
    r0 = torch.from_numpy(np.random.default_rng(7).standard_normal((P, N), dtype=np.float32)).to(dev) * 0.1
    ra, rb = r0.clone(), r0.clone()
    ia, va = sg.topk_ef(g, ra, k)
    e = _events()
    ib, vb = sg.topk_ef(g, rb, k, events=e)
    torch.cuda.synchronize()
    assert_bits_equal(ia.cpu().numpy(), ib.cpu().numpy(), "idx")
    assert_bits_equal(va.cpu().numpy(), vb.cpu().numpy(), "val")
    assert_bits_equal(ra.cpu().numpy(), rb.cpu().numpy(), "residual")
    span = _ms(e.op_start, e.op_stop)
    assert span > 0.0
    if N <= sg.TOPK_ROW_MAX and P * N <= sg.TOPK_ROW_TOTAL_MAX:
        return  # one kernel: it carries the op's pair only
    kern = _ms(e.kernel_start, e.kernel_stop)
    assert 0.0 < kern <= span + 1e-3, (kern, span)


@pytest.mark.parametrize("P,N,k,delta", [(8, 1 << 20, 20000, 0.5), (8, 1 << 16, 4000, 0.1), (300, 70001, 100, 0.5)])
def test_bench_reduce_matches_plain_call(P, N, k, delta):
    """Sparse and dense results, and more nodes than the offsets carried
    inline to the first kernel (the setup launches then open the span)."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(P * 31 + k)
    idx = np.concatenate([np.sort(rng.choice(N, k, replace=False)) for _ in range(P)]).astype(np.uint32)
    val = rng.standard_normal(P * k).astype(np.float32)
    off = [p * k for p in range(P + 1)]
    di = torch.from_numpy(idx.view(np.int32)).to(dev)
    dv = torch.from_numpy(val).to(dev)
    a = sg.sparse_reduce(off, di, dv, N, delta)
    for op_stop in (False, True):
        e = _events(op_stop=op_stop)
        b = sg.sparse_reduce(off, di, dv, N, delta, events=e)
        torch.cuda.synchronize()
        Ka, da, fa, ia, va = a.host()
        Kb, db, fb, ib, vb = b.host()
        assert (Ka, da, fa) == (Kb, db, fb) and fa == 0
        assert np.array_equal(ia.numpy(), ib.numpy())
        assert_bits_equal(va.numpy(), vb.numpy(), "reduce values")
        span = _ms(e.op_start, e.op_stop or e.kernel_stop)
        writer = _ms(e.kernel_start, e.kernel_stop)
        assert 0.0 < writer <= span + 1e-3, (writer, span)


@pytest.mark.parametrize("P,N,k,delta", [(8, 1 << 20, 5243, 0.3), (4, 4096, 41, 0.3), (300, 70001, 30, 0.5)])
def test_bench_run_table_calls_match_plain_calls(P, N, k, delta):
    """sparcml_bench_topk_ef_runs and sparcml_bench_sparse_reduce_runs give
    the results of the plain calls (the table included), and their spans
    contain their dominant kernels; with the table the reduce's first kernel
    is the count pass (or, past 255 nodes, the setup launches)."""
    dev = torch.device("cuda:0")
    g = torch.from_numpy(np.random.default_rng(P + N).standard_normal((P, N), dtype=np.float32)).to(dev)
    ra, rb = torch.zeros_like(g), torch.zeros_like(g)
    ta = torch.empty(sg.run_table_shape(P, N), dtype=torch.int32, device=dev)
    tb = torch.empty_like(ta)
    ia, va = sg.topk_ef(g, ra, k, runs=ta)
    et = _events()
    ib, vb = sg.topk_ef(g, rb, k, runs=tb, events=et)
    torch.cuda.synchronize()
    assert_bits_equal(ia.cpu().numpy(), ib.cpu().numpy(), "idx")
    assert_bits_equal(va.cpu().numpy(), vb.cpu().numpy(), "val")
    assert_bits_equal(ta.cpu().numpy(), tb.cpu().numpy(), "run table")
    assert _ms(et.op_start, et.op_stop) > 0.0
    off = [p * k for p in range(P + 1)]
    a = sg.sparse_reduce(off, ia.view(-1), va.view(-1), N, delta, runs=ta)
    e = _events(op_stop=False)
    b = sg.sparse_reduce(off, ib.view(-1), vb.view(-1), N, delta, runs=tb, events=e)
    torch.cuda.synchronize()
    Ka, da, fa, xa, ya = a.host()
    Kb, db, fb, xb, yb = b.host()
    assert (Ka, da, fa) == (Kb, db, fb) and fa == 0
    assert np.array_equal(xa.numpy(), xb.numpy())
    assert_bits_equal(ya.numpy(), yb.numpy(), "reduce values")
    writer = _ms(e.kernel_start, e.kernel_stop)
    assert 0.0 < writer <= _ms(e.op_start, e.kernel_stop) + 1e-3


def test_bench_q4_dq4_and_reference_stream():
    dev = torch.device("cuda:0")
    P, n, B = 4, 100003, 512
    v = torch.from_numpy(np.random.default_rng(3).standard_normal((P, n), dtype=np.float32)).to(dev)
    ca, sa = sg.q4(v, B, 99, 5)
    eq = _events(kernel=False)
    cb, sb = sg.q4(v, B, 99, 5, events=eq)
    da = sg.dq4(ca, sa, n, B)
    ed = _events(kernel=False)
    db = sg.dq4(cb, sb, n, B, events=ed)
    torch.cuda.synchronize()
    assert_bits_equal(ca.cpu().numpy(), cb.cpu().numpy(), "codes")
    assert_bits_equal(sa.cpu().numpy(), sb.cpu().numpy(), "scales")
    assert_bits_equal(da.cpu().numpy(), db.cpu().numpy(), "dequantized")
    assert _ms(eq.op_start, eq.op_stop) > 0.0 and _ms(ed.op_start, ed.op_stop) > 0.0

    # the bandwidth reference is a plain r += g
    g = torch.from_numpy(np.random.default_rng(4).standard_normal(1 << 20 | 7, dtype=np.float32)).to(dev)
    r = torch.from_numpy(np.random.default_rng(5).standard_normal(1 << 20 | 7, dtype=np.float32)).to(dev)
    want = (r.cpu() + g.cpu()).numpy()
    e = _events(kernel=False)
    st = sg.bench_lib().sparcml_bench_reference_stream(g.numel(), ctypes.c_void_p(g.data_ptr()),
                                                       ctypes.c_void_p(r.data_ptr()), ctypes.byref(e),
                                                       ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == sg.OK
    torch.cuda.synchronize()
    assert_bits_equal(r.cpu().numpy(), want, "reference stream")
    assert _ms(e.op_start, e.op_stop) > 0.0
