"""CPU oracle for the SparCML hot path (error-feedback Top-k, 4-bit stochastic
quantization, sparse reduction with the dense switch).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by the bench's ``cpu_baseline`` leg, never by the product package. It
shares no code with the HIP path. The arithmetic lives in ``oracle.cpp``; this
module only marshals numpy arrays through ctypes.

Parity status per function (what pins it is in each C function's header):
  topk_ef   pinned (brute force, characterisation, special cases, EF identity)
  topk_ef_layers
            pinned (brute force per layer, the one-layer case equals topk_ef,
            EF identity)
  topk_ef_bucketed
            pinned (brute force per bucket, the one-bucket case equals topk_ef,
            EF identity)
  philox    pinned (rocRAND's Philox-4x32-10 engine, compared in a test)
  q4 / dq4, qsgd / dqsgd (2, 4, 8 bits)
            pinned by invariants, unbiasedness and a recomputation from
            rocRAND's Philox stream; the exact code stream is fixed by the
            reading documented in oracle.cpp
  reduce    pinned (np.bincount / np.unique, overlap extremes, switch at T)
  run_table pinned (brute-force count per node and range, end entries, every
            pair inside its range)
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build(force=True)
        L = ctypes.CDLL(path)
        u32, u64, f64, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        L.oracle_topk_ef.argtypes = [u32, u64, u64, vp, vp, vp, vp]
        L.oracle_topk_ef.restype = None
        L.oracle_topk_ef_layers.argtypes = [u32, u64, u32, vp, vp, vp, vp, vp, vp]
        L.oracle_topk_ef_layers.restype = None
        L.oracle_bucketed_count.argtypes = [u64, u32, u32]
        L.oracle_bucketed_count.restype = u64
        L.oracle_topk_ef_bucketed.argtypes = [u32, u64, u32, u32, vp, vp, vp, vp]
        L.oracle_topk_ef_bucketed.restype = None
        L.oracle_philox4x32_10.argtypes = [vp, vp, vp]
        L.oracle_philox4x32_10.restype = None
        L.oracle_q4.argtypes = [u32, u64, u32, u64, u32, vp, vp, vp]
        L.oracle_q4.restype = None
        L.oracle_dq4.argtypes = [u32, u64, u32, vp, vp, vp]
        L.oracle_dq4.restype = None
        L.oracle_qsgd.argtypes = [u32, u32, u64, u32, u64, u32, u32, vp, vp, vp]
        L.oracle_qsgd.restype = None
        L.oracle_dqsgd.argtypes = [u32, u32, u64, u32, vp, vp, vp]
        L.oracle_dqsgd.restype = None
        L.oracle_reduce.argtypes = [u32, u64, f64, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_run_table.argtypes = [u32, u64, u32, vp, vp, vp]
        L.oracle_run_table.restype = ctypes.c_int
        L.oracle_reduce.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = ctypes.c_int
        _LIB = L
    return _LIB


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def topk_ef(grad, residual, k):
    """grad, residual: [P, N] float32. Returns (idx [P,k] u32, val [P,k] f32,
    r_new [P,N] f32). The inputs are not modified."""
    g = _c(grad, np.float32)
    r = _c(residual, np.float32).copy()
    assert g.ndim == 2 and g.shape == r.shape
    P, N = g.shape
    k = int(k)
    assert 0 <= k <= N
    idx = np.zeros((P, k), np.uint32)
    val = np.zeros((P, k), np.float32)
    lib().oracle_topk_ef(P, N, k, _ptr(g), _ptr(r), _ptr(idx), _ptr(val))
    return idx, val, r


def topk_ef_layers(grad, residual, layer_offsets, ks):
    """Top-k of every layer [off[l], off[l+1]) of every node. grad, residual:
    [P, N] float32. Returns (idx [P, sum k] u32, val, r_new [P, N])."""
    g = _c(grad, np.float32)
    r = _c(residual, np.float32).copy()
    P, N = g.shape
    off = _c(layer_offsets, np.uint64)
    kk = _c(ks, np.uint64)
    nl = kk.size
    assert off.size == nl + 1 and off[0] == 0 and off[-1] == N
    K = int(kk.sum())
    idx = np.zeros((P, K), np.uint32)
    val = np.zeros((P, K), np.float32)
    lib().oracle_topk_ef_layers(P, N, nl, _ptr(off), _ptr(kk), _ptr(g), _ptr(r), _ptr(idx), _ptr(val))
    return idx, val, r


def bucketed_count(N, bucket, k_per_bucket):
    return int(lib().oracle_bucketed_count(int(N), int(bucket), int(k_per_bucket)))


def topk_ef_bucketed(grad, residual, bucket, k_per_bucket):
    """Top-k within every bucket of `bucket` positions. grad, residual: [P, N]
    float32. Returns (idx [P, K] u32, val [P, K] f32, r_new [P, N] f32) with K
    = bucketed_count(N, bucket, k_per_bucket); inputs are not modified."""
    g = _c(grad, np.float32)
    r = _c(residual, np.float32).copy()
    assert g.ndim == 2 and g.shape == r.shape
    P, N = g.shape
    K = bucketed_count(N, bucket, k_per_bucket)
    idx = np.zeros((P, K), np.uint32)
    val = np.zeros((P, K), np.float32)
    lib().oracle_topk_ef_bucketed(P, N, int(bucket), int(k_per_bucket), _ptr(g), _ptr(r), _ptr(idx), _ptr(val))
    return idx, val, r


def philox4x32_10(counter, key):
    c = np.ascontiguousarray(counter, np.uint32)
    kk = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(kk), _ptr(out))
    return out


def q4(val, bucket, seed, step):
    """val: [P, n] float32 -> (codes [P, ceil(n/2)] u8, scales [P, ceil(n/bucket)] f32)."""
    v = _c(val, np.float32)
    P, n = v.shape
    codes = np.zeros((P, (n + 1) // 2), np.uint8)
    scales = np.zeros((P, (n + bucket - 1) // bucket), np.float32)
    lib().oracle_q4(P, n, int(bucket), int(seed), int(step), _ptr(v), _ptr(codes), _ptr(scales))
    return codes, scales


def dq4(codes, scales, n, bucket):
    c = _c(codes, np.uint8)
    s = _c(scales, np.float32)
    P = c.shape[0]
    out = np.zeros((P, n), np.float32)
    lib().oracle_dq4(P, n, int(bucket), _ptr(c), _ptr(s), _ptr(out))
    return out


def qsgd(val, bits, bucket, seed, step, node0=0):
    """val: [P, n] float32, bits in {2, 4, 8}; row r is node node0 + r ->
    (codes [P, ceil(n*bits/8)] u8, scales [P, ceil(n/bucket)] f32)."""
    assert bits in (2, 4, 8)
    v = _c(val, np.float32)
    P, n = v.shape
    codes = np.zeros((P, (n * bits + 7) // 8), np.uint8)
    scales = np.zeros((P, (n + bucket - 1) // bucket), np.float32)
    lib().oracle_qsgd(bits, P, n, int(bucket), int(seed), int(step), int(node0), _ptr(v), _ptr(codes),
                      _ptr(scales))
    return codes, scales


def dqsgd(codes, scales, n, bits, bucket):
    assert bits in (2, 4, 8)
    c = _c(codes, np.uint8)
    s = _c(scales, np.float32)
    P = c.shape[0]
    out = np.zeros((P, n), np.float32)
    lib().oracle_dqsgd(bits, P, n, int(bucket), _ptr(c), _ptr(s), _ptr(out))
    return out


def reduce(offsets, idx, val, N, delta):
    """offsets: [P+1] u64 (node p owns [offsets[p], offsets[p+1])), idx u32, val f32.
    Returns (K, is_dense, out_idx, out_val): dense -> out_idx empty, out_val [N];
    sparse -> out_idx [K] ascending, out_val [K]."""
    off = _c(offsets, np.uint64)
    ii = _c(idx, np.uint32)
    vv = _c(val, np.float32)
    P = off.shape[0] - 1
    out_idx = np.zeros(max(N, 1), np.uint32)
    out_val = np.zeros(max(N, 1), np.float32)
    K = np.zeros(1, np.uint64)
    dense = np.zeros(1, np.uint32)
    rc = lib().oracle_reduce(P, N, float(delta), _ptr(off), _ptr(ii), _ptr(vv), _ptr(K),
                             _ptr(dense), _ptr(out_idx), _ptr(out_val))
    if rc != 0:
        raise ValueError("oracle_reduce: an index is >= N")
    K = int(K[0])
    if dense[0]:
        return K, True, np.zeros(0, np.uint32), out_val[:N].copy()
    return K, False, out_idx[:K].copy(), out_val[:K].copy()


SEGMENT = 4096  # indices per range of a run table


def run_table(offsets, idx, N, seg=SEGMENT):
    """Run table of sorted sparse contributions: [P, S+1] uint32 with
    runs[p, s] = offsets[p] + (node p's pairs with index < s * seg),
    S = ceil(N / seg)."""
    off = _c(offsets, np.uint64)
    ii = _c(idx, np.uint32)
    P = off.shape[0] - 1
    S = (N + seg - 1) // seg
    runs = np.zeros((P, S + 1), np.uint32)
    rc = lib().oracle_run_table(P, N, seg, _ptr(off), _ptr(ii), _ptr(runs))
    if rc != 0:
        raise ValueError("oracle_run_table: an index is >= N")
    return runs
