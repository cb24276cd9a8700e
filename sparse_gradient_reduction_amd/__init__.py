"""MI355X (gfx950) SparCML hot path: error-feedback Top-k, 2/4/8-bit stochastic
quantization and sparse reduction with the dense switch.

Thin ctypes binding over the C ABI in include/sparcml.h: it checks tensor
dtype/device/contiguity, allocates outputs and workspaces with torch, and
passes raw pointers and the current HIP stream. Every step of the path runs
in the HIP kernels of libsparcml.so; there is no CPU fallback. If the library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparcml.so")
BENCH_LIB_PATH = os.path.join(_PKG, "libsparcml_bench.so")

OK, ERR_INVALID_ARG, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
REDUCE_SCRATCH_BYTES = 32 << 20  # SPARCML_REDUCE_SCRATCH_BYTES: static scratch of sparse_reduce_noalloc
FLAG_INDEX_RANGE, FLAG_NOT_ASCENDING = 1, 2

_lib = None


class SparcmlError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _load().sparcml_status_string(status).decode()
        super().__init__(f"{what}: {msg}")
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m sparse_gradient_reduction_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    u32, u64, sz, vp, f64 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_double
    st = ctypes.c_int
    L.sparcml_status_string.argtypes = [st]
    L.sparcml_status_string.restype = ctypes.c_char_p
    L.sparcml_topk_ef_workspace.argtypes = [u32, u64, u64]
    L.sparcml_topk_ef_workspace.restype = sz
    L.sparcml_topk_ef.argtypes = [u32, u64, u64, vp, vp, vp, vp, vp, sz, vp]
    L.sparcml_topk_ef.restype = st
    L.sparcml_topk_ef_runs.argtypes = [u32, u64, u64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sparcml_topk_ef_runs.restype = st
    L.sparcml_topk_ef_layers_workspace.argtypes = [u32, u64, u32, vp, vp]
    L.sparcml_topk_ef_layers_workspace.restype = sz
    L.sparcml_topk_ef_layers.argtypes = [u32, u64, u32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sparcml_topk_ef_layers.restype = st
    L.sparcml_topk_bucketed_count.argtypes = [u64, u32, u32]
    L.sparcml_topk_bucketed_count.restype = u64
    L.sparcml_topk_ef_bucketed.argtypes = [u32, u64, u32, u32, vp, vp, vp, vp, vp]
    L.sparcml_topk_ef_bucketed.restype = st
    L.sparcml_q4.argtypes = [u32, u64, u32, u64, u32, vp, vp, vp, vp]
    L.sparcml_q4.restype = st
    L.sparcml_dq4.argtypes = [u32, u64, u32, vp, vp, vp, vp]
    L.sparcml_dq4.restype = st
    L.sparcml_qsgd.argtypes = [u32, u32, u64, u32, u64, u32, u32, vp, vp, vp, vp]
    L.sparcml_qsgd.restype = st
    L.sparcml_dqsgd.argtypes = [u32, u32, u64, u32, vp, vp, vp, vp]
    L.sparcml_dqsgd.restype = st
    L.sparcml_qsgd_dense_result.argtypes = [u32, u64, u32, u64, u32, u32, vp, vp, vp, vp, vp]
    L.sparcml_qsgd_dense_result.restype = st
    L.sparcml_sparse_reduce_qsgd.argtypes = [u32, u32, u32, u64, f64, vp, vp, vp, vp, u64, vp, vp, vp, vp, sz, vp]
    L.sparcml_sparse_reduce_qsgd.restype = st
    L.sparcml_sparse_reduce_qsgd_runs.argtypes = [u32, u32, u32, u64, f64, vp, vp, vp, vp, vp, u64, vp, vp, vp, vp,
                                                  sz, vp]
    L.sparcml_sparse_reduce_qsgd_runs.restype = st
    L.sparcml_sparse_reduce_workspace.argtypes = [u32, u64, u64]
    L.sparcml_sparse_reduce_workspace.restype = sz
    L.sparcml_sparse_reduce.argtypes = [u32, u64, f64, vp, vp, vp, u64, vp, vp, vp, vp, sz, vp]
    L.sparcml_sparse_reduce.restype = st
    L.sparcml_sparse_reduce_runs.argtypes = [u32, u64, f64, vp, vp, vp, vp, u64, vp, vp, vp, vp, sz, vp]
    L.sparcml_sparse_reduce_runs.restype = st
    L.sparcml_sparse_reduce_union.argtypes = [u32, u64, f64, vp, vp, vp, u64, vp, vp, sz, vp]
    L.sparcml_sparse_reduce_union.restype = st
    L.sparcml_sparse_reduce_sums.argtypes = [u32, u64, f64, vp, vp, vp, vp, u64, vp, vp, vp, vp, sz, vp]
    L.sparcml_sparse_reduce_sums.restype = st
    L.sparcml_sparse_reduce_noalloc.argtypes = [u32, u64, f64, vp, vp, vp, u64, vp, vp, vp, vp]
    L.sparcml_sparse_reduce_noalloc.restype = st
    L.sparcml_estimate_nnz.argtypes = [u32, u64, vp]
    L.sparcml_estimate_nnz.restype = f64
    ev = ctypes.POINTER(BenchEvents)
    L.sparcml_bench_topk_ef.argtypes = [u32, u64, u64, vp, vp, vp, vp, vp, sz, ev, vp]
    L.sparcml_bench_topk_ef.restype = st
    L.sparcml_bench_topk_ef_runs.argtypes = [u32, u64, u64, vp, vp, vp, vp, vp, vp, sz, ev, vp]
    L.sparcml_bench_topk_ef_runs.restype = st
    L.sparcml_bench_qsgd.argtypes = [u32, u32, u64, u32, u64, u32, u32, vp, vp, vp, ev, vp]
    L.sparcml_bench_qsgd.restype = st
    L.sparcml_bench_dqsgd.argtypes = [u32, u32, u64, u32, vp, vp, vp, ev, vp]
    L.sparcml_bench_dqsgd.restype = st
    L.sparcml_bench_sparse_reduce.argtypes = [u32, u64, f64, vp, vp, vp, u64, vp, vp, vp, vp, sz, ev, vp]
    L.sparcml_bench_sparse_reduce.restype = st
    L.sparcml_bench_sparse_reduce_runs.argtypes = [u32, u64, f64, vp, vp, vp, vp, u64, vp, vp, vp, vp, sz, ev, vp]
    L.sparcml_bench_sparse_reduce_runs.restype = st
    L.sparcml_bench_sparse_reduce_union.argtypes = [u32, u64, f64, vp, vp, vp, u64, vp, vp, sz, ev, vp]
    L.sparcml_bench_sparse_reduce_union.restype = st
    L.sparcml_bench_sparse_reduce_sums.argtypes = [u32, u64, f64, vp, vp, vp, vp, u64, vp, vp, vp, vp, sz, ev, vp]
    L.sparcml_bench_sparse_reduce_sums.restype = st
    L.sparcml_bench_sparse_reduce_qsgd_runs.argtypes = [u32, u32, u32, u64, f64, vp, vp, vp, vp, vp, u64, vp, vp, vp,
                                                        vp, sz, ev, vp]
    L.sparcml_bench_sparse_reduce_qsgd_runs.restype = st
    _lib = L
    return L


def lib():
    """The loaded ctypes handle of libsparcml.so."""
    return _load()


class BenchEvents(ctypes.Structure):
    """sparcml_bench_events: HIP events (raw handles, or None) that the
    measurement entry points attach to kernel dispatches."""
    _fields_ = [("op_start", ctypes.c_void_p), ("op_stop", ctypes.c_void_p),
                ("kernel_start", ctypes.c_void_p), ("kernel_stop", ctypes.c_void_p)]


_bench_lib = None


def bench_lib():
    """The loaded ctypes handle of libsparcml_bench.so (measurement only: the
    bandwidth reference kernel)."""
    global _bench_lib
    if _bench_lib is None:
        if not os.path.exists(BENCH_LIB_PATH):
            raise RuntimeError(f"{BENCH_LIB_PATH} is not built; run `python -m sparse_gradient_reduction_amd.build`")
        L = ctypes.CDLL(BENCH_LIB_PATH)
        L.sparcml_bench_reference_stream.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.POINTER(BenchEvents), ctypes.c_void_p]
        L.sparcml_bench_reference_stream.restype = ctypes.c_int
        _bench_lib = L
    return _bench_lib


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} tensor on a GPU")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _raise(status: int, what: str):
    if status != OK:
        raise SparcmlError(status, what)


# ---------------------------------------------------------------------------
def topk_ef_workspace_bytes(P: int, N: int, k: int) -> int:
    return int(_load().sparcml_topk_ef_workspace(P, N, k))


SEGMENT = 4096  # indices per segment of a run table (SPARCML_SEGMENT)


def run_table_shape(P: int, N: int):
    """Shape of the run table of P sorted contributions over N indices."""
    return (P, (N + SEGMENT - 1) // SEGMENT + 1)


def topk_ef(grad: torch.Tensor, residual: torch.Tensor, k: int, out_idx: Optional[torch.Tensor] = None,
            out_val: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            events: Optional[BenchEvents] = None, runs: Optional[torch.Tensor] = None):
    """Error-feedback Top-k on [P, N] fp32 `grad`; `residual` is updated in place.
    Returns (idx [P, k] int32 holding uint32 indices, val [P, k] float32).
    `runs` (int32 tensor of run_table_shape(P, N)) routes the call through
    sparcml_topk_ef_runs, which also writes the run table of the output.
    `events` (measurement only) routes the call through sparcml_bench_topk_ef(_runs)."""
    _check_dev(grad, torch.float32, "grad")
    _check_dev(residual, torch.float32, "residual")
    if grad.dim() != 2 or grad.shape != residual.shape:
        raise ValueError("grad and residual must both be [P, N]")
    P, N = grad.shape
    dev = grad.device
    if out_idx is None:
        out_idx = torch.empty((P, k), dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty((P, k), dtype=torch.float32, device=dev)
    need = topk_ef_workspace_bytes(P, N, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    L = _load()
    s = ctypes.c_void_p(_stream(dev))
    if runs is not None:
        _check_dev(runs, torch.int32, "runs")
        if tuple(runs.shape) != run_table_shape(P, N) or not runs.is_contiguous():
            raise ValueError(f"runs must be a contiguous {run_table_shape(P, N)} tensor")
        if events is None:
            st = L.sparcml_topk_ef_runs(P, N, k, _ptr(grad), _ptr(residual), _ptr(out_idx), _ptr(out_val),
                                        _ptr(runs), _ptr(workspace), workspace.numel(), s)
        else:
            st = L.sparcml_bench_topk_ef_runs(P, N, k, _ptr(grad), _ptr(residual), _ptr(out_idx), _ptr(out_val),
                                              _ptr(runs), _ptr(workspace), workspace.numel(), ctypes.byref(events),
                                              s)
        _raise(st, "sparcml_topk_ef_runs")
        return out_idx, out_val
    if events is None:
        st = L.sparcml_topk_ef(P, N, k, _ptr(grad), _ptr(residual), _ptr(out_idx), _ptr(out_val),
                               _ptr(workspace), workspace.numel(), s)
    else:
        st = L.sparcml_bench_topk_ef(P, N, k, _ptr(grad), _ptr(residual), _ptr(out_idx), _ptr(out_val),
                                     _ptr(workspace), workspace.numel(), ctypes.byref(events), s)
    _raise(st, "sparcml_topk_ef")
    return out_idx, out_val


def _u64s(xs):
    xs = [int(x) for x in xs]
    return (ctypes.c_uint64 * len(xs))(*xs)


def topk_ef_layers_workspace_bytes(P: int, N: int, layer_offsets: Sequence[int], ks: Sequence[int]) -> int:
    return int(_load().sparcml_topk_ef_layers_workspace(P, N, len(ks), _u64s(layer_offsets), _u64s(ks)))


def topk_ef_layers(grad: torch.Tensor, residual: torch.Tensor, layer_offsets: Sequence[int], ks: Sequence[int],
                   out_idx: Optional[torch.Tensor] = None, out_val: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None):
    """Error-feedback Top-k of every layer [off[l], off[l+1]) of every node,
    keeping ks[l] of layer l; `residual` is updated in place. Returns (idx
    [P, sum ks] int32 holding node-relative uint32 indices, val [P, sum ks])."""
    _check_dev(grad, torch.float32, "grad")
    _check_dev(residual, torch.float32, "residual")
    if grad.dim() != 2 or grad.shape != residual.shape:
        raise ValueError("grad and residual must both be [P, N]")
    P, N = grad.shape
    K = sum(int(x) for x in ks)
    dev = grad.device
    if out_idx is None:
        out_idx = torch.empty((P, K), dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty((P, K), dtype=torch.float32, device=dev)
    need = topk_ef_layers_workspace_bytes(P, N, layer_offsets, ks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = _load().sparcml_topk_ef_layers(P, N, len(ks), _u64s(layer_offsets), _u64s(ks), _ptr(grad), _ptr(residual),
                                        _ptr(out_idx), _ptr(out_val), _ptr(workspace), workspace.numel(),
                                        ctypes.c_void_p(_stream(dev)))
    _raise(st, "sparcml_topk_ef_layers")
    return out_idx, out_val


def topk_bucketed_count(N: int, bucket: int, k_per_bucket: int) -> int:
    return int(_load().sparcml_topk_bucketed_count(N, bucket, k_per_bucket))


def topk_ef_bucketed(grad: torch.Tensor, residual: torch.Tensor, bucket: int, k_per_bucket: int,
                     out_idx: Optional[torch.Tensor] = None, out_val: Optional[torch.Tensor] = None):
    """Error-feedback Top-k within every bucket of `bucket` positions (64 ..
    1024, a power of two); `residual` is updated in place. Returns (idx [P, K]
    int32 holding uint32 indices, val [P, K] float32), K = topk_bucketed_count."""
    _check_dev(grad, torch.float32, "grad")
    _check_dev(residual, torch.float32, "residual")
    if grad.dim() != 2 or grad.shape != residual.shape:
        raise ValueError("grad and residual must both be [P, N]")
    P, N = grad.shape
    K = topk_bucketed_count(N, bucket, k_per_bucket)
    dev = grad.device
    if out_idx is None:
        out_idx = torch.empty((P, K), dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty((P, K), dtype=torch.float32, device=dev)
    st = _load().sparcml_topk_ef_bucketed(P, N, bucket, k_per_bucket, _ptr(grad), _ptr(residual), _ptr(out_idx),
                                          _ptr(out_val), ctypes.c_void_p(_stream(dev)))
    _raise(st, "sparcml_topk_ef_bucketed")
    return out_idx, out_val


TOPK_ROW_MAX = 1 << 17  # SPARCML_TOPK_ROW_MAX: rows this short are selected by one workgroup per node ...
TOPK_ROW_TOTAL_MAX = 1 << 24  # SPARCML_TOPK_ROW_TOTAL_MAX: ... in calls of at most this many elements


def topk_ef_paths(workspace: torch.Tensor, P: int) -> torch.Tensor:
    """Per node, which path the last sparcml_topk_ef in `workspace` took
    (0 candidates, 1 exact rescan, 2 one workgroup over a short row), and its
    consistency flag: [2, P] int32."""
    return workspace[: 8 * P].view(torch.int32).view(2, P)


# ---------------------------------------------------------------------------
def q4(val: torch.Tensor, bucket: int, seed: int, step: int, codes: Optional[torch.Tensor] = None,
       scales: Optional[torch.Tensor] = None, events: Optional[BenchEvents] = None):
    """[P, n] fp32 -> (codes [P, ceil(n/2)] uint8, scales [P, ceil(n/bucket)] fp32)."""
    _check_dev(val, torch.float32, "val")
    P, n = val.shape
    dev = val.device
    if codes is None:
        codes = torch.empty((P, (n + 1) // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((P, (n + bucket - 1) // bucket), dtype=torch.float32, device=dev)
    if events is None:
        st = _load().sparcml_q4(P, n, bucket, seed & ((1 << 64) - 1), step, _ptr(val), _ptr(codes), _ptr(scales),
                                ctypes.c_void_p(_stream(dev)))
    else:  # measurement: the same call with events on its kernel
        st = _load().sparcml_bench_qsgd(4, P, n, bucket, seed & ((1 << 64) - 1), step, 0, _ptr(val), _ptr(codes),
                                        _ptr(scales), ctypes.byref(events), ctypes.c_void_p(_stream(dev)))
    _raise(st, "sparcml_q4")
    return codes, scales


def dq4(codes: torch.Tensor, scales: torch.Tensor, n: int, bucket: int, out: Optional[torch.Tensor] = None,
        events: Optional[BenchEvents] = None):
    _check_dev(codes, torch.uint8, "codes")
    _check_dev(scales, torch.float32, "scales")
    P = codes.shape[0]
    if out is None:
        out = torch.empty((P, n), dtype=torch.float32, device=codes.device)
    if events is None:
        st = _load().sparcml_dq4(P, n, bucket, _ptr(codes), _ptr(scales), _ptr(out),
                                 ctypes.c_void_p(_stream(codes.device)))
    else:  # measurement: the same call with events on its kernel
        st = _load().sparcml_bench_dqsgd(4, P, n, bucket, _ptr(codes), _ptr(scales), _ptr(out), ctypes.byref(events),
                                         ctypes.c_void_p(_stream(codes.device)))
    _raise(st, "sparcml_dq4")
    return out


def qsgd_row_bytes(bits: int, n: int) -> int:
    return (n * bits + 7) // 8


def qsgd(val: torch.Tensor, bits: int, bucket: int, seed: int, step: int, node0: int = 0,
         codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """b-bit (2, 4, 8) stochastic quantization of [P, n] fp32; row p is node
    node0 + p. Returns (codes [P, ceil(n*bits/8)] uint8, scales [P, ceil(n/bucket)] fp32)."""
    _check_dev(val, torch.float32, "val")
    P, n = val.shape
    dev = val.device
    if codes is None:
        codes = torch.empty((P, qsgd_row_bytes(bits, n)), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((P, (n + bucket - 1) // bucket), dtype=torch.float32, device=dev)
    st = _load().sparcml_qsgd(bits, P, n, bucket, seed & ((1 << 64) - 1), step, node0, _ptr(val), _ptr(codes),
                              _ptr(scales), ctypes.c_void_p(_stream(dev)))
    _raise(st, "sparcml_qsgd")
    return codes, scales


def dqsgd(codes: torch.Tensor, scales: torch.Tensor, n: int, bits: int, bucket: int,
          out: Optional[torch.Tensor] = None):
    _check_dev(codes, torch.uint8, "codes")
    _check_dev(scales, torch.float32, "scales")
    P = codes.shape[0]
    if out is None:
        out = torch.empty((P, n), dtype=torch.float32, device=codes.device)
    st = _load().sparcml_dqsgd(bits, P, n, bucket, _ptr(codes), _ptr(scales), _ptr(out),
                               ctypes.c_void_p(_stream(codes.device)))
    _raise(st, "sparcml_dqsgd")
    return out


# ---------------------------------------------------------------------------
def dense_threshold(delta: float, N: int) -> int:
    t = math.ceil(delta * float(N))
    return max(0, min(t, N + 1))


def sparse_reduce_workspace_bytes(P: int, N: int, total_nnz: int) -> int:
    return int(_load().sparcml_sparse_reduce_workspace(P, N, total_nnz))


def estimate_nnz(offsets: Sequence[int], N: int) -> float:
    off = (ctypes.c_uint64 * len(offsets))(*[int(x) for x in offsets])
    return float(_load().sparcml_estimate_nnz(len(offsets) - 1, N, off))


class ReduceOutput:
    """Device-resident result of sparse_reduce. `result` is a 16-byte tensor
    holding sparcml_reduce_result; `read()` copies it to the host."""

    def __init__(self, result, out_idx, out_val, N):
        self.result, self.out_idx, self.out_val, self.N = result, out_idx, out_val, N

    def read(self):
        r = self.result.cpu()
        nnz = int(r[:8].view(torch.int64).item())
        is_dense = bool(r[8:12].view(torch.int32).item())
        flags = int(r[12:16].view(torch.int32).item())
        return nnz, is_dense, flags

    def host(self):
        """(K, is_dense, flags, idx, val) as host tensors: dense -> idx empty, val [N];
        sparse -> idx [K] int64, val [K]."""
        K, dense, flags = self.read()
        if dense:
            return K, True, flags, torch.zeros(0, dtype=torch.int64), self.out_val[: self.N].cpu()
        idx = self.out_idx[:K].cpu().to(torch.int64) & 0xFFFFFFFF
        return K, False, flags, idx, self.out_val[:K].cpu()


def _reduce_outputs(offsets, N, delta, dev, out_idx, out_val, result, workspace):
    P = len(offsets) - 1
    T = dense_threshold(delta, N)
    cap = 0 if T == 0 else min(N, T - 1)
    if out_idx is None:
        out_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if out_val is None:
        out_val = torch.empty(N, dtype=torch.float32, device=dev)
    if result is None:
        result = torch.zeros(16, dtype=torch.uint8, device=dev)
    need = sparse_reduce_workspace_bytes(P, N, int(offsets[-1]))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    return out_idx, out_val, result, workspace


def sparse_reduce_qsgd(offsets: Sequence[int], idx: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                       bits: int, bucket: int, N: int, delta: float, expected_nnz_hint: int = 0,
                       out_idx: Optional[torch.Tensor] = None, out_val: Optional[torch.Tensor] = None,
                       result: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, runs: Optional[torch.Tensor] = None,
                       events: Optional[BenchEvents] = None) -> "ReduceOutput":
    """sparse_reduce with node p's values given as b-bit codes: node p's code
    row starts at byte sum_{q<p} ceil(nnz_q*bits/8), its scales at
    sum_{q<p} ceil(nnz_q/bucket) (the layout qsgd writes when every node has
    the same count). `runs` (the run table, as for sparse_reduce) routes the
    call through sparcml_sparse_reduce_qsgd_runs, and with `events`
    (measurement only) through sparcml_bench_sparse_reduce_qsgd_runs."""
    _check_dev(idx, torch.int32, "idx")
    _check_dev(codes, torch.uint8, "codes")
    _check_dev(scales, torch.float32, "scales")
    P = len(offsets) - 1
    off = (ctypes.c_uint64 * (P + 1))(*[int(x) for x in offsets])
    dev = idx.device
    out_idx, out_val, result, workspace = _reduce_outputs(offsets, N, delta, dev, out_idx, out_val, result,
                                                          workspace)
    if runs is not None:
        _check_dev(runs, torch.int32, "runs")
        if tuple(runs.shape) != run_table_shape(P, N):
            raise ValueError(f"runs must be a contiguous {run_table_shape(P, N)} tensor")
        s = ctypes.c_void_p(_stream(dev))
        if events is None:
            st = _load().sparcml_sparse_reduce_qsgd_runs(bits, bucket, P, N, float(delta), off, _ptr(idx), _ptr(codes),
                                                         _ptr(scales), _ptr(runs), int(expected_nnz_hint),
                                                         _ptr(out_idx), _ptr(out_val), _ptr(result), _ptr(workspace),
                                                         workspace.numel(), s)
        else:
            st = _load().sparcml_bench_sparse_reduce_qsgd_runs(bits, bucket, P, N, float(delta), off, _ptr(idx),
                                                               _ptr(codes), _ptr(scales), _ptr(runs),
                                                               int(expected_nnz_hint), _ptr(out_idx), _ptr(out_val),
                                                               _ptr(result), _ptr(workspace), workspace.numel(),
                                                               ctypes.byref(events), s)
        _raise(st, "sparcml_sparse_reduce_qsgd_runs")
        return ReduceOutput(result, out_idx, out_val, N)
    if events is not None:
        raise ValueError("events need the run table (sparcml_bench_sparse_reduce_qsgd_runs)")
    st = _load().sparcml_sparse_reduce_qsgd(bits, bucket, P, N, float(delta), off, _ptr(idx), _ptr(codes),
                                            _ptr(scales), int(expected_nnz_hint), _ptr(out_idx), _ptr(out_val),
                                            _ptr(result), _ptr(workspace), workspace.numel(),
                                            ctypes.c_void_p(_stream(dev)))
    _raise(st, "sparcml_sparse_reduce_qsgd")
    return ReduceOutput(result, out_idx, out_val, N)


def qsgd_dense_result(out: "ReduceOutput", bits: int, bucket: int, seed: int, step: int, node: int = 0,
                      codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """Quantize the reduction's dense result on the device if (and only if)
    it turned out dense; codes/scales are left untouched otherwise. Returns
    (codes [ceil(N*bits/8)] uint8, scales [ceil(N/bucket)] fp32)."""
    N = out.N
    dev = out.out_val.device
    if codes is None:
        codes = torch.zeros(qsgd_row_bytes(bits, N), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.zeros((N + bucket - 1) // bucket, dtype=torch.float32, device=dev)
    _check_dev(codes, torch.uint8, "codes")
    _check_dev(scales, torch.float32, "scales")
    st = _load().sparcml_qsgd_dense_result(bits, N, bucket, seed & ((1 << 64) - 1), step, node, _ptr(out.result),
                                           _ptr(out.out_val), _ptr(codes), _ptr(scales),
                                           ctypes.c_void_p(_stream(dev)))
    _raise(st, "sparcml_qsgd_dense_result")
    return codes, scales


def sparse_reduce(offsets: Sequence[int], idx: torch.Tensor, val: torch.Tensor, N: int, delta: float,
                  expected_nnz_hint: int = 0, out_idx: Optional[torch.Tensor] = None,
                  out_val: Optional[torch.Tensor] = None, result: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, events: Optional[BenchEvents] = None,
                  runs: Optional[torch.Tensor] = None) -> ReduceOutput:
    """Sum of P sparse contributions (node p owns pairs [offsets[p], offsets[p+1])).
    idx: int32 tensor holding uint32 indices, val: float32 tensor. `runs`, the
    run table of these pairs (int32, run_table_shape(P, N), as topk_ef(runs=...)
    writes it), routes the call through sparcml_sparse_reduce_runs. `events`
    (measurement only) routes the call through sparcml_bench_sparse_reduce(_runs)."""
    _check_dev(idx, torch.int32, "idx")
    _check_dev(val, torch.float32, "val")
    P = len(offsets) - 1
    off = (ctypes.c_uint64 * (P + 1))(*[int(x) for x in offsets])
    dev = idx.device
    out_idx, out_val, result, workspace = _reduce_outputs(offsets, N, delta, dev, out_idx, out_val, result,
                                                          workspace)
    if runs is not None:
        _check_dev(runs, torch.int32, "runs")
        if tuple(runs.shape) != run_table_shape(P, N) or not runs.is_contiguous():
            raise ValueError(f"runs must be a contiguous {run_table_shape(P, N)} tensor")
        s = ctypes.c_void_p(_stream(dev))
        if events is None:
            st = _load().sparcml_sparse_reduce_runs(P, N, float(delta), off, _ptr(idx), _ptr(val), _ptr(runs),
                                                    int(expected_nnz_hint), _ptr(out_idx), _ptr(out_val),
                                                    _ptr(result), _ptr(workspace), workspace.numel(), s)
        else:
            st = _load().sparcml_bench_sparse_reduce_runs(P, N, float(delta), off, _ptr(idx), _ptr(val), _ptr(runs),
                                                          int(expected_nnz_hint), _ptr(out_idx), _ptr(out_val),
                                                          _ptr(result), _ptr(workspace), workspace.numel(),
                                                          ctypes.byref(events), s)
        _raise(st, "sparcml_sparse_reduce_runs")
        return ReduceOutput(result, out_idx, out_val, N)
    if events is None:
        st = _load().sparcml_sparse_reduce(P, N, float(delta), off, _ptr(idx), _ptr(val), int(expected_nnz_hint),
                                           _ptr(out_idx), _ptr(out_val), _ptr(result), _ptr(workspace),
                                           workspace.numel(), ctypes.c_void_p(_stream(dev)))
    else:
        st = _load().sparcml_bench_sparse_reduce(P, N, float(delta), off, _ptr(idx), _ptr(val),
                                                 int(expected_nnz_hint), _ptr(out_idx), _ptr(out_val), _ptr(result),
                                                 _ptr(workspace), workspace.numel(), ctypes.byref(events),
                                                 ctypes.c_void_p(_stream(dev)))
    _raise(st, "sparcml_sparse_reduce")
    return ReduceOutput(result, out_idx, out_val, N)


class ReduceUnion:
    """What sparse_reduce_union prepared for sparse_reduce_sums: the call's
    arguments and the device buffers (workspace, result record) it filled."""

    def __init__(self, offsets, off, idx, N, delta, runs, hint, result, workspace):
        self.offsets, self.off, self.idx, self.N, self.delta = offsets, off, idx, N, delta
        self.runs, self.hint, self.result, self.workspace = runs, hint, result, workspace


def _check_runs(runs, P, N):
    _check_dev(runs, torch.int32, "runs")
    if tuple(runs.shape) != run_table_shape(P, N):
        raise ValueError(f"runs must be a contiguous {run_table_shape(P, N)} tensor")


def sparse_reduce_union(offsets: Sequence[int], idx: torch.Tensor, N: int, delta: float,
                        runs: Optional[torch.Tensor] = None, expected_nnz_hint: int = 0,
                        result: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        events: Optional[BenchEvents] = None) -> ReduceUnion:
    """The union phase of the sparse reduce (indices only): run starts, union
    bitmaps and counts, K and the dense decision. sparse_reduce_sums then
    adds the values; together they give sparse_reduce's result."""
    _check_dev(idx, torch.int32, "idx")
    P = len(offsets) - 1
    off = (ctypes.c_uint64 * (P + 1))(*[int(x) for x in offsets])
    dev = idx.device
    if runs is not None:
        _check_runs(runs, P, N)
    if result is None:
        result = torch.zeros(16, dtype=torch.uint8, device=dev)
    if workspace is None:
        need = sparse_reduce_workspace_bytes(P, N, int(offsets[-1]))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    s = ctypes.c_void_p(_stream(dev))
    args = (P, N, float(delta), off, _ptr(idx), _ptr(runs), int(expected_nnz_hint), _ptr(result), _ptr(workspace),
            workspace.numel())
    if events is None:
        st = _load().sparcml_sparse_reduce_union(*args, s)
    else:
        st = _load().sparcml_bench_sparse_reduce_union(*args, ctypes.byref(events), s)
    _raise(st, "sparcml_sparse_reduce_union")
    return ReduceUnion(offsets, off, idx, N, delta, runs, int(expected_nnz_hint), result, workspace)


def sparse_reduce_sums(u: ReduceUnion, val: torch.Tensor, out_idx: Optional[torch.Tensor] = None,
                       out_val: Optional[torch.Tensor] = None,
                       events: Optional[BenchEvents] = None) -> ReduceOutput:
    """The sums phase after sparse_reduce_union (same stream, the indices,
    table and workspace unchanged in between)."""
    _check_dev(val, torch.float32, "val")
    P = len(u.offsets) - 1
    dev = val.device
    out_idx, out_val, result, workspace = _reduce_outputs(u.offsets, u.N, u.delta, dev, out_idx, out_val, u.result,
                                                          u.workspace)
    s = ctypes.c_void_p(_stream(dev))
    args = (P, u.N, float(u.delta), u.off, _ptr(u.idx), _ptr(val), _ptr(u.runs), u.hint, _ptr(out_idx),
            _ptr(out_val), _ptr(result), _ptr(workspace), workspace.numel())
    if events is None:
        st = _load().sparcml_sparse_reduce_sums(*args, s)
    else:
        st = _load().sparcml_bench_sparse_reduce_sums(*args, ctypes.byref(events), s)
    _raise(st, "sparcml_sparse_reduce_sums")
    return ReduceOutput(result, out_idx, out_val, u.N)


def sparse_reduce_noalloc(offsets, idx: torch.Tensor, val: torch.Tensor, N: int, delta: float,
                          out_idx: torch.Tensor, out_val: torch.Tensor, result: torch.Tensor,
                          expected_nnz_hint: int = 0) -> ReduceOutput:
    """sparse_reduce through the allocation-free entry point: the library's
    static per-GPU scratch replaces the workspace, and the caller passes every
    output (out_idx with capacity min(N, T-1), out_val [N], result 16 bytes),
    so nothing is allocated on the device. `offsets` may be a sequence or a
    prepared (ctypes.c_uint64 * (P+1)) array. Calls that overlap in time on
    one GPU share the scratch and race."""
    _check_dev(idx, torch.int32, "idx")
    _check_dev(val, torch.float32, "val")
    _check_dev(out_idx, torch.int32, "out_idx")
    _check_dev(out_val, torch.float32, "out_val")
    _check_dev(result, torch.uint8, "result")
    if isinstance(offsets, ctypes.Array):
        off, P = offsets, len(offsets) - 1
    else:
        P = len(offsets) - 1
        off = (ctypes.c_uint64 * (P + 1))(*[int(x) for x in offsets])
    dev = idx.device
    st = _load().sparcml_sparse_reduce_noalloc(P, N, float(delta), off, _ptr(idx), _ptr(val),
                                               int(expected_nnz_hint), _ptr(out_idx), _ptr(out_val),
                                               _ptr(result), ctypes.c_void_p(_stream(dev)))
    _raise(st, "sparcml_sparse_reduce_noalloc")
    return ReduceOutput(result, out_idx, out_val, N)
