"""The C-ABI libraries on the host (no GPU needed): they load, export every
function include/sparcml.h and include/sparcml_bench.h declare, reject bad
arguments before launching anything, and report a missing device as a HIP
error without aborting."""
import ctypes
import math
import os
import re

import pytest

import sparse_gradient_reduction_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparcml.h")
BENCH_HEADER = os.path.join(ROOT, "include", "sparcml_bench.h")

if not os.path.exists(sg.LIB_PATH):
    pytest.skip("libsparcml.so not built", allow_module_level=True)

FAKE = ctypes.c_void_p(4096)       # never dereferenced: every call below fails validation first
FAKE_ODD = ctypes.c_void_p(4100)   # not 16-byte aligned
FAKE_WS_ODD = ctypes.c_void_p(4096 + 128)  # 16- but not 256-byte aligned


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparcml_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for want in ["sparcml_topk_ef", "sparcml_sparse_reduce", "sparcml_q4", "sparcml_dq4",
                 "sparcml_topk_ef_workspace", "sparcml_sparse_reduce_workspace", "sparcml_status_string"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(sg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_measurement_entry_points_are_exported_apart():
    """The measurement variants of the method's calls come from libsparcml.so;
    the bandwidth reference kernel only from libsparcml_bench.so."""
    names = declared_functions(BENCH_HEADER)
    assert set(names) == {"sparcml_bench_topk_ef", "sparcml_bench_topk_ef_runs", "sparcml_bench_qsgd",
                          "sparcml_bench_dqsgd", "sparcml_bench_sparse_reduce", "sparcml_bench_sparse_reduce_runs",
                          "sparcml_bench_sparse_reduce_qsgd_runs", "sparcml_bench_sparse_reduce_union",
                          "sparcml_bench_sparse_reduce_sums", "sparcml_bench_reference_stream"}
    L = ctypes.CDLL(sg.LIB_PATH)
    B = ctypes.CDLL(sg.BENCH_LIB_PATH)
    for name in names:
        if name == "sparcml_bench_reference_stream":
            assert hasattr(B, name) and not hasattr(L, name)
        else:
            assert hasattr(L, name), name
            # each is the call of the same name plus its events
            assert name.replace("sparcml_bench_", "sparcml_") in declared_functions()
    # no hidden profiling state: nothing else in the method's library is about measurement
    assert not hasattr(L, "sparcml_profile_next_topk") and not hasattr(L, "sparcml_reference_stream")


def test_measurement_entry_points_check_arguments_first():
    L = sg.lib()
    ev = sg.BenchEvents()
    evp = ctypes.byref(ev)
    ws = sg.topk_ef_workspace_bytes(4, 1000, 10)
    assert L.sparcml_bench_topk_ef(0, 1000, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws, evp, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_bench_topk_ef(4, 1000, 10, FAKE_ODD, FAKE, FAKE, FAKE, FAKE, ws, evp, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_bench_topk_ef(4, 1000, 10, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None, None) == sg.ERR_WORKSPACE
    assert L.sparcml_bench_qsgd(3, 1, 100, 512, 1, 0, 0, FAKE, FAKE, FAKE, evp, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_bench_dqsgd(4, 1, 100, 12, FAKE, FAKE, FAKE, evp, None) == sg.ERR_INVALID_ARG
    off = (ctypes.c_uint64 * 3)(0, 100, 200)
    wsr = sg.sparse_reduce_workspace_bytes(2, 1000, 200)
    assert L.sparcml_bench_sparse_reduce(2, 1000, 0.5, off, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE_WS_ODD, wsr,
                                         evp, None) == sg.ERR_WORKSPACE
    assert L.sparcml_bench_sparse_reduce(0, 1000, 0.5, off, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, wsr,
                                         evp, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_bench_topk_ef_runs(4, 1000, 10, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, evp,
                                        None) == sg.ERR_INVALID_ARG
    assert L.sparcml_bench_sparse_reduce_runs(2, 1000, 0.5, off, FAKE, FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, wsr,
                                              evp, None) == sg.ERR_INVALID_ARG
    B = sg.bench_lib()
    assert B.sparcml_bench_reference_stream(1000, FAKE_ODD, FAKE, evp, None) == sg.ERR_INVALID_ARG
    assert B.sparcml_bench_reference_stream((1 << 34) - 1023, FAKE, FAKE, evp, None) == sg.ERR_INVALID_ARG
    assert B.sparcml_bench_reference_stream(0, None, None, None, None) == sg.OK


_NO_DEVICE_CLIENT = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import sparse_gradient_reduction_amd as sg
L, B = sg.lib(), sg.bench_lib()
F = ctypes.c_void_p(1 << 20)  # 16- and 256-byte aligned; never dereferenced on the host
off = (ctypes.c_uint64 * 3)(0, 100, 200)
wt = sg.topk_ef_workspace_bytes(2, 1 << 20, 1000)
wr = sg.sparse_reduce_workspace_bytes(2, 1000, 200)
ev = ctypes.byref(sg.BenchEvents())
calls = {
    "topk_ef": lambda: L.sparcml_topk_ef(2, 1 << 20, 1000, F, F, F, F, F, wt, None),
    "topk_ef_rows": lambda: L.sparcml_topk_ef(2, 4096, 100, F, F, F, F, F, sg.topk_ef_workspace_bytes(2, 4096, 100),
                                              None),
    "topk_ef_runs": lambda: L.sparcml_topk_ef_runs(2, 1 << 20, 1000, F, F, F, F, F, F, wt, None),
    "q4": lambda: L.sparcml_q4(1, 1024, 512, 1, 0, F, F, F, None),
    "dq4": lambda: L.sparcml_dq4(1, 1024, 512, F, F, F, None),
    "sparse_reduce": lambda: L.sparcml_sparse_reduce(2, 1000, 0.5, off, F, F, 0, F, F, F, F, wr, None),
    "sparse_reduce_noalloc": lambda: L.sparcml_sparse_reduce_noalloc(2, 1000, 0.5, off, F, F, 0, F, F, F, None),
    "sparse_reduce_runs": lambda: L.sparcml_sparse_reduce_runs(2, 1000, 0.5, off, F, F, F, 0, F, F, F, F, wr, None),
    "sparse_reduce_union": lambda: L.sparcml_sparse_reduce_union(2, 1000, 0.5, off, F, None, 0, F, F, wr, None),
    "sparse_reduce_sums": lambda: L.sparcml_sparse_reduce_sums(2, 1000, 0.5, off, F, F, None, 0, F, F, F, F, wr, None),
    "sparse_reduce_qsgd_runs": lambda: L.sparcml_sparse_reduce_qsgd_runs(4, 512, 2, 1000, 0.5, off, F, F, F, F, 0, F, F,
                                                                         F, F, wr, None),
    "bench_sparse_reduce": lambda: L.sparcml_bench_sparse_reduce(2, 1000, 0.5, off, F, F, 0, F, F, F, F, wr, ev,
                                                                 None),
    "bench_reference_stream": lambda: B.sparcml_bench_reference_stream(4096, F, F, ev, None),
}
for name, call in calls.items():
    print(name, call(), flush=True)
print("done", flush=True)
"""


def test_launching_call_without_a_device_returns_hip_error():
    """With no visible GPU, calls whose arguments pass every check reach their
    first HIP call and return SPARCML_ERR_HIP; the process goes on and exits
    normally (no abort, no exception out of the library)."""
    import subprocess
    import sys
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    out = subprocess.run([sys.executable, "-c", _NO_DEVICE_CLIENT, ROOT], env=env, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    lines = out.stdout.split()
    assert lines[-1] == "done", out.stdout
    got = dict(zip(lines[0:-1:2], lines[1:-1:2]))
    assert len(got) == 13 and all(v == str(sg.ERR_HIP) for v in got.values()), got


def test_status_strings():
    L = sg.lib()
    for st in range(5):
        s = L.sparcml_status_string(st).decode()
        assert s.startswith("SPARCML")
    assert L.sparcml_status_string(99).decode()


def test_topk_argument_checks():
    L = sg.lib()
    ws = sg.topk_ef_workspace_bytes(4, 1000, 10)
    assert ws > 0
    call = lambda P, N, k, g=FAKE, r=FAKE, oi=FAKE, ov=FAKE, w=FAKE, wb=ws: L.sparcml_topk_ef(
        P, N, k, g, r, oi, ov, w, wb, None)
    assert call(0, 1000, 10) == sg.ERR_INVALID_ARG
    assert call(4, 1000, 1001) == sg.ERR_INVALID_ARG
    assert call(4, 1 << 32, 10) == sg.ERR_INVALID_ARG
    # tile slots: P * ceil((N + 31) / 1024) must stay below 2^24 (one launch dimension)
    assert call(16384, 1024 * 1023 - 30, 10) == sg.ERR_INVALID_ARG  # 1024 slots per node: 2^24 in all
    assert call(16384, 1024 * 1023 - 31, 10, w=None) == sg.ERR_WORKSPACE  # 1023 slots: within the limit
    assert call(4, 1000, 10, g=None) == sg.ERR_INVALID_ARG
    assert call(4, 1000, 10, r=FAKE_ODD) == sg.ERR_INVALID_ARG
    assert call(4, 1000, 10, oi=None) == sg.ERR_INVALID_ARG
    assert call(4, 1000, 10, w=None) == sg.ERR_WORKSPACE
    assert call(4, 1000, 10, w=FAKE_WS_ODD) == sg.ERR_WORKSPACE
    assert call(4, 1000, 10, wb=ws - 1) == sg.ERR_WORKSPACE
    assert sg.topk_ef_workspace_bytes(0, 10, 1) == 0
    assert sg.topk_ef_workspace_bytes(2, 10, 11) == 0


def test_run_table_call_argument_checks():
    """The run-table variants reject a missing table, and Top-k outputs whose
    positions would not fit the table's 32-bit words, before anything else."""
    L = sg.lib()
    ws = sg.topk_ef_workspace_bytes(4, 1000, 10)
    assert L.sparcml_topk_ef_runs(4, 1000, 10, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None) == sg.ERR_INVALID_ARG
    # P * k >= 2^32 - 15: 65535 nodes of 65537 pairs
    assert L.sparcml_topk_ef_runs(65535, 65537, 65537, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                                  None) == sg.ERR_INVALID_ARG
    assert L.sparcml_topk_ef_runs(4, 1000, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, None) == sg.ERR_WORKSPACE
    off = (ctypes.c_uint64 * 3)(0, 5, 9)
    wr = sg.sparse_reduce_workspace_bytes(2, 100, 9)
    f64 = ctypes.c_double
    assert L.sparcml_sparse_reduce_runs(2, 100, f64(0.25), off, FAKE, FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, wr,
                                        None) == sg.ERR_INVALID_ARG
    assert L.sparcml_sparse_reduce_runs(0, 100, f64(0.25), off, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, wr,
                                        None) == sg.ERR_INVALID_ARG
    assert L.sparcml_sparse_reduce_runs(2, 100, f64(0.25), off, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, wr,
                                        None) == sg.ERR_WORKSPACE
    assert L.sparcml_sparse_reduce_qsgd_runs(4, 512, 2, 100, f64(0.25), off, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE,
                                             FAKE, FAKE, wr, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_sparse_reduce_qsgd_runs(3, 512, 2, 100, f64(0.25), off, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE,
                                             FAKE, FAKE, wr, None) == sg.ERR_INVALID_ARG
    ev = ctypes.byref(sg.BenchEvents())
    assert L.sparcml_bench_sparse_reduce_qsgd_runs(4, 512, 2, 100, f64(0.25), off, FAKE, FAKE, FAKE, None, 0, FAKE,
                                                   FAKE, FAKE, FAKE, wr, ev, None) == sg.ERR_INVALID_ARG
    assert sg.run_table_shape(3, 4096 * 5 + 1) == (3, 7)


def test_reduce_phase_argument_checks():
    """The union phase takes no values or outputs; the sums phase checks them."""
    L = sg.lib()
    off = (ctypes.c_uint64 * 3)(0, 5, 9)
    wr = sg.sparse_reduce_workspace_bytes(2, 100, 9)
    f64 = ctypes.c_double
    assert L.sparcml_sparse_reduce_union(0, 100, f64(0.25), off, FAKE, None, 0, FAKE, FAKE, wr,
                                         None) == sg.ERR_INVALID_ARG
    assert L.sparcml_sparse_reduce_union(2, 100, f64(0.25), off, None, None, 0, FAKE, FAKE, wr,
                                         None) == sg.ERR_INVALID_ARG
    assert L.sparcml_sparse_reduce_union(2, 100, f64(0.25), off, FAKE, None, 0, None, FAKE, wr,
                                         None) == sg.ERR_INVALID_ARG
    assert L.sparcml_sparse_reduce_union(2, 100, f64(0.25), off, FAKE, None, 0, FAKE, None, wr,
                                         None) == sg.ERR_WORKSPACE
    assert L.sparcml_sparse_reduce_sums(2, 100, f64(0.25), off, FAKE, None, None, 0, FAKE, FAKE, FAKE, FAKE, wr,
                                        None) == sg.ERR_INVALID_ARG  # no values
    assert L.sparcml_sparse_reduce_sums(2, 100, f64(0.25), off, FAKE, FAKE, None, 0, FAKE, FAKE_ODD, FAKE, FAKE, wr,
                                        None) == sg.ERR_INVALID_ARG  # unaligned out_val


def test_q4_argument_checks():
    L = sg.lib()
    assert L.sparcml_q4(2, 100, 12, 1, 0, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG  # bucket % 8
    assert L.sparcml_q4(2, 100, 0, 1, 0, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_q4(0, 100, 512, 1, 0, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_q4(2, 100, 512, 1, 0, None, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_q4(2, 100, 512, 1, 0, FAKE_ODD, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_dq4(2, 100, 512, FAKE, None, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_q4(2, 0, 512, 1, 0, None, None, None, None) == sg.OK  # nothing to do


def test_reduce_argument_checks():
    L = sg.lib()
    off = (ctypes.c_uint64 * 3)(0, 5, 9)
    ws = sg.sparse_reduce_workspace_bytes(2, 100, 9)
    assert ws > 0
    f64 = ctypes.c_double

    def call(P=2, N=100, delta=0.25, o=off, oi=FAKE, ov=FAKE, res=FAKE, w=FAKE, wb=ws):
        return L.sparcml_sparse_reduce(P, N, f64(delta), o, FAKE, FAKE, 0, oi, ov, res, w, wb, None)

    assert call(delta=float("nan")) == sg.ERR_INVALID_ARG
    assert call(delta=float("inf")) == sg.ERR_INVALID_ARG
    assert call(P=0) == sg.ERR_INVALID_ARG
    assert call(P=1025) == sg.ERR_INVALID_ARG
    assert call(N=0) == sg.ERR_INVALID_ARG
    assert call(o=None) == sg.ERR_INVALID_ARG
    assert call(o=(ctypes.c_uint64 * 3)(0, 5, 4)) == sg.ERR_INVALID_ARG  # decreasing
    assert call(o=(ctypes.c_uint64 * 3)(1, 5, 9)) == sg.ERR_INVALID_ARG  # not starting at 0
    assert call(o=(ctypes.c_uint64 * 3)(0, 5, 2**32 - 15)) == sg.ERR_INVALID_ARG  # too many pairs
    assert call(ov=FAKE_ODD) == sg.ERR_INVALID_ARG
    assert call(oi=None) == sg.ERR_INVALID_ARG
    assert call(res=None) == sg.ERR_INVALID_ARG
    assert call(w=None) == sg.ERR_WORKSPACE
    assert call(w=FAKE_WS_ODD) == sg.ERR_WORKSPACE
    assert call(wb=ws - 1) == sg.ERR_WORKSPACE


def test_reduce_noalloc_rejects_what_exceeds_its_scratch():
    """The allocation-free reduce refuses, before touching any device, a call
    whose workspace would exceed SPARCML_REDUCE_SCRATCH_BYTES, and takes one
    that fits up to its other argument checks."""
    L = sg.lib()
    L.sparcml_sparse_reduce_noalloc.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p]
    assert sg.REDUCE_SCRATCH_BYTES == 32 << 20
    big_P, big_N = 1024, 1 << 27  # the run-start table alone is 4 * 1024 * 32769 bytes
    assert sg.sparse_reduce_workspace_bytes(big_P, big_N, 1000) > sg.REDUCE_SCRATCH_BYTES
    off = (ctypes.c_uint64 * (big_P + 1))(*([0] * (big_P + 1)))
    st = L.sparcml_sparse_reduce_noalloc(big_P, big_N, 0.3, off, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None)
    assert st == sg.ERR_SCRATCH_LIMIT
    assert "SCRATCH" in L.sparcml_status_string(st).decode()
    # the wide-ResNet-sized reduce (64 nodes over 2^27 indices) fits
    assert sg.sparse_reduce_workspace_bytes(64, 1 << 27, 64 * 671088) <= sg.REDUCE_SCRATCH_BYTES
    off = (ctypes.c_uint64 * 2)(0, 10)
    assert L.sparcml_sparse_reduce_noalloc(0, 100, 0.3, off, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None) == \
        sg.ERR_INVALID_ARG
    assert L.sparcml_sparse_reduce_noalloc(1, 100, 0.3, None, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None) == \
        sg.ERR_INVALID_ARG


def test_layers_argument_checks():
    L = sg.lib()
    u64 = lambda *xs: (ctypes.c_uint64 * len(xs))(*xs)
    off, ks = u64(0, 10, 100), u64(2, 5)
    ws = L.sparcml_topk_ef_layers_workspace(2, 100, 2, off, ks)
    assert ws > 0

    def call(P=2, N=100, nl=2, o=off, k=ks, g=FAKE, w=FAKE, wb=ws):
        return L.sparcml_topk_ef_layers(P, N, nl, o, k, g, FAKE, FAKE, FAKE, w, wb, None)

    assert call(P=0) == sg.ERR_INVALID_ARG
    assert call(nl=0) == sg.ERR_INVALID_ARG
    assert call(P=70000) == sg.ERR_INVALID_ARG
    assert call(o=u64(0, 10, 99)) == sg.ERR_INVALID_ARG      # does not end at N
    assert call(o=u64(1, 10, 100)) == sg.ERR_INVALID_ARG     # does not start at 0
    assert call(o=u64(0, 50, 40)) == sg.ERR_INVALID_ARG      # decreasing
    assert call(k=u64(11, 5)) == sg.ERR_INVALID_ARG          # k above the layer size
    assert call(g=None) == sg.ERR_INVALID_ARG
    assert call(g=FAKE_ODD) == sg.ERR_INVALID_ARG
    assert call(w=None) == sg.ERR_WORKSPACE
    assert call(w=FAKE_WS_ODD) == sg.ERR_WORKSPACE
    assert call(wb=ws - 1) == sg.ERR_WORKSPACE
    assert L.sparcml_topk_ef_layers_workspace(0, 100, 2, off, ks) == 0
    assert L.sparcml_topk_ef_layers_workspace(40000, 100, 2, off, ks) == 0   # rows above 65535


def test_bucketed_argument_checks():
    L = sg.lib()
    for b in (0, 32, 100, 2048):
        assert L.sparcml_topk_ef_bucketed(2, 1000, b, 16, FAKE, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
        assert L.sparcml_topk_bucketed_count(1000, b, 16) == 0
    assert L.sparcml_topk_ef_bucketed(0, 1000, 512, 16, FAKE, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_topk_ef_bucketed(2, 1000, 512, 16, None, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_topk_ef_bucketed(2, 1000, 512, 16, FAKE, FAKE, None, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_topk_ef_bucketed(2, 0, 512, 16, None, None, None, None, None) == sg.OK
    assert L.sparcml_topk_bucketed_count(1000, 512, 16) == 32
    assert L.sparcml_topk_bucketed_count(1000, 512, 600) == 1000
    assert L.sparcml_topk_bucketed_count(1000, 64, 3) == 15 * 3 + 3


def test_qsgd_argument_checks():
    L = sg.lib()
    for bits in (0, 1, 3, 16):
        assert L.sparcml_qsgd(bits, 2, 100, 512, 1, 0, 0, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
        assert L.sparcml_dqsgd(bits, 2, 100, 512, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_qsgd(2, 2, 100, 12, 1, 0, 0, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG  # bucket % 8
    assert L.sparcml_qsgd(8, 2, 100, 512, 1, 0, 0xFFFFFFFF, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG  # node range
    assert L.sparcml_qsgd(8, 2, 100, 512, 1, 0, 0, FAKE_ODD, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_qsgd(2, 2, 0, 512, 1, 0, 0, None, None, None, None) == sg.OK  # nothing to do
    assert L.sparcml_qsgd_dense_result(4, 100, 512, 1, 0, 0, None, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_qsgd_dense_result(5, 100, 512, 1, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    assert L.sparcml_qsgd_dense_result(4, 1 << 33, 512, 1, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == sg.ERR_INVALID_ARG
    off = (ctypes.c_uint64 * 3)(0, 5, 9)
    ws = sg.sparse_reduce_workspace_bytes(2, 100, 9)
    f64 = ctypes.c_double

    def red(bits=4, bucket=512, codes=FAKE, scales=FAKE, w=FAKE):
        return L.sparcml_sparse_reduce_qsgd(bits, bucket, 2, 100, f64(0.25), off, FAKE, codes, scales, 0,
                                            FAKE, FAKE, FAKE, w, ws, None)

    assert red(bits=3) == sg.ERR_INVALID_ARG
    assert red(bucket=4) == sg.ERR_INVALID_ARG
    assert red(codes=None) == sg.ERR_INVALID_ARG
    assert red(scales=None) == sg.ERR_INVALID_ARG
    assert red(w=FAKE_WS_ODD) == sg.ERR_WORKSPACE


@pytest.mark.parametrize("P,N,k", [(1, 1000, 10), (8, 1 << 20, 10485), (64, 4096, 0), (3, 17, 17)])
def test_estimate_matches_uniform_closed_form(P, N, k):
    """Appendix B.1 (uniform sampling): E[K] = N(1 - (1 - k/N)^P), never above P*k."""
    offsets = [p * k for p in range(P + 1)]
    got = sg.estimate_nnz(offsets, N)
    want = min(N * (1 - (1 - k / N) ** P), P * k)
    assert math.isclose(got, want, rel_tol=1e-12, abs_tol=1e-9)
    assert got <= P * k + 1e-9


def test_row_limit_matches_header():
    """The binding's short-row limit mirrors SPARCML_TOPK_ROW_MAX."""
    import re
    text = open(os.path.join(ROOT, "include", "sparcml.h")).read()
    m = re.search(r"#define SPARCML_TOPK_ROW_MAX \(1u << (\d+)\)", text)
    assert m and sg.TOPK_ROW_MAX == 1 << int(m.group(1))
    m = re.search(r"#define SPARCML_TOPK_ROW_TOTAL_MAX \(1ull << (\d+)\)", text)
    assert m and sg.TOPK_ROW_TOTAL_MAX == 1 << int(m.group(1))


def test_dense_threshold_reading():
    assert sg.dense_threshold(0.25, 65536) == 16384
    assert sg.dense_threshold(0.3, 1 << 27) == 40265319
    assert sg.dense_threshold(0.0, 10) == 0
    assert sg.dense_threshold(-1.0, 10) == 0
    assert sg.dense_threshold(1.5, 10) == 11


def test_header_is_plain_c_and_links():
    """include/sparcml.h compiles as C99 and a C program links the library and
    gets answers from the calls that need no device (tests/c_abi_client.c)."""
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("gcc or the HIP headers are not available")
    sg.lib()  # the library is built
    libdir = os.path.dirname(sg.LIB_PATH)
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "client")
        subprocess.run([gcc, "-std=c99", "-Wall", "-Werror=implicit-function-declaration", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_abi_client.c"), "-o", exe, "-L" + libdir, "-lsparcml",
                        "-Wl,-rpath," + libdir, "-lm"], check=True, capture_output=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
