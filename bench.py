"""Throughput of the SparCML hot path on one MI355X.

One step = error-feedback Top-k over P gradients -> 4-bit stochastic quantize
-> dequantize -> sparse reduce with the dense switch, on seeded synthetic
data already resident in HBM. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload I] [--no-cpu-baseline]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "sparse-reduce input GB/s & % of HBM peak; top-k sparsify Gelem/s (1 GPU)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, help="0..4; 4 = wide-ResNet (2^27 x 64, q4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-nodes", type=int, default=16, help="nodes in the oracle's timed sample")
    ap.add_argument("--seed", type=int, default=987654321)
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the other workloads' timings (profiling runs: their kernels would mix into the averages)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="copy 1 GiB device-to-device once before warmup (reference for PMC byte counters)")
    return ap.parse_args()


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_stream_wideresnet_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_gradient_reduction_amd", "csrc", f)
                  for f in ("topk_ef.hip", "device_common.hpp")]


def kernel_source_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload_name: str):
    """HBM bytes per k_stream launch from the committed PMC summary, if it was
    taken on this workload with the kernel source as it is now; else None."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    fields = {}
    with open(TRAFFIC_SUMMARY) as fh:
        for line in fh:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != kernel_source_sha256() or fields.get("workload") != workload_name:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class CacheFlush:
    """Evicts the caches before a cold measurement by reading 1 GiB (four
    times the last-level cache) and reducing it to one number: the caches end
    up full of clean lines of this buffer, so the measured op neither hits its
    inputs in cache nor pays for writing back dirty lines left by the flush."""

    def __init__(self, torch, dev, nbytes=1 << 30):
        self.torch = torch
        self.buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        self.out = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        self.torch.sum(self.buf, dim=0, out=self.out)


def med(xs):
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


class HipEvents:
    """Raw HIP events: the measurement entry points (sparcml_bench_*) take
    hipEvent_t handles and attach them to kernel dispatches."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)

    def op_events(self, sg, kernel_pair: bool, op_stop: bool = True):
        """A sparcml_bench_events with fresh events: the op's start (and stop),
        and the dominant kernel's pair when asked for."""
        new = lambda: self.create().value
        return sg.BenchEvents(new(), new() if op_stop else None, new() if kernel_pair else None,
                              new() if kernel_pair else None)

    def span_ms(self, e):
        """First kernel's start to last kernel's end of one op. Where the
        dominant kernel is the op's last (the reduce's writer), its own stop
        event closes the span."""
        return self.elapsed_ms(ctypes.c_void_p(e.op_start), ctypes.c_void_p(e.op_stop or e.kernel_stop))

    def kernel_ms(self, e):
        """The dominant kernel's own duration; without a kernel pair (an op
        that is one kernel, which then carries the op's pair), the op's span."""
        if not e.kernel_start:
            return self.span_ms(e)
        return self.elapsed_ms(ctypes.c_void_p(e.kernel_start), ctypes.c_void_p(e.kernel_stop))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only: the P node contributions live in one "
                                   "GPU's HBM and no collective between GPUs is part of it; run with --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_gradient_reduction_amd as sg
    from sparse_gradient_reduction_amd import workloads as W

    w = W.workload(args.workload)
    dev = torch.device("cuda:0")
    if not w.has_topk:  # already-sparse contributions: the step is the reduce alone
        reduce_only(args, w, sg, W, dev)
        return
    P, N, k = w.P, w.N, w.k
    B = w.q4_bucket
    steps, warmup = args.steps, args.warmup
    print(f"[bench] workload {w.name}: P={P} N={N} k={k} delta={w.delta} q4_bucket={B}", file=sys.stderr, flush=True)

    # ---- resident inputs and buffers -------------------------------------
    pool = [W.gradients(w, s, device=dev) for s in range(2)]  # two fresh gradients, alternated
    residual = torch.zeros((P, N), dtype=torch.float32, device=dev)
    ws_topk = torch.empty(sg.topk_ef_workspace_bytes(P, N, k), dtype=torch.uint8, device=dev)
    idx = torch.empty((P, k), dtype=torch.int32, device=dev)
    val = torch.empty((P, k), dtype=torch.float32, device=dev)
    if B:
        codes = torch.empty((P, (k + 1) // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((P, (k + B - 1) // B), dtype=torch.float32, device=dev)
        dval = torch.empty((P, k), dtype=torch.float32, device=dev)
    offsets = [p * k for p in range(P + 1)]
    T = sg.dense_threshold(w.delta, N)
    red_idx = torch.empty(max(1, min(N, T - 1)), dtype=torch.int32, device=dev)
    red_val = torch.empty(N, dtype=torch.float32, device=dev)
    red_res = torch.zeros(16, dtype=torch.uint8, device=dev)
    ws_red = torch.empty(sg.sparse_reduce_workspace_bytes(P, N, P * k), dtype=torch.uint8, device=dev)
    # the run table of the Top-k output, written by its emit pass and read by the reduce
    runs = torch.empty(sg.run_table_shape(P, N), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    print("[bench] inputs resident", file=sys.stderr, flush=True)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ev = HipEvents()
    lib = sg.lib()
    # per timed step: events on the kernel dispatches of each op (Top-k: the
    # op's span and k_stream's own pair; q4 and dq4: their one kernel; the
    # reduce: its span, closed by the writer's own stop, and the writer's pair)
    # (rows short enough for one workgroup each: Top-k is that one kernel, which carries the op's pair)
    row_path = N <= sg.TOPK_ROW_MAX and P * N <= sg.TOPK_ROW_TOTAL_MAX
    # The reduce runs in its two phases: the union phase (indices only) right
    # after the Top-k, while its output is still in the memory-side cache,
    # and the sums once the values are dequantized. Its time is the sum of
    # the two phases' spans.
    recs = [{"topk": ev.op_events(sg, not row_path), "q4": ev.op_events(sg, False), "dq4": ev.op_events(sg, False),
             "union": ev.op_events(sg, False), "sums": ev.op_events(sg, False)} for _ in range(steps)]

    def step(t, rec=None):
        e = rec or {}
        sg.topk_ef(pool[t % 2], residual, k, out_idx=idx, out_val=val, workspace=ws_topk, events=e.get("topk"),
                   runs=runs)
        u = sg.sparse_reduce_union(offsets, idx.view(-1), N, w.delta, runs=runs, result=red_res, workspace=ws_red,
                                   events=e.get("union"))
        red_in = val
        if B:
            sg.q4(val, B, args.seed, t, codes=codes, scales=scales, events=e.get("q4"))
            sg.dq4(codes, scales, k, B, out=dval, events=e.get("dq4"))
            red_in = dval
        sg.sparse_reduce_sums(u, red_in.view(-1), out_idx=red_idx, out_val=red_val, events=e.get("sums"))

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    for t in range(steps):
        step(warmup + t, recs[t])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_step = 1000.0 * wall / steps
    mean = lambda xs: sum(xs) / len(xs)
    topk_spans = [ev.span_ms(r["topk"]) for r in recs]
    k1_list = sorted(ev.kernel_ms(r["topk"]) for r in recs)
    union_spans = [ev.span_ms(r["union"]) for r in recs]
    writer_list = sorted(ev.span_ms(r["sums"]) for r in recs)  # the sums phase is the writer
    red_spans = [a + b for a, b in zip(union_spans, [ev.span_ms(r["sums"]) for r in recs])]
    t_topk, t_red, t_k1 = mean(topk_spans), mean(red_spans), mean(k1_list)
    t_q4 = mean([ev.span_ms(r["q4"]) for r in recs]) if B else 0.0
    t_dq4 = mean([ev.span_ms(r["dq4"]) for r in recs]) if B else 0.0
    # the GPU's own clock from the step's first dispatch to its last kernel's end
    step_list = sorted(ev.elapsed_ms(ctypes.c_void_p(r["topk"].op_start), ctypes.c_void_p(r["sums"].op_stop))
                       for r in recs)
    t_gpu_step = mean(step_list)
    K, is_dense, flags = sg.ReduceOutput(red_res, red_idx, red_val, N).read()  # the timed steps' result

    # ---- reduce alone, cold (caches flushed by a 1 GiB read) and warm --------
    def time_reduce(cold, reps=10, table=True):
        flush = CacheFlush(torch, dev) if cold else None
        rr = [ev.op_events(sg, True, op_stop=False) for _ in range(reps)]
        for e in rr:
            if cold:
                flush()
            sg.sparse_reduce(offsets, idx.view(-1), red_in_last.view(-1), N, w.delta, out_idx=red_idx,
                             out_val=red_val, result=red_res, workspace=ws_red, events=e,
                             runs=runs if table else None)
        torch.cuda.synchronize()
        return sorted(ev.span_ms(e) for e in rr), sorted(ev.kernel_ms(e) for e in rr)

    red_in_last = dval if B else val
    red_cold, red_cold_writer = time_reduce(True)
    red_warm, red_warm_writer = time_reduce(False)
    red_own_cold, _ = time_reduce(True, table=False)  # the reduce finding the runs itself (bounds pass)

    def time_ops(fn, reps=10):
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        fn()
        for a, b in e:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return med(sorted(a.elapsed_time(b) for a, b in e))

    extra = {}
    if B:
        # dequantization fused into the reduce's loader, against dq4 + reduce
        def unfused():
            sg.dq4(codes, scales, k, B, out=dval)
            sg.sparse_reduce(offsets, idx.view(-1), dval.view(-1), N, w.delta, out_idx=red_idx, out_val=red_val,
                             result=red_res, workspace=ws_red)

        def fused():
            sg.sparse_reduce_qsgd(offsets, idx.view(-1), codes.view(-1), scales.view(-1), 4, B, N, w.delta,
                                  out_idx=red_idx, out_val=red_val, result=red_res, workspace=ws_red)

        t_unf, t_fus = time_ops(unfused), time_ops(fused)
        fused_in = P * k * 4.5 + 4 * P * ((k + B - 1) // B)
        extra["fused_dq4_reduce"] = {"unfused_ms": round(t_unf, 4), "fused_ms": round(t_fus, 4),
                                     "fused_input_gb_per_s": round(fused_in / (t_fus * 1e-3) / 1e9, 2)}
        # b-bit QSGD of the same sent values (2, 4 and 8 bits) and the reduce over its codes
        nsc = (k + B - 1) // B
        for bits in (2, 4, 8):
            cb = torch.empty((P, sg.qsgd_row_bytes(bits, k)), dtype=torch.uint8, device=dev)
            sb = torch.empty((P, nsc), dtype=torch.float32, device=dev)
            t_q = time_ops(lambda: sg.qsgd(val, bits, B, args.seed, 1, codes=cb, scales=sb))
            t_r = time_ops(lambda: sg.sparse_reduce_qsgd(offsets, idx.view(-1), cb.view(-1), sb.view(-1), bits, B, N,
                                                         w.delta, out_idx=red_idx, out_val=red_val, result=red_res,
                                                         workspace=ws_red))
            q_bytes = P * k * 4 + P * sg.qsgd_row_bytes(bits, k) + 4 * P * nsc
            r_in = P * k * 4 + P * sg.qsgd_row_bytes(bits, k) + 4 * P * nsc
            extra[f"qsgd_{bits}bit"] = {"quantize_ms": round(t_q, 4),
                                        "quantize_gb_per_s": round(q_bytes / (t_q * 1e-3) / 1e9, 1),
                                        "fused_reduce_ms": round(t_r, 4),
                                        "fused_reduce_input_gb_per_s": round(r_in / (t_r * 1e-3) / 1e9, 1)}
            del cb, sb
    # the dense phase: a reduce whose result turns dense (delta lowered below K / N), then
    # 4-bit quantization of the dense sum in buckets of 1024, gated on the device
    delta_d = 0.25
    red_idx_d = torch.empty(max(1, min(N, sg.dense_threshold(delta_d, N) - 1)), dtype=torch.int32, device=dev)
    dcodes = torch.empty(sg.qsgd_row_bytes(4, N), dtype=torch.uint8, device=dev)
    dscales = torch.empty((N + 1023) // 1024, dtype=torch.float32, device=dev)
    holder = {}

    def dense_reduce():
        holder["out"] = sg.sparse_reduce(offsets, idx.view(-1), red_in_last.view(-1), N, delta_d, out_idx=red_idx_d,
                                         out_val=red_val, result=red_res, workspace=ws_red)

    t_dred = time_ops(dense_reduce)
    t_dq = time_ops(lambda: sg.qsgd_dense_result(holder["out"], 4, 1024, args.seed, 0, 0, codes=dcodes,
                                                 scales=dscales))
    dK, d_is_dense, _ = holder["out"].read()
    extra["dense_phase"] = {"delta": delta_d, "dense": d_is_dense, "reduce_ms": round(t_dred, 4),
                            "q4_dense_result_ms": round(t_dq, 4),
                            "q4_dense_gb_per_s": round((4 * N + N / 2 + 4 * ((N + 1023) // 1024)) / (t_dq * 1e-3) / 1e9,
                                                       1)}
    del red_idx_d, dcodes, dscales

    # ---- bucketed Top-k (16 of every 512) on the same gradients and residual --
    if w.has_topk:
        Kb = sg.topk_bucketed_count(N, 512, 16)
        b_idx = torch.empty((P, Kb), dtype=torch.int32, device=dev)
        b_val = torch.empty((P, Kb), dtype=torch.float32, device=dev)
        t_b = time_ops(lambda: sg.topk_ef_bucketed(pool[0], residual, 512, 16, out_idx=b_idx, out_val=b_val), reps=5)
        b_bytes = 12 * P * N + 8 * P * Kb
        extra["bucketed_topk_16_of_512"] = {"ms": round(t_b, 4), "gelem_per_s": round(P * N / (t_b * 1e-3) / 1e9, 1),
                                           "gb_per_s": round(b_bytes / (t_b * 1e-3) / 1e9, 1),
                                           "frac_hbm_peak": round(b_bytes / (t_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del b_idx, b_val
        # the same density (1 in 32) in the smallest buckets, several buckets per wave
        for bs, kb in ((64, 2), (128, 4)):
            Kb = sg.topk_bucketed_count(N, bs, kb)
            b_idx = torch.empty((P, Kb), dtype=torch.int32, device=dev)
            b_val = torch.empty((P, Kb), dtype=torch.float32, device=dev)
            t_b = time_ops(lambda: sg.topk_ef_bucketed(pool[0], residual, bs, kb, out_idx=b_idx, out_val=b_val),
                           reps=5)
            b_bytes = 12 * P * N + 8 * P * Kb
            extra[f"bucketed_topk_{kb}_of_{bs}"] = {"ms": round(t_b, 4),
                                                    "gb_per_s": round(b_bytes / (t_b * 1e-3) / 1e9, 1),
                                                    "frac_hbm_peak": round(b_bytes / (t_b * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                                                           4)}
            del b_idx, b_val

    # ---- per-layer Top-k (1% of each of 160 layers) on the same arrays ------
    if w.has_topk:
        off_l = W.layer_offsets(N, 160)
        ks_l = W.layer_ks(off_l, 1, 100)
        Kl = int(ks_l.sum())
        l_idx = torch.empty((P, Kl), dtype=torch.int32, device=dev)
        l_val = torch.empty((P, Kl), dtype=torch.float32, device=dev)
        l_ws = torch.empty(sg.topk_ef_layers_workspace_bytes(P, N, off_l, ks_l), dtype=torch.uint8, device=dev)
        t_l = time_ops(lambda: sg.topk_ef_layers(pool[1], residual, off_l, ks_l, out_idx=l_idx, out_val=l_val,
                                                 workspace=l_ws), reps=5)
        l_bytes = 12 * P * N + 8 * P * Kl
        extra["layers_topk_1pct_of_160"] = {"ms": round(t_l, 4), "gelem_per_s": round(P * N / (t_l * 1e-3) / 1e9, 1),
                                            "gb_per_s": round(l_bytes / (t_l * 1e-3) / 1e9, 1),
                                            "frac_hbm_peak": round(l_bytes / (t_l * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                            "rescan_rows": int((l_ws[: 4 * P * 160].view(torch.int32) == 1).sum())}
        del l_idx, l_val, l_ws

    # ---- attainable-bandwidth ceiling: plain torch streaming kernels on [P][N]
    scratch = torch.empty_like(residual)
    def time_torch(fn, reps=5):
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        fn()
        for a, b in e:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return min(a.elapsed_time(b) for a, b in e)

    t_copy = time_torch(lambda: scratch.copy_(residual))
    t_add = time_torch(lambda: torch.add(pool[0], residual, out=scratch))
    # the library's plain streaming add with the stream kernel's access pattern, timed like k_stream
    ref_ev = [ev.op_events(sg, False) for _ in range(5)]
    stream_h = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for e in [ref_ev[0]] + ref_ev:
        st = sg.bench_lib().sparcml_bench_reference_stream(P * N, ctypes.c_void_p(pool[0].data_ptr()),
                                                           ctypes.c_void_p(scratch.data_ptr()), ctypes.byref(e),
                                                           stream_h)
        assert st == 0, st
    torch.cuda.synchronize()
    t_ref = min(ev.span_ms(e) for e in ref_ev)
    del scratch

    paths = sg.topk_ef_paths(ws_topk, P).cpu()
    assert flags == 0 and int(paths[1].abs().sum()) == 0

    # algorithmic bytes per step
    nb = (k + B - 1) // B if B else 0
    b_topk = 12 * P * N + 8 * P * k
    b_q4 = P * k * 4.5 + 4 * P * nb if B else 0  # read values, write codes and scales
    b_dq4 = b_q4                                 # read codes and scales, write values
    b_red_in = 8 * P * k
    b_red_out = 4 * N if is_dense else 8 * K
    b_step = b_topk + b_q4 + b_dq4 + b_red_in + b_red_out
    k1_bytes = 12 * P * N
    k1_gbs = k1_bytes / (t_k1 * 1e-3) / 1e9
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    frac = lambda nbytes, ms: round(gbs(nbytes, ms) / HBM_PEAK_GBS, 4)

    out = {
        "metric": METRIC,
        "value": round(gbs(b_step, ms_step), 2),
        "value_is": "whole-step algorithmic GB/s: the bytes one step's ops must move (Top-k EF, q4, dq4, reduce "
                    "input and output) over the wall-clock time per step; the metric's own parts follow as "
                    "reduce_*, topk_* and q4_*",
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded gradients resident in HBM; no dataset)",
        "config": {"workload": w.name, "P": P, "N": N, "k": k, "delta": w.delta, "q4_bucket": B,
                   "ef_steps": "carried across all timed steps", "parallelism": "none (1 GPU)"},
        # the metric's parts, each from events on its ops' own kernel dispatches in the timed steps
        "reduce_input_gb_per_s": round(gbs(b_red_in, t_red), 2),
        "reduce_gb_per_s": round(gbs(b_red_in + b_red_out, t_red), 2),
        "reduce_frac_hbm_peak": frac(b_red_in + b_red_out, t_red),
        "topk_gelem_per_s": round(P * N / (t_topk * 1e-3) / 1e9, 2),
        "topk_gb_per_s": round(gbs(b_topk, t_topk), 2),
        "topk_frac_hbm_peak": frac(b_topk, t_topk),
        "q4_gb_per_s": round(gbs(b_q4, t_q4), 2) if B else None,
        "q4_frac_hbm_peak": frac(b_q4, t_q4) if B else None,
        "dq4_gb_per_s": round(gbs(b_dq4, t_dq4), 2) if B else None,
        "dq4_frac_hbm_peak": frac(b_dq4, t_dq4) if B else None,
        "breakdown_ms": {"what": "mean over the timed steps of each op's span on the GPU clock: its first "
                                 "kernel's start to its last kernel's end (events attached to the dispatches); "
                                 "the reduce runs as its union phase right after the Top-k and its sums phase "
                                 "after dq4, and its time is the sum of the two spans",
                         "topk_ef": round(t_topk, 4), "q4": round(t_q4, 4), "dq4": round(t_dq4, 4),
                         "sparse_reduce": round(t_red, 4), "reduce_union": round(mean(union_spans), 4),
                         "reduce_sums": round(mean(writer_list), 4), "gpu_step": round(t_gpu_step, 4),
                         "between_ops": round(t_gpu_step - t_topk - t_q4 - t_dq4 - t_red, 4),
                         "k_stream": round(t_k1, 4), "reduce_writer": round(mean(writer_list), 4)},
        "step_gpu_ms_median_min": [round(med(step_list), 4), round(step_list[0], 4)],
        "step_frac_hbm_peak": frac(b_step, t_gpu_step),
        "algorithmic_bytes": {"topk_ef": b_topk, "q4": b_q4, "dq4": b_dq4, "reduce_in": b_red_in,
                              "reduce_out": b_red_out, "step": b_step},
        "reduce_alone_ms": {"what": "the reduce of the last step's pairs repeated alone, its span from dispatch "
                                    "events, with the Top-k's run table as in the step; cold = after a 1 GiB "
                                    "read that flushes the caches; own_runs = without the table (the reduce's "
                                    "own pass over the indices finds the runs)",
                            "cold_median": round(med(red_cold), 4), "cold_min": round(red_cold[0], 4),
                            "warm_median": round(med(red_warm), 4), "warm_min": round(red_warm[0], 4),
                            "cold_writer_median": round(med(red_cold_writer), 4),
                            "cold_input_gb_per_s": round(gbs(b_red_in, med(red_cold)), 2),
                            "cold_frac_hbm_peak": frac(b_red_in + b_red_out, med(red_cold)),
                            "own_runs_cold_median": round(med(red_own_cold), 4),
                            "own_runs_cold_frac_hbm_peak": frac(b_red_in + b_red_out, med(red_own_cold))},
        "reduce_result": {"nnz": K, "dense": is_dense},
        **extra,
        "topk_rescan_nodes": int((paths[0] == 1).sum()),
        "roofline": {"kernel": ("k_topk_row (one workgroup per node: accumulate, select, emit)" if row_path else
                               "k_stream (error-feedback accumulate + candidate compaction)"),
                     "bound": "hbm", "achieved": round(k1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k1_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name),
                     "avg_launch_ms": round(t_k1, 4), "median_min_launch_ms": [round(med(k1_list), 4),
                                                                              round(k1_list[0], 4)],
                     "algorithmic_bytes": k1_bytes},
        "streaming_ceiling": {"what": "torch copy/add and the plain streaming add of libsparcml_bench.so (the "
                                      "stream kernel's access pattern, no candidates) on the same [P][N] fp32 "
                                      "arrays, best of 5",
                              "copy_gb_per_s": round(8 * P * N / (t_copy * 1e-3) / 1e9, 1),
                              "add_gb_per_s": round(12 * P * N / (t_add * 1e-3) / 1e9, 1),
                              "k_stream_over_add": round(t_add / t_k1, 4),
                              "reference_stream_gb_per_s": round(12 * P * N / (t_ref * 1e-3) / 1e9, 1),
                              "k_stream_over_reference": round(t_ref / t_k1, 4)},
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, pool[0], args, sg)
    if not args.no_other_configs:
        del pool, residual, ws_topk, idx, val, red_idx, red_val, ws_red, runs
        if B:
            del codes, scales, dval
        torch.cuda.synchronize()
        out["other_configs"] = other_configs(sg, W, dev, w.wid, ev)
    print(json.dumps(out), flush=True)


def reduce_only(args, w, sg, W, dev):
    """The step of a workload whose contributions are already sparse (Zipf
    feature indices): the sparse reduce alone over its seeded pairs, timed
    like the Top-k step's reduce (events on its own kernel dispatches)."""
    import numpy as np
    import torch

    P, N = w.P, w.N
    o, i_np, v_np = W.zipf_sparse(w)
    off = [int(x) for x in o]
    idx = torch.from_numpy(i_np.view(np.int32)).to(dev)
    val = torch.from_numpy(v_np).to(dev)
    T = sg.dense_threshold(w.delta, N)
    ri = torch.empty(max(1, min(N, T - 1)), dtype=torch.int32, device=dev)
    rv = torch.empty(N, dtype=torch.float32, device=dev)
    rr = torch.zeros(16, dtype=torch.uint8, device=dev)
    wr = torch.empty(sg.sparse_reduce_workspace_bytes(P, N, off[-1]), dtype=torch.uint8, device=dev)
    ev = HipEvents()
    run = lambda e=None: sg.sparse_reduce(off, idx, val, N, w.delta, out_idx=ri, out_val=rv, result=rr,
                                          workspace=wr, events=e)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    recs = [ev.op_events(sg, True, op_stop=False) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in recs:
        run(e)
    torch.cuda.synchronize()
    ms_step = 1000.0 * (time.perf_counter() - t0) / args.steps
    spans = sorted(ev.span_ms(e) for e in recs)
    writer = sorted(ev.kernel_ms(e) for e in recs)
    t_red = sum(spans) / len(spans)
    K, dense, flags = sg.ReduceOutput(rr, ri, rv, N).read()
    assert flags == 0
    b_in, b_out = 8 * off[-1], (4 * N if dense else 8 * K)
    gbs = lambda nbytes, t: nbytes / (t * 1e-3) / 1e9
    t_w = sum(writer) / len(writer)
    print(json.dumps({
        "metric": METRIC, "value": round(gbs(b_in, ms_step), 2),
        "value_is": "sparse-reduce input GB/s over the wall-clock time per step (the step is the reduce alone)",
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded Zipf feature indices, N(0,1) values, resident in HBM)",
        "config": {"workload": w.name, "P": P, "N": N, "pairs": off[-1], "delta": w.delta, "parallelism": "none (1 GPU)"},
        "reduce_input_gb_per_s": round(gbs(b_in, t_red), 2),
        "reduce_gb_per_s": round(gbs(b_in + b_out, t_red), 2),
        "reduce_frac_hbm_peak": round(gbs(b_in + b_out, t_red) / HBM_PEAK_GBS, 4),
        "breakdown_ms": {"what": "mean span of the reduce on the GPU clock (first kernel's start to the writer's "
                                 "end) and of its writer alone", "sparse_reduce": round(t_red, 4),
                         "reduce_writer": round(t_w, 4)},
        "reduce_result": {"nnz": K, "dense": dense},
        "roofline": {"kernel": "reduce writer", "bound": "hbm", "achieved": round(gbs(b_in + b_out, t_w), 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs(b_in + b_out, t_w) / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_ms": round(t_w, 4), "algorithmic_bytes": b_in + b_out},
        "cpu_baseline": None,
    }), flush=True)


def other_configs(sg, W, dev, skip_wid, ev):
    """The other workloads at their full sizes, outside the timed steps: the
    median per-step span of Top-k EF and of the reduce of its pairs over the
    workload's error-feedback steps (from a zero residual), or of the reduce
    alone for the already-sparse workload, each with its algorithmic bytes.
    Spans come from events on the ops' own kernel dispatches; `cold` runs each
    op after a 1 GiB read that flushes the caches (the headline
    figures), `warm` right after the previous op. Also the same step (or
    reduce) captured once as a HIP graph and replayed, which removes the
    launch gaps that dominate the small workloads."""
    import numpy as np
    import torch

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]

    def graph_ms(fn, reps=10):
        """fn captured once as a HIP graph (after a warm-up on a side stream of
        default priority), then the median time of a replay."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        graph.replay()
        tev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in tev:
            a.record()
            graph.replay()
            b.record()
        torch.cuda.synchronize()
        del graph
        return med([a.elapsed_time(b) for a, b in tev])

    flush = CacheFlush(torch, dev)
    res = {}
    for wi in range(5):
        w = W.workload(wi)
        if w.wid == skip_wid:
            continue
        P, N, k = w.P, w.N, w.k
        T = sg.dense_threshold(w.delta, N)
        if not w.has_topk:  # already-sparse contributions: the reduce alone
            o, i_np, v_np = W.zipf_sparse(w)
            off = [int(x) for x in o]
            ii = torch.from_numpy(i_np.view(np.int32)).to(dev)
            vv = torch.from_numpy(v_np).to(dev)
            ri = torch.empty(max(1, min(N, T - 1)), dtype=torch.int32, device=dev)
            rv = torch.empty(N, dtype=torch.float32, device=dev)
            rr = torch.zeros(16, dtype=torch.uint8, device=dev)
            wr = torch.empty(sg.sparse_reduce_workspace_bytes(P, N, off[-1]), dtype=torch.uint8, device=dev)
            run = lambda e=None: sg.sparse_reduce(off, ii, vv, N, w.delta, out_idx=ri, out_val=rv, result=rr,
                                                  workspace=wr, events=e)
            run()
            spans = {}
            for mode in ("cold", "warm"):
                es = [ev.op_events(sg, True, op_stop=False) for _ in range(10)]
                for e in es:
                    if mode == "cold":
                        flush()
                    run(e)
                torch.cuda.synchronize()
                spans[mode] = med([ev.span_ms(e) for e in es])
            t = spans["cold"]
            K, dense, flags = sg.ReduceOutput(rr, ri, rv, N).read()
            b_in, b_out = 8 * off[-1], (4 * N if dense else 8 * K)
            res[w.name] = {"reduce_ms": round(t, 4), "reduce_warm_ms": round(spans["warm"], 4), "pairs": off[-1],
                           "nnz": K, "dense": dense,
                           "reduce_input_gb_per_s": round(b_in / (t * 1e-3) / 1e9, 1),
                           "reduce_frac_hbm_peak": round((b_in + b_out) / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "reduce_graph_ms": round(graph_ms(run), 4)}
            continue
        grads = [W.gradients(w, t, device=dev) for t in range(w.steps)]
        r = torch.zeros((P, N), dtype=torch.float32, device=dev)
        ws = torch.empty(sg.topk_ef_workspace_bytes(P, N, k), dtype=torch.uint8, device=dev)
        idx = torch.empty((P, k), dtype=torch.int32, device=dev)
        val = torch.empty((P, k), dtype=torch.float32, device=dev)
        off = [p * k for p in range(P + 1)]
        ri = torch.empty(max(1, min(N, T - 1)), dtype=torch.int32, device=dev)
        rv = torch.empty(N, dtype=torch.float32, device=dev)
        rr = torch.zeros(16, dtype=torch.uint8, device=dev)
        wr = torch.empty(sg.sparse_reduce_workspace_bytes(P, N, P * k), dtype=torch.uint8, device=dev)
        runs = torch.empty(sg.run_table_shape(P, N), dtype=torch.int32, device=dev)  # Top-k -> reduce
        t_topk = {"cold": [], "warm": []}
        t_red = {"cold": [], "warm": []}
        per_step = []
        for mode in ("warm-up", "warm", "cold"):  # each pass from a zero residual over the EF steps
            r.zero_()
            for t in range(w.steps):
                et, er = ev.op_events(sg, True), ev.op_events(sg, True, op_stop=False)
                if mode == "cold":
                    flush()
                sg.topk_ef(grads[t], r, k, out_idx=idx, out_val=val, workspace=ws, events=et, runs=runs)
                if mode == "cold":
                    flush()
                sg.sparse_reduce(off, idx.view(-1), val.view(-1), N, w.delta, out_idx=ri, out_val=rv, result=rr,
                                 workspace=wr, events=er, runs=runs)
                if mode == "warm-up":
                    continue
                torch.cuda.synchronize()
                t_topk[mode].append(ev.span_ms(et))
                t_red[mode].append(ev.span_ms(er))
                if mode == "cold":
                    K, dense, flags = sg.ReduceOutput(rr, ri, rv, N).read()
                    per_step.append({"nnz": K, "dense": dense})
        torch.cuda.synchronize()
        tk, tr = med(t_topk["cold"]), med(t_red["cold"])

        def one_step():
            sg.topk_ef(grads[0], r, k, out_idx=idx, out_val=val, workspace=ws, runs=runs)
            sg.sparse_reduce(off, idx.view(-1), val.view(-1), N, w.delta, out_idx=ri, out_val=rv, result=rr,
                             workspace=wr, runs=runs)

        t_graph = graph_ms(one_step)  # the residual keeps accumulating: EF steps on the first gradient
        # the same rows as 20 layers (sizes log-uniform), the same fraction kept per layer
        lo = W.layer_offsets(N, 20)
        lks = W.layer_ks(lo, k, N)
        wl = torch.empty(sg.topk_ef_layers_workspace_bytes(P, N, lo, lks), dtype=torch.uint8, device=dev)
        li = torch.empty((P, int(lks.sum())), dtype=torch.int32, device=dev)
        lv = torch.empty((P, int(lks.sum())), dtype=torch.float32, device=dev)
        layers_call = lambda: sg.topk_ef_layers(grads[0], r, lo, lks, out_idx=li, out_val=lv, workspace=wl)
        layers_call()
        tev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for a, b in tev:
            a.record()
            layers_call()
            b.record()
        torch.cuda.synchronize()
        t_layers = med([a.elapsed_time(b) for a, b in tev])
        del wl, li, lv
        b_topk = 12 * P * N + 8 * P * k
        b_in = 8 * P * k
        b_out = [4 * N if s["dense"] else 8 * s["nnz"] for s in per_step]
        res[w.name] = {"steps": w.steps, "topk_ms": round(tk, 4), "reduce_ms": round(tr, 4),
                       "topk_warm_ms": round(med(t_topk["warm"]), 4), "reduce_warm_ms": round(med(t_red["warm"]), 4),
                       "topk_gelem_per_s": round(P * N / (tk * 1e-3) / 1e9, 1),
                       "topk_frac_hbm_peak": round(b_topk / (tk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "reduce_input_gb_per_s": round(b_in / (tr * 1e-3) / 1e9, 1),
                       "reduce_frac_hbm_peak": round((b_in + med(b_out)) / (tr * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "step_graph_ms": round(t_graph, 4),
                       "topk_20_layers_ms": round(t_layers, 4),
                       "per_step": per_step}
        del grads, r, ws, idx, val, ri, rv, rr, wr, runs
        torch.cuda.synchronize()
    del flush
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, g_dev, args, sg):
    """The oracle, untuned, on a bounded sample of the same step: Top-k of
    `cpu_nodes` nodes (full N each), q4/dq4 of their sent values and the
    reduce of their pairs, timed on the host's cores."""
    import numpy as np

    import oracle

    S = min(args.cpu_nodes, w.P)
    g = g_dev[:S].cpu().numpy()
    r = np.zeros_like(g)
    threads = min(oracle.max_threads(), S)
    t0 = time.perf_counter()
    oi, ov, _ = oracle.topk_ef(g, r, w.k)
    t1 = time.perf_counter()
    B = w.q4_bucket
    if B:
        oc, osc = oracle.q4(ov, B, args.seed, 0)
        ov = oracle.dq4(oc, osc, w.k, B)
    t2 = time.perf_counter()
    off = np.arange(S + 1, dtype=np.uint64) * w.k
    K, dense, _, _ = oracle.reduce(off, oi.ravel(), ov.ravel(), w.N, w.delta)
    t3 = time.perf_counter()
    nb = (w.k + B - 1) // B if B else 0
    b = 12 * S * w.N + 8 * S * w.k + ((S * w.k * 4.5 + 4 * S * nb) * 2 if B else 0) + 8 * S * w.k + \
        (4 * w.N if dense else 8 * K)
    return {"value": round(b / (t3 - t0) / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{S} of {w.P} nodes, full N={w.N} each: Top-k EF, q4+dq4, and the reduce of these {S} "
                      f"nodes' pairs only (K={K} of the sample, not of all {w.P} nodes)",
            "threads_used": threads,
            "thread_cap": f"the oracle runs one thread per node (OpenMP over nodes), so it uses at most the "
                          f"{S} sampled nodes' worth of threads: min(OpenMP threads {oracle.max_threads()}, {S})",
            "host_cores": len(os.sched_getaffinity(0)),
            "cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(),
            "seconds": {"topk_ef": round(t1 - t0, 3), "q4_dq4": round(t2 - t1, 3), "reduce": round(t3 - t2, 3)},
            "topk_gelem_per_s": round(S * w.N / (t1 - t0) / 1e9, 4)}


if __name__ == "__main__":
    main()
