/*
 * sparcml_bench.h - measurement entry points of the SparCML hot path.
 *
 * Not part of the method: these calls exist so that a benchmark can time the
 * path's kernels on the GPU's own clock without a profiler and without state
 * kept in the library. Each takes a pointer to caller-owned HIP events
 * (created on the current device; any member, or the pointer itself, may be
 * NULL) and attaches them to kernel dispatches with hipExtLaunchKernel, so
 * that an event is recorded when that kernel starts or ends and not when the
 * host queued it:
 *   op_start      the op's first kernel starts
 *   op_stop       the op's last kernel ends
 *   kernel_start  the op's dominant kernel starts
 *   kernel_stop   the op's dominant kernel ends
 * hipEventElapsedTime(op_start, op_stop) is then the op's span on the GPU
 * and hipEventElapsedTime(kernel_start, kernel_stop) its dominant kernel's
 * own duration. Where one dispatch would carry two stop events (the
 * dominant kernel is also the last), op_stop is recorded on the stream right
 * after it; where the op is a single kernel, that kernel carries the op's
 * pair when one is given, else the kernel pair.
 *
 * Apart from the events, each call is the call of the same name in sparcml.h
 * (sparcml_bench_X is sparcml_X): the same arguments, checks, workspace,
 * results and errors. Arguments are checked before any event is touched; an
 * argument error records none.
 *
 * Exported by libsparcml.so, except sparcml_bench_reference_stream, which
 * lives in libsparcml_bench.so.
 */
#ifndef SPARCML_BENCH_H
#define SPARCML_BENCH_H

#include "sparcml.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sparcml_bench_events {
  hipEvent_t op_start;
  hipEvent_t op_stop;
  hipEvent_t kernel_start;
  hipEvent_t kernel_stop;
} sparcml_bench_events;

/* Dominant kernel: the streaming error-feedback pass (r += g and the
 * candidate compaction) of the whole-vector path; for rows short enough for
 * one workgroup per node, the single row kernel. */
sparcml_status sparcml_bench_topk_ef(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                                     uint32_t* out_idx, float* out_val, void* ws, size_t ws_bytes,
                                     const sparcml_bench_events* ev, hipStream_t stream);

/* sparcml_topk_ef_runs, with the events of sparcml_bench_topk_ef. */
sparcml_status sparcml_bench_topk_ef_runs(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                                          uint32_t* out_idx, float* out_val, uint32_t* runs, void* ws,
                                          size_t ws_bytes, const sparcml_bench_events* ev, hipStream_t stream);

/* One kernel each: it carries the op's pair (or the kernel pair). */
sparcml_status sparcml_bench_qsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed,
                                  uint32_t step, uint32_t node0, const float* val, uint8_t* codes, float* scales,
                                  const sparcml_bench_events* ev, hipStream_t stream);
sparcml_status sparcml_bench_dqsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                                   const float* scales, float* val, const sparcml_bench_events* ev,
                                   hipStream_t stream);

/* Dominant kernel: the writer (the last kernel), which sums the pairs and
 * stores the result. */
sparcml_status sparcml_bench_sparse_reduce(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                           const uint32_t* idx, const float* val, uint64_t expected_nnz_hint,
                                           uint32_t* out_idx, float* out_val, sparcml_reduce_result* d_result,
                                           void* ws, size_t ws_bytes, const sparcml_bench_events* ev,
                                           hipStream_t stream);

/* sparcml_sparse_reduce_runs, with the events of sparcml_bench_sparse_reduce
 * (the op's first kernel is then the count pass). */
sparcml_status sparcml_bench_sparse_reduce_runs(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                                const uint32_t* idx, const float* val, const uint32_t* runs,
                                                uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                                sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                                const sparcml_bench_events* ev, hipStream_t stream);

/* sparcml_sparse_reduce_qsgd_runs, with the events of
 * sparcml_bench_sparse_reduce_runs. */
sparcml_status sparcml_bench_sparse_reduce_qsgd_runs(uint32_t bits, uint32_t bucket, uint32_t P, uint64_t N,
                                                     double delta, const uint64_t* h_offsets, const uint32_t* idx,
                                                     const uint8_t* codes, const float* scales,
                                                     const uint32_t* runs, uint64_t expected_nnz_hint,
                                                     uint32_t* out_idx, float* out_val,
                                                     sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                                     const sparcml_bench_events* ev, hipStream_t stream);

/* The two phases of the reduction: the union phase's span runs from its
 * first kernel to its last (the decide pass, or the count pass); the sums
 * phase is the writer alone, which carries the op's pair when given, else
 * the kernel pair. */
sparcml_status sparcml_bench_sparse_reduce_union(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                                 const uint32_t* idx, const uint32_t* runs, uint64_t expected_nnz_hint,
                                                 sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                                 const sparcml_bench_events* ev, hipStream_t stream);
sparcml_status sparcml_bench_sparse_reduce_sums(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                                const uint32_t* idx, const float* val, const uint32_t* runs,
                                                uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                                sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                                const sparcml_bench_events* ev, hipStream_t stream);

/* Attainable-bandwidth reference, in libsparcml_bench.so: r[i] += g[i] for
 * i < n with exactly the access pattern of the error-feedback stream kernel
 * (one 1024-element tile per 256-thread workgroup, one non-temporal float4
 * load of each array and one non-temporal float4 store per thread), and no
 * other work. One kernel: it carries op_start / op_stop.
 *   g, r   device, n fp32 each, 16-byte aligned, not overlapping
 *   n      <= 2^34 - 1024
 * SPARCML_ERR_INVALID_ARG for a bad argument, SPARCML_ERR_HIP for a failed
 * launch. */
sparcml_status sparcml_bench_reference_stream(uint64_t n, const float* g, float* r, const sparcml_bench_events* ev,
                                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARCML_BENCH_H */
