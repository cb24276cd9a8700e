/*
 * sparcml.h - C ABI of the MI355X (gfx950) SparCML hot path.
 *
 * Three operations of SparCML's data-parallel gradient reduction, run on one
 * GPU whose HBM holds the contributions of P nodes:
 *   - error-feedback Top-k sparsification      (sparcml_topk_ef; per layer:
 *                sparcml_topk_ef_layers; per bucket of positions:
 *                sparcml_topk_ef_bucketed)
 *   - 2-, 4- and 8-bit stochastic quantization and back
 *                              (sparcml_qsgd, sparcml_dqsgd; sparcml_q4, sparcml_dq4)
 *   - sum of P sparse contributions with a switch to a dense result
 *              (sparcml_sparse_reduce; sparcml_sparse_reduce_qsgd takes
 *               quantized values; sparcml_qsgd_dense_result quantizes a
 *               dense result)
 *
 * Sources, cited by page title and section: "SparCML: High-Performance Sparse
 * Communication for Machine Learning" (paperlayer.ai digest of arXiv
 * 1802.08021v3) and the arXiv abstract on the mlsanity summary page of the
 * same paper.
 *
 * Conventions shared by every call:
 *   - Pointers marked "device" are HIP device allocations on the current
 *     device; pointers marked "host" are ordinary host memory.
 *   - The caller owns every buffer. The library allocates nothing and keeps
 *     no state between calls (the allocation-free reduce's static scratch
 *     aside). Measurement variants that attach caller-owned events to the
 *     kernel dispatches are declared in sparcml_bench.h.
 *   - Calls are asynchronous on `stream` and stream-ordered, in the spirit of
 *     the non-blocking collectives of the paper (section 7, "Non-Blocking
 *     Operations"): results are valid once the stream has reached them.
 *   - A call only launches kernels on `stream`: no allocation, copy, fill or
 *     host synchronisation, so a sequence of calls may be captured into a HIP
 *     graph and replayed (host arguments such as offsets and layer lists are
 *     taken by value into the launches at capture time).
 *   - The return value reports argument errors (nothing is launched) and
 *     launch errors. The library never aborts, throws or prints. Errors in
 *     the contents of device buffers are reported in device-written flags.
 *   - Arrays are node-major: node p's part of a [P][n] array starts at p*n.
 */
#ifndef SPARCML_H
#define SPARCML_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sparcml_status {
  SPARCML_OK = 0,
  SPARCML_ERR_INVALID_ARG = 1, /* a null pointer, size, alignment or value out of range */
  SPARCML_ERR_WORKSPACE = 2,   /* workspace null, not 256-byte aligned, or smaller than the *_workspace size */
  SPARCML_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
  SPARCML_ERR_SCRATCH_LIMIT = 4 /* the allocation-free call needs more than its static scratch */
} sparcml_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* sparcml_status_string(sparcml_status status);

#define SPARCML_TOPK_ROW_MAX (1u << 17)        /* longest row selected by one workgroup */
#define SPARCML_TOPK_ROW_TOTAL_MAX (1ull << 24) /* ... when P * N is at most this */

/* ------------------------------------------------------------------------
 * Error-feedback Top-k
 *
 * Paper section 2.2 ("Communication-Reduction Techniques"): every node sends
 * the k components of largest magnitude and accumulates the omitted ones for
 * the next iteration. Section 4 ("Sparse Quantized Reduction"): the unapplied
 * part is carried forward as residual error.
 *
 * For each node p and each i < N:
 *   a_i   = grad_i + residual_i          (one fp32 add, round to nearest even)
 *   S     = the k positions that come first when ordered by |a_i| descending
 *           (compared as the IEEE bit pattern with the sign cleared, so -0
 *           ties +0) and then by index ascending: ties go to the lower index
 *   out_idx[p][0..k) = S in ascending order, out_val[p][j] = a[out_idx[p][j]]
 *   residual_i = a_i, except +0.0 at the positions in S      (in place)
 * Hence residual_new + scatter(out_val) == grad + residual_old exactly.
 * Rows of at most SPARCML_TOPK_ROW_MAX elements, in calls of at most
 * SPARCML_TOPK_ROW_TOTAL_MAX elements (P * N), are selected by one workgroup
 * per node; the others by the predicted-threshold candidate pipeline. Both
 * give the result above.
 *
 *   P, N      nodes and elements per node; 1 <= P <= 65535, N <= 2^32 - 2^19,
 *             P * ceil((N+31)/1024) < 2^24 (about P*N < 2^34: one workgroup
 *             per 1024-element tile in one launch dimension)
 *   k         0 <= k <= N (k == 0 only folds grad into residual)
 *   grad      device, [P][N] fp32, read only, 16-byte aligned
 *   residual  device, [P][N] fp32, read and overwritten, 16-byte aligned
 *   out_idx   device, [P][k] uint32 (may be NULL when k == 0)
 *   out_val   device, [P][k] fp32   (may be NULL when k == 0)
 *   ws        device workspace of at least sparcml_topk_ef_workspace(P,N,k)
 *             bytes, 256-byte aligned (as hipMalloc returns); its content on
 *             entry does not matter. After the call the
 *             first 4*P bytes hold, per node, which path produced the result
 *             (0: predicted-threshold candidates, 1: exact rescan, 2: one
 *             workgroup over the whole row, taken when N <=
 *             SPARCML_TOPK_ROW_MAX and P * N <= SPARCML_TOPK_ROW_TOTAL_MAX),
 *             and the next 4*P bytes hold a nonzero
 *             value for a node whose internal consistency check failed (never
 *             expected).
 * grad and residual must not overlap; neither may overlap the outputs.
 * Inputs are expected finite (NaN and Inf are ordered by their bit pattern).
 * ---------------------------------------------------------------------- */
size_t sparcml_topk_ef_workspace(uint32_t P, uint64_t N, uint64_t k);

sparcml_status sparcml_topk_ef(uint32_t P, uint64_t N, uint64_t k,
                               const float* grad, float* residual,
                               uint32_t* out_idx, float* out_val,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Run tables (paper section 5.3.2: the split phase gives each owner one
 * range of indices and every node sends it the part of its sorted pairs
 * that falls there).
 *
 * The reduction cuts the index space into segments of SPARCML_SEGMENT
 * indices. For sparse contributions laid out as in sparcml_sparse_reduce
 * (node p's pairs at positions [h_offsets[p], h_offsets[p+1]), indices
 * ascending), the run table is the [P][S+1] uint32 array, S =
 * ceil(N / SPARCML_SEGMENT), with
 *   runs[p*(S+1) + s] = position of node p's first pair whose index is
 *                       >= s * SPARCML_SEGMENT, or h_offsets[p+1] if none
 * so node p's pairs in segment s are positions [runs[p][s], runs[p][s+1]),
 * runs[p][0] = h_offsets[p] and runs[p][S] = h_offsets[p+1].
 * ---------------------------------------------------------------------- */
#define SPARCML_SEGMENT 4096u

/* sparcml_topk_ef that also writes the run table of its output (node p's k
 * pairs at positions p*k .. p*k + k - 1, index space N), so that the sparse
 * reduction of these pairs needs no pass of its own to find the runs
 * (sparcml_sparse_reduce_runs). The emit pass, which walks every node's
 * candidates in index order, writes the entries as it places the pairs.
 *   runs   device, [P][ceil(N/SPARCML_SEGMENT) + 1] uint32, written
 * Every other argument, the result and the errors are sparcml_topk_ef's;
 * SPARCML_ERR_INVALID_ARG also for a NULL runs or P * k >= 2^32 - 15. */
sparcml_status sparcml_topk_ef_runs(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                                    uint32_t* out_idx, float* out_val, uint32_t* runs, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-layer error-feedback Top-k (paper section 8.4: the ResNet50 runs
 * sparsify layer by layer; sections 2.2 and 4 as for sparcml_topk_ef).
 *
 * Every node's vector is cut into nlayers layers: layer l is positions
 * [off[l], off[l+1]). The selection of sparcml_topk_ef runs on each layer of
 * each node by itself, keeping k[l] positions of layer l. Node p's output
 * row holds K = sum_l k[l] pairs: layer l's selection, ascending, starts at
 * sum_{l'<l} k[l'], with node-relative indices (off[l] + position in the
 * layer), so the row is ascending. The residual becomes a with +0 at every
 * kept position (in place).
 *
 *   P, N       1 <= P, P * nlayers <= 65535, N <= 2^32 - 2^19, P*N < 2^40;
 *              about P*N + 1024*P*nlayers < 2^34 (one workgroup per
 *              1024-element tile of every layer, in one launch dimension)
 *   h_layer_offsets  host, [nlayers+1] uint64: 0 = off[0] <= ... <= off[nlayers] = N
 *   h_k        host, [nlayers] uint64, k[l] <= off[l+1] - off[l]
 *   grad, residual   device, [P][N] fp32, 16-byte aligned (as sparcml_topk_ef)
 *   out_idx, out_val device, [P][K] (may be NULL when K == 0)
 *   ws         device workspace of sparcml_topk_ef_layers_workspace(...) bytes,
 *              256-byte aligned; afterwards its first 4*P*nlayers bytes hold
 *              the path of every (node, layer) row (row p*nlayers + l), the
 *              next 4*P*nlayers bytes its consistency flag, as for
 *              sparcml_topk_ef (path 2 when every layer holds at most
 *              SPARCML_TOPK_ROW_MAX elements and P * N is at most
 *              SPARCML_TOPK_ROW_TOTAL_MAX: one workgroup per row)
 * sparcml_topk_ef_layers_workspace returns 0 for arguments the call rejects.
 * ---------------------------------------------------------------------- */
size_t sparcml_topk_ef_layers_workspace(uint32_t P, uint64_t N, uint32_t nlayers,
                                        const uint64_t* h_layer_offsets, const uint64_t* h_k);

sparcml_status sparcml_topk_ef_layers(uint32_t P, uint64_t N, uint32_t nlayers,
                                      const uint64_t* h_layer_offsets, const uint64_t* h_k,
                                      const float* grad, float* residual, uint32_t* out_idx,
                                      float* out_val, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Bucketed error-feedback Top-k (paper section 8.3: k entries kept out of
 * every 512, e.g. 16/512; sections 2.2 and 4 for the selection and the
 * residual).
 *
 * Per node p, the N positions form buckets of `bucket` consecutive positions
 * (the last one partial, restarting per node). With a = grad + residual and
 * the key and order of sparcml_topk_ef, bucket j with len_j positions keeps
 * k_j = min(k_per_bucket, len_j) positions: the first k_j of the bucket
 * under (key descending, index ascending). Node p's output row holds
 * K = sparcml_topk_bucketed_count(N, bucket, k_per_bucket) = sum_j k_j pairs:
 * bucket j's selection, ascending, starts at j * min(k_per_bucket, bucket),
 * so the row is ascending. The residual becomes a, with +0 at every kept
 * position (in place).
 *
 *   P, N      1 <= P <= 65535, N < 2^32, P*N < 2^40
 *   bucket    64, 128, 256, 512 or 1024
 *   grad      device, [P][N] fp32, read only
 *   residual  device, [P][N] fp32, read and overwritten
 *   out_idx   device, [P][K] uint32 node-relative indices (NULL if K == 0)
 *   out_val   device, [P][K] fp32                          (NULL if K == 0)
 * No workspace. grad and residual must not overlap each other or the outputs.
 * ---------------------------------------------------------------------- */
uint64_t sparcml_topk_bucketed_count(uint64_t N, uint32_t bucket, uint32_t k_per_bucket);

sparcml_status sparcml_topk_ef_bucketed(uint32_t P, uint64_t N, uint32_t bucket, uint32_t k_per_bucket,
                                        const float* grad, float* residual, uint32_t* out_idx,
                                        float* out_val, hipStream_t stream);

/* ------------------------------------------------------------------------
 * 4-bit stochastic quantization (paper section 6, "Supporting Low-Precision
 * Communication": buckets quantized independently and stochastically, each
 * with one full-precision scale; section 2.2: zero-mean quantization noise).
 *
 * Per node p the n values form buckets of `bucket` consecutive positions (the
 * last one may be partial). For bucket j: scale = max |v| (exact) and
 * st = scale / 7. Position e with value v gets
 *   level = 0                                     if scale == 0
 *   level = floor(x) + (u < x - floor(x))         otherwise,
 *           x = (|v| / scale) * 7  (two fp32 roundings, no fused multiply-add)
 *           u = (w >> 8) * 2^-24, w = word (e & 3) of the Philox-4x32-10 block
 *               for counter {e >> 2, p, step, 0} and key {seed lo32, seed hi32}
 *   code = (v < 0 ? 8 : 0) | level
 * Codes are packed two per byte, even positions in the low nibble; each node's
 * row is ceil(n/2) bytes and an unused high nibble is zero.
 * dq4 returns (code & 8 ? -1 : +1) * (level * st), rounded in fp32.
 *
 *   bucket    multiple of 8, 8 <= bucket <= 2^20
 *   val       device, [P][n] fp32
 *   codes     device, [P][ceil(n/2)] uint8
 *   scales    device, [P][ceil(n/bucket)] fp32
 * ---------------------------------------------------------------------- */
sparcml_status sparcml_q4(uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                          const float* val, uint8_t* codes, float* scales, hipStream_t stream);

sparcml_status sparcml_dq4(uint32_t P, uint64_t n, uint32_t bucket,
                           const uint8_t* codes, const float* scales, float* val,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * b-bit stochastic quantization, b in {2, 4, 8} (paper section 6, "Supporting
 * Low-Precision Communication": QSGD with 2-, 4- and 8-bit outputs).
 *
 * sparcml_q4 / sparcml_dq4 above are the b = 4, node0 = 0 case. In general a
 * code is a sign bit over b-1 magnitude bits, so a bucket has
 * s = 2^(b-1) - 1 nonzero levels (1, 7, 127) and st = scale / s. Position e
 * of row p gets
 *   level = 0                                     if scale == 0
 *   level = floor(x) + (u < x - floor(x))         otherwise,
 *           x = (|v| / scale) * s  (two fp32 roundings, no fused multiply-add)
 *           u = (w >> 8) * 2^-24, w = word (e & 3) of the Philox-4x32-10 block
 *               for counter {e >> 2, node0 + p, step, 0} and key
 *               {seed lo32, seed hi32}
 *   code = (v < 0 ? 2^(b-1) : 0) | level
 * Codes are packed 8/b to a byte: position e sits at bit (e mod 8/b) * b of
 * byte e*b/8, the lowest position in the lowest bits. Each row is
 * ceil(n*b/8) bytes and unused bits are zero. sparcml_dqsgd returns
 * (sign ? -1 : +1) * (level * st), rounded in fp32.
 *
 *   bits      2, 4 or 8
 *   bucket    multiple of 8, 8 <= bucket <= 2^20
 *   node0     node index of row 0 in the Philox counter; node0 + P - 1 < 2^32
 *   val       device, [P][n] fp32, 16-byte aligned
 *   codes     device, [P][ceil(n*bits/8)] uint8
 *   scales    device, [P][ceil(n/bucket)] fp32
 * ---------------------------------------------------------------------- */
sparcml_status sparcml_qsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed,
                            uint32_t step, uint32_t node0, const float* val, uint8_t* codes,
                            float* scales, hipStream_t stream);

sparcml_status sparcml_dqsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket,
                             const uint8_t* codes, const float* scales, float* val,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse reduction with the dense switch.
 *
 * Paper section 5.1 ("Data Representation: Sparse Streams"): index-value
 * pairs that switch to a dense representation once fill-in passes the
 * threshold delta. Section 5.2: the reduction is a coordinate-wise sum with
 * neutral element 0. Section 5.3: the result is dense when its size K reaches
 * delta; a rough estimate of K chooses the algorithm. Appendix B: K counts
 * the indices in the union of the contributed sets (uniform-sampling estimate
 * in B.1).
 *
 *   K = |union of the index sets|   (an index counts even if its sum is 0)
 *   T = ceil(delta * N), computed in double
 *   K >= T  -> dense:  out_val[i] = sum of the values at index i, 0 elsewhere,
 *                      for every i < N; out_idx is not written
 *   K <  T  -> sparse: out_idx[0..K) = the union ascending, out_val[0..K) = sums
 * Sums are accumulated in fp64 and rounded to fp32 once.
 *
 *   P          1 <= P <= 1024 nodes
 *   N          index space, 1 <= N < 2^32
 *   delta      finite; delta <= 0 is always dense, T > N never dense
 *   h_offsets  host, [P+1] uint64, nondecreasing, h_offsets[0] == 0,
 *              h_offsets[P] <= 2^32 - 16: node p owns pairs
 *              [h_offsets[p], h_offsets[p+1])
 *   idx, val   device, [h_offsets[P]] uint32 / fp32; each node's indices
 *              strictly ascending and < N
 *   expected_nnz_hint  0: estimate K from the nonzero counts (uniform model
 *              of Appendix B.1); else the caller's estimate. It only chooses
 *              between the dense-first and the count-first algorithm; the
 *              result does not depend on it.
 *   out_idx    device, uint32, capacity min(N, T-1) (T > 0), else unused
 *   out_val    device, fp32, capacity N (entries past K in the sparse case
 *              are unspecified)
 *   d_result   device, one sparcml_reduce_result, written by the GPU
 *   ws         device workspace of sparcml_sparse_reduce_workspace(P, N, nnz)
 *              bytes, 256-byte aligned; content on entry does not matter
 *
 * Indices >= N or not strictly ascending within a node set bits in
 * d_result->flags; the outputs are then unspecified but no write leaves the
 * stated capacities.
 * ---------------------------------------------------------------------- */
typedef struct sparcml_reduce_result {
  uint64_t nnz;      /* K */
  uint32_t is_dense; /* 1: out_val holds N dense values; 0: K sparse pairs */
  uint32_t flags;    /* SPARCML_FLAG_* bits, 0 for valid input */
} sparcml_reduce_result;

#define SPARCML_FLAG_INDEX_RANGE 1u    /* an index >= N */
#define SPARCML_FLAG_NOT_ASCENDING 2u  /* a node's indices not strictly ascending */
#define SPARCML_FLAG_RUN_TABLE 4u      /* a caller's run table that does not fit the pairs
                                          (sparcml_sparse_reduce_runs) */

size_t sparcml_sparse_reduce_workspace(uint32_t P, uint64_t N, uint64_t total_nnz);

sparcml_status sparcml_sparse_reduce(uint32_t P, uint64_t N, double delta,
                                     const uint64_t* h_offsets,
                                     const uint32_t* idx, const float* val,
                                     uint64_t expected_nnz_hint,
                                     uint32_t* out_idx, float* out_val,
                                     sparcml_reduce_result* d_result,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse reduction with the caller's run table (see "Run tables" above),
 * for pairs whose producer already knows where each node's sorted pairs
 * cross the segments (sparcml_topk_ef_runs writes it for its output): the
 * operation, result, workspace and errors of sparcml_sparse_reduce, without
 * its pass over the indices that finds the runs and checks range and order.
 *   runs   device, [P][ceil(N/SPARCML_SEGMENT) + 1] uint32, read only
 * Instead, the table is checked against the pairs as they are read: entries
 * outside a node's pairs or out of order, a first or last entry other than
 * the node's offsets, or a pair whose index lies outside the segment its run
 * places it in set SPARCML_FLAG_RUN_TABLE in d_result->flags (an index >= N
 * sets SPARCML_FLAG_INDEX_RANGE). A table that passes covers every pair
 * once, in its segment. Order within a segment is not checked: a repeated
 * index within one node then counts once in K and adds all its values.
 * ---------------------------------------------------------------------- */
sparcml_status sparcml_sparse_reduce_runs(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                          const uint32_t* idx, const float* val, const uint32_t* runs,
                                          uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                          sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse reduction in two phases: the union phase reads only the indices
 * (their run starts, the union bitmaps and counts, K and the dense decision:
 * paper Appendix B and section 5.3), the sums phase adds the values into the
 * result. A training step knows its indices before its values are final
 * (they may still be quantized and dequantized), so it can run the union
 * phase right after the Top-k, while the Top-k's output is still in the
 * GPU's memory-side cache, and the sums once the values are ready.
 *
 * sparcml_sparse_reduce_union followed, on the same stream, by
 * sparcml_sparse_reduce_sums with the same P, N, delta, h_offsets (the same
 * values), idx, runs, expected_nnz_hint, d_result and ws, the indices, the
 * table and the workspace left unchanged in between, gives exactly the
 * result of sparcml_sparse_reduce (runs == NULL) or
 * sparcml_sparse_reduce_runs (runs given). d_result is complete after the
 * sums phase. Arguments and errors are those of sparcml_sparse_reduce(_runs);
 * the union phase takes no values or outputs. Other work may run on the
 * stream between the two calls.
 * ---------------------------------------------------------------------- */
sparcml_status sparcml_sparse_reduce_union(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                           const uint32_t* idx, const uint32_t* runs, uint64_t expected_nnz_hint,
                                           sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                           hipStream_t stream);
sparcml_status sparcml_sparse_reduce_sums(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                          const uint32_t* idx, const float* val, const uint32_t* runs,
                                          uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                          sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Allocation-free sparse reduction, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * The operation, arguments, outputs and errors of sparcml_sparse_reduce,
 * without the workspace: its scratch is a static device array of
 * SPARCML_REDUCE_SCRATCH_BYTES in the library, one copy per GPU, kept until
 * the process ends. The first call on a device looks up that device's copy
 * (hipGetSymbolAddress); no call allocates or frees memory. Returns
 * SPARCML_ERR_SCRATCH_LIMIT, launching nothing, when
 * sparcml_sparse_reduce_workspace(P, N, h_offsets[P]) exceeds
 * SPARCML_REDUCE_SCRATCH_BYTES (32 MiB: for instance 64 nodes over an index
 * space of 2^27 take 26.5 MB).
 * Every call on one GPU uses the same scratch: calls that may overlap in time
 * on one GPU (different streams without ordering between them) race and
 * give unspecified results. Calls ordered on one stream are safe; each clears
 * what it needs.
 * ---------------------------------------------------------------------- */
#define SPARCML_REDUCE_SCRATCH_BYTES (32u << 20)

sparcml_status sparcml_sparse_reduce_noalloc(uint32_t P, uint64_t N, double delta,
                                             const uint64_t* h_offsets,
                                             const uint32_t* idx, const float* val,
                                             uint64_t expected_nnz_hint,
                                             uint32_t* out_idx, float* out_val,
                                             sparcml_reduce_result* d_result, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse reduction of quantized contributions (paper section 6: the values
 * travel as QSGD codes; dequantization is fused into the reduction's load).
 *
 * The same operation, arguments, workspace and errors as
 * sparcml_sparse_reduce, except that node p's values are given as b-bit
 * codes of its pairs, in pair order, decoded as sparcml_dqsgd decodes them
 * while they are loaded. The result equals sparcml_sparse_reduce over the
 * dequantized values.
 *   bits, bucket  as for sparcml_qsgd
 *   codes   device: node p's codes start at byte sum_{q<p} ceil(nnz_q*bits/8)
 *   scales  device: node p's scales start at sum_{q<p} ceil(nnz_q/bucket)
 * With nnz = n pairs on every node these are exactly the [P][ceil(n*bits/8)]
 * and [P][ceil(n/bucket)] arrays sparcml_qsgd writes for a [P][n] input.
 * ---------------------------------------------------------------------- */
sparcml_status sparcml_sparse_reduce_qsgd(uint32_t bits, uint32_t bucket, uint32_t P, uint64_t N,
                                          double delta, const uint64_t* h_offsets,
                                          const uint32_t* idx, const uint8_t* codes,
                                          const float* scales, uint64_t expected_nnz_hint,
                                          uint32_t* out_idx, float* out_val,
                                          sparcml_reduce_result* d_result, void* ws,
                                          size_t ws_bytes, hipStream_t stream);

/* sparcml_sparse_reduce_qsgd with the caller's run table: the quantized
 * contributions of sparcml_sparse_reduce_qsgd, the table and its checks of
 * sparcml_sparse_reduce_runs. Where idx is 16-byte aligned and codes 4-byte
 * aligned, the rank-order writer loads the pairs four at a time and decodes
 * their codes from two aligned words. */
sparcml_status sparcml_sparse_reduce_qsgd_runs(uint32_t bits, uint32_t bucket, uint32_t P, uint64_t N,
                                               double delta, const uint64_t* h_offsets, const uint32_t* idx,
                                               const uint8_t* codes, const float* scales, const uint32_t* runs,
                                               uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                               sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * Quantization of a dense reduction result, decided on the device (paper
 * section 4: the sum may be quantized once it has turned dense; section 6:
 * the dense part of the exchange is the one that travels quantized).
 *
 * Reads d_result->is_dense on the device, in stream order after the
 * reduction that wrote it. If it is 1, codes and scales receive
 * sparcml_qsgd(bits, 1, N, bucket, seed, step, node, val, ...) of the dense
 * result val[0..N); otherwise nothing is written. The host never waits.
 *   d_result  device, written by an earlier sparcml_sparse_reduce(_qsgd) on
 *             `stream` (or otherwise complete before this call runs)
 *   val       device, [N] fp32, 16-byte aligned (that reduction's out_val)
 *   codes     device, [ceil(N*bits/8)] uint8
 *   scales    device, [ceil(N/bucket)] fp32
 *   node      the node index in the Philox counter
 * ---------------------------------------------------------------------- */
sparcml_status sparcml_qsgd_dense_result(uint32_t bits, uint64_t N, uint32_t bucket, uint64_t seed,
                                         uint32_t step, uint32_t node,
                                         const sparcml_reduce_result* d_result, const float* val,
                                         uint8_t* codes, float* scales, hipStream_t stream);

/* Uniform-model estimate of K used when no hint is given (Appendix B.1):
 * N * (1 - prod_p (1 - nnz_p / N)), capped by sum_p nnz_p. Host only. */
double sparcml_estimate_nnz(uint32_t P, uint64_t N, const uint64_t* h_offsets);

#ifdef __cplusplus
}
#endif

#endif /* SPARCML_H */
