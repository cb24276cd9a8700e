// C ABI of the SparCML hot path: argument checks, workspace sizing, launch.
// The declarations and their contracts are in include/sparcml.h and, for the
// measurement variants, include/sparcml_bench.h.
#include "sparcml.h"
#include "sparcml_bench.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "kernels.hpp"

// Scratch of the allocation-free reduce: one copy per GPU, held until the
// process ends. Host code never passes this name to a kernel; it uses the
// device address that hipGetSymbolAddress gives on each device.
static __device__ __align__(256) unsigned char scratch[SPARCML_REDUCE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch`, per device ordinal
std::mutex g_scratch_mu;

// Device address of the current device's `scratch`, looked up once per device.
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

sparcml_status from_hip(hipError_t e) { return e == hipSuccess ? SPARCML_OK : SPARCML_ERR_HIP; }

constexpr uint64_t kMaxN = 0xFFFFFFFFull;       // indices are uint32
constexpr uint64_t kMaxTopkN = 0xFFF80000ull;   // 2^32 - 2^19: candidate slot offsets stay below 2^32 - 2^18

// T = ceil(delta * N) in double, clamped to [0, N + 1]
uint64_t dense_threshold(double delta, uint64_t N) {
  const double t = std::ceil(delta * (double)N);
  if (!(t > 0.0)) return 0;
  if (t > (double)N) return N + 1;
  return (uint64_t)t;
}

}  // namespace

extern "C" {

const char* sparcml_status_string(sparcml_status status) {
  switch (status) {
    case SPARCML_OK: return "SPARCML_OK";
    case SPARCML_ERR_INVALID_ARG: return "SPARCML_ERR_INVALID_ARG: invalid argument";
    case SPARCML_ERR_WORKSPACE: return "SPARCML_ERR_WORKSPACE: workspace missing or too small";
    case SPARCML_ERR_HIP: return "SPARCML_ERR_HIP: HIP runtime or launch error";
    case SPARCML_ERR_SCRATCH_LIMIT:
      return "SPARCML_ERR_SCRATCH_LIMIT: the call needs more than SPARCML_REDUCE_SCRATCH_BYTES of scratch";
  }
  return "SPARCML: unknown status";
}

// --------------------------------------------------------------------------
size_t sparcml_topk_ef_workspace(uint32_t P, uint64_t N, uint64_t k) {
  if (P == 0 || N > kMaxTopkN || k > N || P > 65535u) return 0;
  return sparcml::topk_workspace_bytes(P, N, k);
}

// runs: null, or the run table of the output to write (sparcml_topk_ef_runs)
static sparcml_status topk_common(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                                  uint32_t* out_idx, float* out_val, uint32_t* runs, void* ws, size_t ws_bytes,
                                  hipStream_t stream, const sparcml::OpEvents* ev) {
  if (P == 0 || P > 65535u || N > kMaxTopkN || k > N) return SPARCML_ERR_INVALID_ARG;
  if (runs && (uint64_t)P * k > kMaxN - 15) return SPARCML_ERR_INVALID_ARG;  // table positions are uint32
  if ((uint64_t)P * N >= (1ull << 40)) return SPARCML_ERR_INVALID_ARG;
  // one 256-thread workgroup per 1024-element tile slot (a node's tiles start at
  // the 128-byte line of its first element), in one grid dimension of < 2^32 work-items
  if ((uint64_t)P * ((N + 31 + 1023) / 1024) >= (1ull << 24)) return SPARCML_ERR_INVALID_ARG;
  if (N == 0) return SPARCML_OK;
  if (!grad || !residual || !aligned16(grad) || !aligned16(residual)) return SPARCML_ERR_INVALID_ARG;
  if (k > 0 && (!out_idx || !out_val)) return SPARCML_ERR_INVALID_ARG;
  if (!ws || !aligned256(ws) || ws_bytes < sparcml::topk_workspace_bytes(P, N, k)) return SPARCML_ERR_WORKSPACE;
  // short rows in a small call: one workgroup per node beats the candidate pipeline's kernel chain
  if (N <= SPARCML_TOPK_ROW_MAX && (uint64_t)P * N <= SPARCML_TOPK_ROW_TOTAL_MAX) {
    hipError_t e =
        sparcml::topk_row_launch(P, N, k, grad, residual, out_idx, out_val, static_cast<uint32_t*>(ws), stream, ev);
    // the row kernel has no emit pass: the table comes from its output
    if (e == hipSuccess && runs) e = sparcml::topk_runs_of_output_launch(P, N, k, out_idx, runs, stream);
    return from_hip(e);
  }
  return from_hip(sparcml::topk_ef_launch(P, N, k, grad, residual, out_idx, out_val, runs, ws, stream, ev));
}

sparcml_status sparcml_topk_ef(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                               uint32_t* out_idx, float* out_val, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  return topk_common(P, N, k, grad, residual, out_idx, out_val, nullptr, ws, ws_bytes, stream, nullptr);
}

sparcml_status sparcml_topk_ef_runs(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                                    uint32_t* out_idx, float* out_val, uint32_t* runs, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!runs) return SPARCML_ERR_INVALID_ARG;
  return topk_common(P, N, k, grad, residual, out_idx, out_val, runs, ws, ws_bytes, stream, nullptr);
}

// --------------------------------------------------------------------------
// layers: off[0] = 0 < ... nondecreasing ... off[nl] = N, k[l] <= off[l+1] - off[l]
static bool layers_ok(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k) {
  if (P == 0 || P > 65535u || nl == 0 || (uint64_t)P * nl > 65535u || N > kMaxTopkN) return false;
  if (!off || !k || off[0] != 0 || off[nl] != N) return false;
  for (uint32_t l = 0; l < nl; ++l)
    if (off[l + 1] < off[l] || k[l] > off[l + 1] - off[l]) return false;
  if ((uint64_t)P * N >= (1ull << 40)) return false;
  // one 256-thread workgroup per tile of every layer, in one grid dimension
  return sparcml::topk_layers_stream_blocks(P, N, nl, off, k) < (1ull << 24);
}

size_t sparcml_topk_ef_layers_workspace(uint32_t P, uint64_t N, uint32_t nlayers, const uint64_t* h_layer_offsets,
                                        const uint64_t* h_k) {
  if (!layers_ok(P, N, nlayers, h_layer_offsets, h_k)) return 0;
  return sparcml::topk_layers_workspace_bytes(P, N, nlayers, h_layer_offsets, h_k);
}

sparcml_status sparcml_topk_ef_layers(uint32_t P, uint64_t N, uint32_t nlayers, const uint64_t* h_layer_offsets,
                                      const uint64_t* h_k, const float* grad, float* residual, uint32_t* out_idx,
                                      float* out_val, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!layers_ok(P, N, nlayers, h_layer_offsets, h_k)) return SPARCML_ERR_INVALID_ARG;
  if (N == 0) return SPARCML_OK;
  if (!grad || !residual || !aligned16(grad) || !aligned16(residual)) return SPARCML_ERR_INVALID_ARG;
  uint64_t K = 0;
  for (uint32_t l = 0; l < nlayers; ++l) K += h_k[l];
  if (K > 0 && (!out_idx || !out_val)) return SPARCML_ERR_INVALID_ARG;
  if (!ws || !aligned256(ws) ||
      ws_bytes < sparcml::topk_layers_workspace_bytes(P, N, nlayers, h_layer_offsets, h_k))
    return SPARCML_ERR_WORKSPACE;
  uint64_t longest = 0;
  for (uint32_t l = 0; l < nlayers; ++l) longest = std::max(longest, h_layer_offsets[l + 1] - h_layer_offsets[l]);
  if (longest <= SPARCML_TOPK_ROW_MAX && (uint64_t)P * N <= SPARCML_TOPK_ROW_TOTAL_MAX &&
      ws_bytes >= sparcml::topk_layer_rows_workspace_bytes(P, nlayers))
    return from_hip(sparcml::topk_layer_rows_launch(P, N, nlayers, h_layer_offsets, h_k, grad, residual, out_idx,
                                                    out_val, ws, stream));  // only short layers: one workgroup each
  return from_hip(sparcml::topk_layers_launch(P, N, nlayers, h_layer_offsets, h_k, grad, residual, out_idx, out_val,
                                              ws, stream));
}

// --------------------------------------------------------------------------
static bool bucket_ok(uint32_t bucket) {
  return bucket == 64 || bucket == 128 || bucket == 256 || bucket == 512 || bucket == 1024;
}

uint64_t sparcml_topk_bucketed_count(uint64_t N, uint32_t bucket, uint32_t k_per_bucket) {
  if (!bucket_ok(bucket) || N > kMaxN) return 0;
  return sparcml::topk_bucketed_count(N, bucket, k_per_bucket);
}

sparcml_status sparcml_topk_ef_bucketed(uint32_t P, uint64_t N, uint32_t bucket, uint32_t k_per_bucket,
                                        const float* grad, float* residual, uint32_t* out_idx, float* out_val,
                                        hipStream_t stream) {
  if (P == 0 || P > 65535u || N > kMaxN || !bucket_ok(bucket)) return SPARCML_ERR_INVALID_ARG;
  if ((uint64_t)P * N >= (1ull << 40)) return SPARCML_ERR_INVALID_ARG;
  if (N == 0) return SPARCML_OK;
  if (!grad || !residual) return SPARCML_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(grad) | reinterpret_cast<uintptr_t>(residual)) & 3u) return SPARCML_ERR_INVALID_ARG;
  if (sparcml::topk_bucketed_count(N, bucket, k_per_bucket) > 0 && (!out_idx || !out_val))
    return SPARCML_ERR_INVALID_ARG;
  return from_hip(sparcml::topk_bucketed_launch(P, N, bucket, k_per_bucket, grad, residual, out_idx, out_val,
                                                stream));
}

// --------------------------------------------------------------------------
static bool qsgd_args_ok(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket) {
  if (bits != 2 && bits != 4 && bits != 8) return false;
  if (P == 0 || P > 65535u) return false;
  if (bucket < 8 || bucket > (1u << 20) || (bucket % 8) != 0) return false;
  if (n >= (1ull << 34)) return false;
  return true;  // any number of buckets: the kernels loop over them
}

static sparcml_status qsgd_common(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed,
                                  uint32_t step, uint32_t node0, const float* val, uint8_t* codes, float* scales,
                                  hipStream_t stream, const sparcml::OpEvents* ev) {
  if (!qsgd_args_ok(bits, P, n, bucket)) return SPARCML_ERR_INVALID_ARG;
  if ((uint64_t)node0 + P - 1 > 0xFFFFFFFFull) return SPARCML_ERR_INVALID_ARG;
  if (n == 0) return SPARCML_OK;
  if (!val || !codes || !scales || !aligned16(val)) return SPARCML_ERR_INVALID_ARG;
  return from_hip(
      sparcml::qsgd_launch(bits, P, n, bucket, seed, step, node0, nullptr, val, codes, scales, stream, ev));
}

static sparcml_status dqsgd_common(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                                   const float* scales, float* val, hipStream_t stream, const sparcml::OpEvents* ev) {
  if (!qsgd_args_ok(bits, P, n, bucket)) return SPARCML_ERR_INVALID_ARG;
  if (n == 0) return SPARCML_OK;
  if (!val || !codes || !scales || !aligned16(val)) return SPARCML_ERR_INVALID_ARG;
  return from_hip(sparcml::dqsgd_launch(bits, P, n, bucket, codes, scales, val, stream, ev));
}

sparcml_status sparcml_qsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                            uint32_t node0, const float* val, uint8_t* codes, float* scales, hipStream_t stream) {
  return qsgd_common(bits, P, n, bucket, seed, step, node0, val, codes, scales, stream, nullptr);
}

sparcml_status sparcml_dqsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                             const float* scales, float* val, hipStream_t stream) {
  return dqsgd_common(bits, P, n, bucket, codes, scales, val, stream, nullptr);
}

sparcml_status sparcml_q4(uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                          const float* val, uint8_t* codes, float* scales, hipStream_t stream) {
  return sparcml_qsgd(4, P, n, bucket, seed, step, 0u, val, codes, scales, stream);
}

sparcml_status sparcml_dq4(uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes, const float* scales,
                           float* val, hipStream_t stream) {
  return sparcml_dqsgd(4, P, n, bucket, codes, scales, val, stream);
}

sparcml_status sparcml_qsgd_dense_result(uint32_t bits, uint64_t N, uint32_t bucket, uint64_t seed, uint32_t step,
                                         uint32_t node, const sparcml_reduce_result* d_result, const float* val,
                                         uint8_t* codes, float* scales, hipStream_t stream) {
  if (!qsgd_args_ok(bits, 1, N, bucket) || N > kMaxN || !d_result) return SPARCML_ERR_INVALID_ARG;
  if (N == 0) return SPARCML_OK;
  if (!val || !codes || !scales || !aligned16(val)) return SPARCML_ERR_INVALID_ARG;
  return from_hip(sparcml::qsgd_launch(bits, 1, N, bucket, seed, step, node, &d_result->is_dense, val, codes,
                                       scales, stream));
}

// --------------------------------------------------------------------------
double sparcml_estimate_nnz(uint32_t P, uint64_t N, const uint64_t* h_offsets) {
  if (!h_offsets || N == 0) return 0.0;
  double miss = 1.0, sum = 0.0;
  for (uint32_t p = 0; p < P; ++p) {
    const double c = (double)(h_offsets[p + 1] - h_offsets[p]);
    sum += c;
    const double q = c / (double)N;
    miss *= (q >= 1.0 ? 0.0 : 1.0 - q);
  }
  const double e = (double)N * (1.0 - miss);
  return e < sum ? e : sum;
}

size_t sparcml_sparse_reduce_workspace(uint32_t P, uint64_t N, uint64_t total_nnz) {
  if (P == 0 || P > 1024u || N == 0 || N > kMaxN || total_nnz > kMaxN) return 0;
  return sparcml::reduce_workspace_bytes(P, N, total_nnz);
}

// runs: null, or the caller's run table; phase: both phases, or one of them
// (the union phase needs neither values nor outputs)
static sparcml_status reduce_common(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                    const uint32_t* idx, const float* val, const sparcml::ReduceQuantized* quant,
                                    const uint32_t* runs, uint64_t expected_nnz_hint, uint32_t* out_idx,
                                    float* out_val, sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                    hipStream_t stream, const sparcml::OpEvents* ev = nullptr,
                                    int phase = sparcml::kReduceBoth) {
  const bool sums = (phase & sparcml::kReduceSums) != 0;
  if (P == 0 || P > 1024u || N == 0 || N > kMaxN || !std::isfinite(delta)) return SPARCML_ERR_INVALID_ARG;
  if (!h_offsets || !d_result || (sums && (!out_val || !aligned16(out_val)))) return SPARCML_ERR_INVALID_ARG;
  if (h_offsets[0] != 0) return SPARCML_ERR_INVALID_ARG;
  for (uint32_t p = 0; p < P; ++p)
    if (h_offsets[p + 1] < h_offsets[p]) return SPARCML_ERR_INVALID_ARG;
  const uint64_t total = h_offsets[P];
  if (total > kMaxN - 15) return SPARCML_ERR_INVALID_ARG;  // positions and quad ends fit in 32 bits
  if (total > 0 && (!idx || (sums && (quant ? (!quant->codes || !quant->scales) : !val))))
    return SPARCML_ERR_INVALID_ARG;
  const uint64_t T = dense_threshold(delta, N);
  const uint64_t cap = T == 0 ? 0 : (T - 1 < N ? T - 1 : N);
  if (sums && cap > 0 && !out_idx) return SPARCML_ERR_INVALID_ARG;
  if (!ws || !aligned256(ws) || ws_bytes < sparcml::reduce_workspace_bytes(P, N, total)) return SPARCML_ERR_WORKSPACE;
  // the model's union estimate sizes the writer groups; a hint, where given,
  // picks the writer in its place
  const double model = sparcml_estimate_nnz(P, N, h_offsets);
  const double est = expected_nnz_hint ? (double)expected_nnz_hint : model;
  const bool dense_first = est >= (double)T;
  return from_hip(sparcml::sparse_reduce_launch(P, N, T, h_offsets, idx, val, quant, runs, dense_first, model,
                                                out_idx, cap, out_val,
                                                reinterpret_cast<sparcml::ReduceResultDev*>(d_result), ws, stream,
                                                ev, phase));
}

sparcml_status sparcml_sparse_reduce(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                     const uint32_t* idx, const float* val, uint64_t expected_nnz_hint,
                                     uint32_t* out_idx, float* out_val, sparcml_reduce_result* d_result,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  return reduce_common(P, N, delta, h_offsets, idx, val, nullptr, nullptr, expected_nnz_hint, out_idx, out_val, d_result, ws,
                       ws_bytes, stream);
}

sparcml_status sparcml_sparse_reduce_runs(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                          const uint32_t* idx, const float* val, const uint32_t* runs,
                                          uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                          sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  if (!runs) return SPARCML_ERR_INVALID_ARG;
  return reduce_common(P, N, delta, h_offsets, idx, val, nullptr, runs, expected_nnz_hint, out_idx, out_val,
                       d_result, ws, ws_bytes, stream);
}

sparcml_status sparcml_sparse_reduce_union(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                           const uint32_t* idx, const uint32_t* runs, uint64_t expected_nnz_hint,
                                           sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  return reduce_common(P, N, delta, h_offsets, idx, nullptr, nullptr, runs, expected_nnz_hint, nullptr, nullptr,
                       d_result, ws, ws_bytes, stream, nullptr, sparcml::kReduceUnion);
}

sparcml_status sparcml_sparse_reduce_sums(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                          const uint32_t* idx, const float* val, const uint32_t* runs,
                                          uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                          sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  return reduce_common(P, N, delta, h_offsets, idx, val, nullptr, runs, expected_nnz_hint, out_idx, out_val,
                       d_result, ws, ws_bytes, stream, nullptr, sparcml::kReduceSums);
}

sparcml_status sparcml_sparse_reduce_noalloc(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                             const uint32_t* idx, const float* val, uint64_t expected_nnz_hint,
                                             uint32_t* out_idx, float* out_val, sparcml_reduce_result* d_result,
                                             hipStream_t stream) {
  if (P == 0 || P > 1024u || N == 0 || N > kMaxN || !h_offsets) return SPARCML_ERR_INVALID_ARG;
  if (h_offsets[P] > kMaxN) return SPARCML_ERR_INVALID_ARG;
  if (sparcml::reduce_workspace_bytes(P, N, h_offsets[P]) > SPARCML_REDUCE_SCRATCH_BYTES)
    return SPARCML_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return SPARCML_ERR_HIP;
  return reduce_common(P, N, delta, h_offsets, idx, val, nullptr, nullptr, expected_nnz_hint, out_idx, out_val, d_result, ws,
                       SPARCML_REDUCE_SCRATCH_BYTES, stream);
}

static sparcml_status reduce_qsgd_common(uint32_t bits, uint32_t bucket, uint32_t P, uint64_t N, double delta,
                                         const uint64_t* h_offsets, const uint32_t* idx, const uint8_t* codes,
                                         const float* scales, const uint32_t* runs, uint64_t expected_nnz_hint,
                                         uint32_t* out_idx, float* out_val, sparcml_reduce_result* d_result,
                                         void* ws, size_t ws_bytes, hipStream_t stream,
                                         const sparcml::OpEvents* ev = nullptr) {
  if (!qsgd_args_ok(bits, 1, 0, bucket)) return SPARCML_ERR_INVALID_ARG;
  const sparcml::ReduceQuantized q{bits, bucket, codes, scales};
  return reduce_common(P, N, delta, h_offsets, idx, nullptr, &q, runs, expected_nnz_hint, out_idx, out_val,
                       d_result, ws, ws_bytes, stream, ev);
}

sparcml_status sparcml_sparse_reduce_qsgd(uint32_t bits, uint32_t bucket, uint32_t P, uint64_t N, double delta,
                                          const uint64_t* h_offsets, const uint32_t* idx, const uint8_t* codes,
                                          const float* scales, uint64_t expected_nnz_hint, uint32_t* out_idx,
                                          float* out_val, sparcml_reduce_result* d_result, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  return reduce_qsgd_common(bits, bucket, P, N, delta, h_offsets, idx, codes, scales, nullptr, expected_nnz_hint,
                            out_idx, out_val, d_result, ws, ws_bytes, stream);
}

sparcml_status sparcml_sparse_reduce_qsgd_runs(uint32_t bits, uint32_t bucket, uint32_t P, uint64_t N,
                                               double delta, const uint64_t* h_offsets, const uint32_t* idx,
                                               const uint8_t* codes, const float* scales, const uint32_t* runs,
                                               uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                               sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                               hipStream_t stream) {
  if (!runs) return SPARCML_ERR_INVALID_ARG;
  return reduce_qsgd_common(bits, bucket, P, N, delta, h_offsets, idx, codes, scales, runs, expected_nnz_hint,
                            out_idx, out_val, d_result, ws, ws_bytes, stream);
}

// --------------------------------------------------------------------------
// Measurement entry points: the calls above with caller-owned events
// attached to their kernel dispatches.
static sparcml::OpEvents op_events(const sparcml_bench_events* ev) {
  sparcml::OpEvents e;
  if (ev) {
    e.op_start = ev->op_start;
    e.op_stop = ev->op_stop;
    e.k_start = ev->kernel_start;
    e.k_stop = ev->kernel_stop;
  }
  return e;
}

sparcml_status sparcml_bench_topk_ef(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                                     uint32_t* out_idx, float* out_val, void* ws, size_t ws_bytes,
                                     const sparcml_bench_events* ev, hipStream_t stream) {
  const sparcml::OpEvents e = op_events(ev);
  return topk_common(P, N, k, grad, residual, out_idx, out_val, nullptr, ws, ws_bytes, stream, &e);
}

sparcml_status sparcml_bench_topk_ef_runs(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                                          uint32_t* out_idx, float* out_val, uint32_t* runs, void* ws,
                                          size_t ws_bytes, const sparcml_bench_events* ev, hipStream_t stream) {
  if (!runs) return SPARCML_ERR_INVALID_ARG;
  const sparcml::OpEvents e = op_events(ev);
  return topk_common(P, N, k, grad, residual, out_idx, out_val, runs, ws, ws_bytes, stream, &e);
}

sparcml_status sparcml_bench_qsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed,
                                  uint32_t step, uint32_t node0, const float* val, uint8_t* codes, float* scales,
                                  const sparcml_bench_events* ev, hipStream_t stream) {
  const sparcml::OpEvents e = op_events(ev);
  return qsgd_common(bits, P, n, bucket, seed, step, node0, val, codes, scales, stream, &e);
}

sparcml_status sparcml_bench_dqsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                                   const float* scales, float* val, const sparcml_bench_events* ev,
                                   hipStream_t stream) {
  const sparcml::OpEvents e = op_events(ev);
  return dqsgd_common(bits, P, n, bucket, codes, scales, val, stream, &e);
}

sparcml_status sparcml_bench_sparse_reduce(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                           const uint32_t* idx, const float* val, uint64_t expected_nnz_hint,
                                           uint32_t* out_idx, float* out_val, sparcml_reduce_result* d_result,
                                           void* ws, size_t ws_bytes, const sparcml_bench_events* ev,
                                           hipStream_t stream) {
  const sparcml::OpEvents e = op_events(ev);
  return reduce_common(P, N, delta, h_offsets, idx, val, nullptr, nullptr, expected_nnz_hint, out_idx, out_val,
                       d_result, ws, ws_bytes, stream, &e);
}

sparcml_status sparcml_bench_sparse_reduce_runs(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                                const uint32_t* idx, const float* val, const uint32_t* runs,
                                                uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                                sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                                const sparcml_bench_events* ev, hipStream_t stream) {
  if (!runs) return SPARCML_ERR_INVALID_ARG;
  const sparcml::OpEvents e = op_events(ev);
  return reduce_common(P, N, delta, h_offsets, idx, val, nullptr, runs, expected_nnz_hint, out_idx, out_val,
                       d_result, ws, ws_bytes, stream, &e);
}

sparcml_status sparcml_bench_sparse_reduce_qsgd_runs(uint32_t bits, uint32_t bucket, uint32_t P, uint64_t N,
                                                     double delta, const uint64_t* h_offsets, const uint32_t* idx,
                                                     const uint8_t* codes, const float* scales,
                                                     const uint32_t* runs, uint64_t expected_nnz_hint,
                                                     uint32_t* out_idx, float* out_val,
                                                     sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                                     const sparcml_bench_events* ev, hipStream_t stream) {
  if (!runs) return SPARCML_ERR_INVALID_ARG;
  const sparcml::OpEvents e = op_events(ev);
  return reduce_qsgd_common(bits, bucket, P, N, delta, h_offsets, idx, codes, scales, runs, expected_nnz_hint,
                            out_idx, out_val, d_result, ws, ws_bytes, stream, &e);
}

sparcml_status sparcml_bench_sparse_reduce_union(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                                 const uint32_t* idx, const uint32_t* runs, uint64_t expected_nnz_hint,
                                                 sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                                 const sparcml_bench_events* ev, hipStream_t stream) {
  const sparcml::OpEvents e = op_events(ev);
  return reduce_common(P, N, delta, h_offsets, idx, nullptr, nullptr, runs, expected_nnz_hint, nullptr, nullptr,
                       d_result, ws, ws_bytes, stream, &e, sparcml::kReduceUnion);
}

sparcml_status sparcml_bench_sparse_reduce_sums(uint32_t P, uint64_t N, double delta, const uint64_t* h_offsets,
                                                const uint32_t* idx, const float* val, const uint32_t* runs,
                                                uint64_t expected_nnz_hint, uint32_t* out_idx, float* out_val,
                                                sparcml_reduce_result* d_result, void* ws, size_t ws_bytes,
                                                const sparcml_bench_events* ev, hipStream_t stream) {
  const sparcml::OpEvents e = op_events(ev);
  return reduce_common(P, N, delta, h_offsets, idx, val, nullptr, runs, expected_nnz_hint, out_idx, out_val,
                       d_result, ws, ws_bytes, stream, &e, sparcml::kReduceSums);
}

}  // extern "C"
