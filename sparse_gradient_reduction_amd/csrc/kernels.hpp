// Host-side launchers of the gfx950 kernels, called by the C ABI after its
// argument checks. Each returns hipSuccess or the first HIP error.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sparcml {

// Measurement only: events a sparcml_bench_* call attaches to kernel
// dispatches (any may be null). op_start rides on the op's first kernel,
// op_stop on its last; k_start / k_stop on the op's dominant kernel (the
// error-feedback stream kernel of Top-k).
struct OpEvents {
  hipEvent_t op_start = nullptr;
  hipEvent_t op_stop = nullptr;
  hipEvent_t k_start = nullptr;
  hipEvent_t k_stop = nullptr;
};

template <class T>
struct same_type {
  using type = T;
};

// Launches fn on `stream`; `start` / `stop`, when not null, are recorded as
// the kernel itself starts and ends (hipExtLaunchKernel), so that their
// elapsed time is that kernel's and nothing queued around it.
// `lds` bytes of dynamic LDS.
template <typename... P>
hipError_t launch_ev_lds(void (*fn)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop, typename same_type<P>::type... a) {
  if (start == nullptr && stop == nullptr) {
    hipLaunchKernelGGL(fn, grid, block, lds, stream, a...);
    return hipGetLastError();
  }
  void* args[] = {static_cast<void*>(&a)...};
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, args, lds, stream, start,
                                          stop, 0);
  return e != hipSuccess ? e : hipGetLastError();
}

template <typename... P>
hipError_t launch_ev(void (*fn)(P...), dim3 grid, dim3 block, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                     typename same_type<P>::type... a) {
  return launch_ev_lds(fn, grid, block, 0, stream, start, stop, a...);
}

// ---- error-feedback Top-k -------------------------------------------------
size_t topk_workspace_bytes(uint32_t P, uint64_t N, uint64_t k);
// runs: null, or the [P][ceil(N / SPARCML_SEGMENT) + 1] run table of the
// output, written by the emit pass
hipError_t topk_ef_launch(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                          uint32_t* out_idx, float* out_val, uint32_t* runs, void* ws, hipStream_t stream,
                          const OpEvents* ev);
// the run table of a finished [P][k] output (P * k < 2^32)
hipError_t topk_runs_of_output_launch(uint32_t P, uint64_t N, uint64_t k, const uint32_t* out_idx, uint32_t* runs,
                                      hipStream_t stream);

// ---- error-feedback Top-k of short rows: one workgroup per node; info holds
// the [P] path words (2) and the [P] consistency words the workspace reports
hipError_t topk_row_launch(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                           uint32_t* out_idx, float* out_val, uint32_t* info, hipStream_t stream,
                           const OpEvents* ev);

// per-layer call whose layers all hold at most SPARCML_TOPK_ROW_MAX elements:
// one workgroup per (node, layer) row. Uses the first
// topk_layer_rows_workspace_bytes(P, nl) bytes of the per-layer workspace:
// the [P * nl] path and consistency words, then the layer tables.
size_t topk_layer_rows_workspace_bytes(uint32_t P, uint32_t nl);
hipError_t topk_layer_rows_launch(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k,
                                  const float* grad, float* residual, uint32_t* out_idx, float* out_val, void* ws,
                                  hipStream_t stream);

// ---- per-layer error-feedback Top-k (layers [off[l], off[l+1]) of every node)
size_t topk_layers_workspace_bytes(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k);
uint64_t topk_layers_stream_blocks(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k);
hipError_t topk_layers_launch(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k,
                              const float* grad, float* residual, uint32_t* out_idx, float* out_val, void* ws,
                              hipStream_t stream);

// ---- bucketed error-feedback Top-k (bucket = 64, 128, 256, 512 or 1024) -----
uint64_t topk_bucketed_count(uint64_t N, uint32_t bucket, uint32_t k);
hipError_t topk_bucketed_launch(uint32_t P, uint64_t N, uint32_t bucket, uint32_t k, const float* grad,
                                float* residual, uint32_t* out_idx, float* out_val, hipStream_t stream);

// ---- b-bit stochastic quantization (b = 2, 4, 8) ----------------------------
// gate: null, or a device word that must be nonzero for the quantizer to run
hipError_t qsgd_launch(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                       uint32_t node0, const uint32_t* gate, const float* val, uint8_t* codes, float* scales,
                       hipStream_t stream, const OpEvents* ev = nullptr);
hipError_t dqsgd_launch(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                        const float* scales, float* val, hipStream_t stream, const OpEvents* ev = nullptr);

// ---- sparse reduction --------------------------------------------------------
struct ReduceResultDev {
  uint64_t nnz;
  uint32_t is_dense;
  uint32_t flags;
};
size_t reduce_workspace_bytes(uint32_t P, uint64_t N, uint64_t total_nnz);
// quantized input: node p's values are the b-bit codes of its pairs, each
// node's code row and scale row following the previous node's
struct ReduceQuantized {
  uint32_t bits;  // 2, 4 or 8
  uint32_t bucket;
  const uint8_t* codes;
  const float* scales;
};
// val is used when quant is null, quant otherwise; runs, when not null, is
// the caller's run table and replaces the bounds pass;
// union_est, the expected union size, sizes the writer groups
// The reduce in one call, or its two phases: the union phase (run starts,
// union count, decision; reads only the indices) and the sums phase (the
// writer), which needs the workspace as the union phase left it and the same
// arguments.
enum ReducePhase { kReduceUnion = 1, kReduceSums = 2, kReduceBoth = 3 };
hipError_t sparse_reduce_launch(uint32_t P, uint64_t N, uint64_t T, const uint64_t* h_offsets,
                                const uint32_t* idx, const float* val, const ReduceQuantized* quant,
                                const uint32_t* runs, bool dense_first, double union_est, uint32_t* out_idx,
                                uint64_t out_idx_cap, float* out_val, ReduceResultDev* d_result, void* ws,
                                hipStream_t stream, const OpEvents* ev = nullptr, int phase = kReduceBoth);

}  // namespace sparcml
