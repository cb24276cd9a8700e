// Host-side launchers of the gfx950 kernels, called by the C ABI after its
// argument checks. Each returns hipSuccess or the first HIP error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sparcml {

// ---- error-feedback Top-k -------------------------------------------------
size_t topk_workspace_bytes(uint32_t P, uint64_t N, uint64_t k);
hipError_t topk_ef_launch(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                          uint32_t* out_idx, float* out_val, void* ws, hipStream_t stream,
                          hipEvent_t ev_start, hipEvent_t ev_stop);

// ---- 4-bit stochastic quantization ------------------------------------------
hipError_t q4_launch(uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                     const float* val, uint8_t* codes, float* scales, hipStream_t stream);
hipError_t dq4_launch(uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                      const float* scales, float* val, hipStream_t stream);

// ---- sparse reduction --------------------------------------------------------
struct ReduceResultDev {
  uint64_t nnz;
  uint32_t is_dense;
  uint32_t flags;
};
size_t reduce_workspace_bytes(uint32_t P, uint64_t N, uint64_t total_nnz);
hipError_t sparse_reduce_launch(uint32_t P, uint64_t N, uint64_t T, const uint64_t* h_offsets,
                                const uint32_t* idx, const float* val, bool dense_first,
                                uint32_t* out_idx, uint64_t out_idx_cap, float* out_val,
                                ReduceResultDev* d_result, void* ws, hipStream_t stream);

}  // namespace sparcml
