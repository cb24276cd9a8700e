// Attainable-bandwidth reference for the roofline (measurement only).
//
// r += g over n floats with the access pattern of the error-feedback stream
// kernel and nothing else: one 1024-element tile per 256-thread workgroup,
// one non-temporal float4 load of each array and one non-temporal float4
// store per thread. Its rate is the streaming bandwidth the hardware gives a
// kernel of this shape; the stream kernel's rate divided by it is the cost of
// the candidate compaction it adds.
#include "device_common.hpp"
#include "kernels.hpp"

#include <hip/hip_ext.h>

namespace sparcml {
namespace {

__global__ __launch_bounds__(256) void k_reference_add(const float* __restrict__ g, float* __restrict__ r,
                                                       uint64_t n) {
  const uint64_t q = (uint64_t)blockIdx.x * 256 + threadIdx.x;  // float4 group
  if (4 * q + 4 <= n) {
    const f32x4 a = load_nt(reinterpret_cast<const f32x4*>(g) + q) + load_nt(reinterpret_cast<const f32x4*>(r) + q);
    store_nt(a, reinterpret_cast<f32x4*>(r) + q);
  } else {
    for (uint64_t i = 4 * q; i < n; ++i) r[i] += g[i];
  }
}

}  // namespace

hipError_t reference_add_launch(uint64_t n, const float* g, float* r, hipStream_t stream, hipEvent_t ev_start,
                                hipEvent_t ev_stop) {
  if (n == 0) return hipSuccess;
  const uint64_t blocks = (n + 1023) / 1024;
  const float* ga = g;
  float* ra = r;
  uint64_t na = n;
  void* args[] = {&ga, &ra, &na};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(&k_reference_add), dim3((uint32_t)blocks), dim3(256), args, 0,
                            stream, ev_start, ev_stop, 0);
}

}  // namespace sparcml
