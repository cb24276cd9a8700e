// Attainable-bandwidth reference for the roofline (measurement only).
//
// r += g over n floats with the access pattern of the error-feedback stream
// kernel and nothing else: one 1024-element tile per 256-thread workgroup,
// one non-temporal float4 load of each array and one non-temporal float4
// store per thread. Its rate is the streaming bandwidth the hardware gives a
// kernel of this shape; the stream kernel's rate divided by it is the cost of
// the candidate compaction it adds.
// Built into its own library, libsparcml_bench.so, apart from the method's.
#include "sparcml_bench.h"

#include "device_common.hpp"
#include "kernels.hpp"

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
}  // namespace sparcml

extern "C" sparcml_status sparcml_bench_reference_stream(uint64_t n, const float* g, float* r,
                                                         const sparcml_bench_events* ev, hipStream_t stream) {
  const auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (n > (1ull << 34) - 1024 || (n > 0 && (!g || !r || misaligned(g) || misaligned(r)))) return SPARCML_ERR_INVALID_ARG;
  if (n == 0) return SPARCML_OK;
  const uint64_t blocks = (n + 1023) / 1024;  // < 2^24 workgroups of 256: one launch dimension
  const hipError_t e = sparcml::launch_ev(sparcml::k_reference_add, dim3((uint32_t)blocks), dim3(256), stream,
                                          ev ? ev->op_start : nullptr, ev ? ev->op_stop : nullptr, g, r, n);
  return e == hipSuccess ? SPARCML_OK : SPARCML_ERR_HIP;
}
