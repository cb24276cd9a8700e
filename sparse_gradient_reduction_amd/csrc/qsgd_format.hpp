// The b-bit stochastic quantization format (b = 2, 4, 8) shared by the
// quantizer, the dequantizer and the reduce's fused loader.
//
// SparCML (paperlayer.ai digest of arXiv 1802.08021v3), section 6
// "Supporting Low-Precision Communication": QSGD with 2-, 4- and 8-bit
// outputs, buckets quantized independently, each with one full-precision
// scale. A code is a sign bit over b-1 magnitude bits, so a bucket has
// s = 2^(b-1) - 1 nonzero levels of step fl32(scale / s); codes are packed
// 8/b to a byte with the lowest position in the lowest bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparcml {

template <int BITS>
struct Qsgd {
  static_assert(BITS == 2 || BITS == 4 || BITS == 8, "2-, 4- or 8-bit codes");
  static constexpr uint32_t kLevels = (1u << (BITS - 1)) - 1u;  // s: 1, 7, 127
  static constexpr uint32_t kSign = 1u << (BITS - 1);
  static constexpr uint32_t kMask = (1u << BITS) - 1u;
  static constexpr uint32_t kPerByte = 8 / BITS;

  // level step of a bucket: correctly rounded fp32 division
  __device__ static __forceinline__ float step(float scale) { return scale / (float)kLevels; }

  // +-fl32(level * st)
  __device__ static __forceinline__ float value(uint32_t code, float st) {
    const float mag = (float)(code & kLevels) * st;
    return (code & kSign) ? -mag : mag;
  }

  // code of position e in a row that starts at `row`
  __device__ static __forceinline__ uint32_t code_at(const uint8_t* row, uint64_t e) {
    return ((uint32_t)row[e / kPerByte] >> ((uint32_t)(e % kPerByte) * BITS)) & kMask;
  }
};

inline uint64_t qsgd_row_bytes(uint32_t bits, uint64_t n) { return (n * bits + 7) / 8; }

}  // namespace sparcml
