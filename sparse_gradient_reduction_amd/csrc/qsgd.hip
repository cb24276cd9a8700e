// b-bit stochastic quantization (and its inverse) for gfx950, b = 2, 4, 8.
//
// SparCML (paperlayer.ai digest of arXiv 1802.08021v3), section 6
// "Supporting Low-Precision Communication": QSGD quantizes buckets of values
// independently and stochastically, each with one full-precision scale, to
// 2, 4 or 8 bits; section 2.2: the quantization noise is zero-mean; section
// 4: the reduced dense vector may itself be quantized.
//
// Format (qsgd_format.hpp): per node, buckets of `bucket` consecutive values
// (last partial), scale = max |v|, code = sign bit + level 0..s with
// s = 2^(b-1) - 1, the level rounded up with probability equal to the
// fractional part of |v|/scale*s using a Philox-4x32-10 word keyed by the
// seed and addressed by (position/4, node, step). One wave per bucket: a
// wave-wide max, then each lane turns 8 consecutive values into b bytes of
// codes (two Philox blocks). A device-side gate word lets the quantizer run
// only when the reduction's result turned out dense, with no host round trip.
#include "device_common.hpp"
#include "kernels.hpp"
#include "qsgd_format.hpp"

#include <algorithm>

namespace sparcml {
namespace {

// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, SC'11, "Parallel
// Random Numbers: As Easy as 1, 2, 3"): per round, 32x32->64-bit products of
// counter words 0 and 2 with the two Philox-4x32 multipliers; the high halves
// are mixed with counter words 1 and 3 and the round key; the key advances by
// the two Weyl increments between rounds.
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32x32->64 multiply (v_mad_u64_u32) gives both halves
    const uint64_t prod_a = (uint64_t)kMulA * c0, prod_b = (uint64_t)kMulB * c2;
    const uint32_t hi_a = (uint32_t)(prod_a >> 32), lo_a = (uint32_t)prod_a;
    const uint32_t hi_b = (uint32_t)(prod_b >> 32), lo_b = (uint32_t)prod_b;
    const uint32_t n0 = hi_b ^ c1 ^ k0;
    const uint32_t n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  return Philox4{{c0, c1, c2, c3}};
}

constexpr int kPerLane = 8;
constexpr int kChunk = kWave * kPerLane;  // 512 positions per wave step

template <int BITS>
__device__ __forceinline__ uint32_t quantize_one(float v, float scale, uint32_t word) {
  using F = Qsgd<BITS>;
  uint32_t level = 0u;
  if (scale != 0.0f) {
    const float ratio = fabsf(v) / scale;
    const float x = ratio * (float)F::kLevels;
    const float l = floorf(x);
    const float f = x - l;
    const float u = (float)(word >> 8) * (1.0f / 16777216.0f);
    level = (uint32_t)l + (u < f ? 1u : 0u);
  }
  return (v < 0.0f ? F::kSign : 0u) | level;
}

struct QArgs {
  uint32_t P;
  uint64_t n;
  uint32_t bucket;
  uint64_t nb;  // buckets per node
  uint64_t row_bytes;
  uint32_t key0, key1, step, node0;
};

__device__ __forceinline__ void load8(const float* row, uint64_t e, uint64_t end, bool vec_ok, float v[8]) {
  if (vec_ok && e + 8 <= end) {
    const float4 a = *reinterpret_cast<const float4*>(row + e);
    const float4 b = *reinterpret_cast<const float4*>(row + e + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e + i < end) ? row[e + i] : 0.0f;
  }
}

// the BITS bytes holding positions e..e+7 (e a multiple of 8)
template <int BITS>
__device__ __forceinline__ void store_lane(uint8_t* crow, uint64_t byte, uint64_t row_bytes, uint64_t packed,
                                           bool whole) {
  if (whole && (reinterpret_cast<uintptr_t>(crow + byte) % BITS) == 0) {
    if (BITS == 2) *reinterpret_cast<uint16_t*>(crow + byte) = (uint16_t)packed;
    else if (BITS == 4) *reinterpret_cast<uint32_t*>(crow + byte) = (uint32_t)packed;
    else *reinterpret_cast<uint64_t*>(crow + byte) = packed;
  } else {
#pragma unroll
    for (int b = 0; b < BITS; ++b)
      if (byte + b < row_bytes) crow[byte + b] = (uint8_t)(packed >> (8 * b));
  }
}

template <int BITS>
__device__ __forceinline__ uint64_t load_lane(const uint8_t* crow, uint64_t byte, uint64_t row_bytes) {
  if (byte + BITS <= row_bytes && (reinterpret_cast<uintptr_t>(crow + byte) % BITS) == 0) {
    if (BITS == 2) return *reinterpret_cast<const uint16_t*>(crow + byte);
    if (BITS == 4) return *reinterpret_cast<const uint32_t*>(crow + byte);
    return *reinterpret_cast<const uint64_t*>(crow + byte);
  }
  uint64_t packed = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b)
    if (byte + b < row_bytes) packed |= (uint64_t)crow[byte + b] << (8 * b);
  return packed;
}

template <int BITS>
__global__ __launch_bounds__(256) void k_qsgd(const float* __restrict__ val, uint8_t* __restrict__ codes,
                                              float* __restrict__ scales, QArgs A, const uint32_t* gate) {
  if (gate != nullptr && *gate == 0u) return;  // the result this would quantize is not dense
  const uint32_t p = blockIdx.y;
  const uint32_t lane = lane_id();
  for (uint64_t j = (uint64_t)blockIdx.x * 4 + threadIdx.x / kWave; j < A.nb; j += (uint64_t)gridDim.x * 4) {  // bucket
    const uint32_t node = A.node0 + p;
    const float* row = val + (uint64_t)p * A.n;
    uint8_t* crow = codes + (uint64_t)p * A.row_bytes;
    const bool vec_ok = (((uint64_t)p * A.n) & 3u) == 0;
    const uint64_t b0 = j * A.bucket;
    const uint64_t b1 = std::min<uint64_t>(b0 + A.bucket, A.n);

    // buckets of up to kHeld chunks stay in registers between the max and the
    // quantization; longer ones are read twice
    constexpr int kHeld = 2;
    float held[kHeld][8];
    float m = 0.0f;
    const bool fits = (b1 - b0) <= (uint64_t)kHeld * kChunk;
    if (fits) {
#pragma unroll
      for (int h = 0; h < kHeld; ++h) {
        load8(row, b0 + (uint64_t)h * kChunk + lane * kPerLane, b1, vec_ok, held[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(held[h][i]));
      }
    } else {
      for (uint64_t c = b0; c < b1; c += kChunk) {
        float v[8];
        load8(row, c + lane * kPerLane, b1, vec_ok, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
      }
    }
    const float scale = wave_max(m);
    if (lane == 0) scales[(uint64_t)p * A.nb + j] = scale;

    for (uint64_t c = b0, h = 0; c < b1; c += kChunk, ++h) {
      const uint64_t e = c + lane * kPerLane;
      float v[8];
      if (fits) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = h == 0 ? held[0][i] : held[1][i];
      } else {
        load8(row, e, b1, vec_ok, v);
      }
      if (e >= b1) continue;
      const uint32_t ctr = (uint32_t)(e >> 2);
      const Philox4 r0 = philox4x32_10(ctr, node, A.step, 0u, A.key0, A.key1);
      const Philox4 r1 = philox4x32_10(ctr + 1u, node, A.step, 0u, A.key0, A.key1);
      uint64_t packed = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (e + i < b1) {
          const uint32_t rnd = i < 4 ? r0.w[i] : r1.w[i - 4];
          packed |= (uint64_t)quantize_one<BITS>(v[i], scale, rnd) << (BITS * i);
        }
      }
      store_lane<BITS>(crow, e / 8 * BITS, A.row_bytes, packed, e + 8 <= A.n);
    }
  }  // buckets of this wave
}

template <int BITS>
__global__ __launch_bounds__(256) void k_dqsgd(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                                               float* __restrict__ val, QArgs A) {
  using F = Qsgd<BITS>;
  const uint32_t p = blockIdx.y;
  const uint64_t e = ((uint64_t)blockIdx.x * 256 + threadIdx.x) * kPerLane;
  if (e >= A.n) return;
  const uint8_t* crow = codes + (uint64_t)p * A.row_bytes;
  float* row = val + (uint64_t)p * A.n;
  const uint64_t packed = load_lane<BITS>(crow, e / 8 * BITS, A.row_bytes);
  const float st = F::step(scales[(uint64_t)p * A.nb + e / A.bucket]);
  float out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = F::value((uint32_t)(packed >> (BITS * i)) & F::kMask, st);
  if ((((uint64_t)p * A.n) & 3u) == 0 && e + 8 <= A.n) {
    *reinterpret_cast<float4*>(row + e) = make_float4(out[0], out[1], out[2], out[3]);
    *reinterpret_cast<float4*>(row + e + 4) = make_float4(out[4], out[5], out[6], out[7]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (e + i < A.n) row[e + i] = out[i];
  }
}

QArgs make_args(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                uint32_t node0) {
  QArgs A;
  A.P = P;
  A.n = n;
  A.bucket = bucket;
  A.nb = (n + bucket - 1) / bucket;
  A.row_bytes = qsgd_row_bytes(bits, n);
  A.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  A.key1 = (uint32_t)(seed >> 32);
  A.step = step;
  A.node0 = node0;
  return A;
}

}  // namespace

hipError_t qsgd_launch(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                       uint32_t node0, const uint32_t* gate, const float* val, uint8_t* codes, float* scales,
                       hipStream_t stream, const OpEvents* ev) {
  const QArgs A = make_args(bits, P, n, bucket, seed, step, node0);
  if (n == 0) return hipSuccess;
  // a wave per bucket, up to the 2^32 work-items a grid dimension allows
  const dim3 grid((uint32_t)std::min<uint64_t>((A.nb + 3) / 4, 1u << 22), P);
  const hipEvent_t e0 = ev ? ev->op_start : nullptr, e1 = ev ? ev->op_stop : nullptr;
  switch (bits) {
    case 2: return launch_ev(k_qsgd<2>, grid, dim3(256), stream, e0, e1, val, codes, scales, A, gate);
    case 4: return launch_ev(k_qsgd<4>, grid, dim3(256), stream, e0, e1, val, codes, scales, A, gate);
    case 8: return launch_ev(k_qsgd<8>, grid, dim3(256), stream, e0, e1, val, codes, scales, A, gate);
    default: return hipErrorInvalidValue;
  }
}

hipError_t dqsgd_launch(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                        const float* scales, float* val, hipStream_t stream, const OpEvents* ev) {
  const QArgs A = make_args(bits, P, n, bucket, 0, 0, 0);
  if (n == 0) return hipSuccess;
  const uint64_t lanes = (n + kPerLane - 1) / kPerLane;
  const dim3 grid((uint32_t)((lanes + 255) / 256), P);
  const hipEvent_t e0 = ev ? ev->op_start : nullptr, e1 = ev ? ev->op_stop : nullptr;
  switch (bits) {
    case 2: return launch_ev(k_dqsgd<2>, grid, dim3(256), stream, e0, e1, codes, scales, val, A);
    case 4: return launch_ev(k_dqsgd<4>, grid, dim3(256), stream, e0, e1, codes, scales, val, A);
    case 8: return launch_ev(k_dqsgd<8>, grid, dim3(256), stream, e0, e1, codes, scales, val, A);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sparcml
