// 4-bit stochastic quantization (and its inverse) for gfx950.
//
// SparCML (paperlayer.ai digest of arXiv 1802.08021v3), section 6
// "Supporting Low-Precision Communication": QSGD quantizes buckets of values
// independently and stochastically, each with one full-precision scale, to
// 2, 4 or 8 bits; section 2.2: the quantization noise is zero-mean.
//
// Format: per node, buckets of `bucket` consecutive values (last partial),
// scale = max |v|, 4-bit code = sign bit + level 0..7, level rounded up with
// probability equal to the fractional part of |v|/scale*7 using a
// Philox-4x32-10 word keyed by the seed and addressed by (position/4, node,
// step). One wave per bucket: a wave-wide max, then each lane turns 8
// consecutive values into one 32-bit word of codes (two Philox blocks).
#include "device_common.hpp"
#include "kernels.hpp"

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
    const uint32_t hi_a = __umulhi(kMulA, c0), lo_a = kMulA * c0;
    const uint32_t hi_b = __umulhi(kMulB, c2), lo_b = kMulB * c2;
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

constexpr int kLanesPerChunk = kWave;
constexpr int kPerLane = 8;
constexpr int kChunk = kLanesPerChunk * kPerLane;  // 512 positions per wave step

__device__ __forceinline__ uint32_t quantize_one(float v, float scale, uint32_t word) {
  uint32_t level = 0u;
  if (scale != 0.0f) {
    const float ratio = fabsf(v) / scale;
    const float x = ratio * 7.0f;
    const float l = floorf(x);
    const float f = x - l;
    const float u = (float)(word >> 8) * (1.0f / 16777216.0f);
    level = (uint32_t)l + (u < f ? 1u : 0u);
  }
  return (v < 0.0f ? 8u : 0u) | level;
}

struct Q4Args {
  uint32_t P;
  uint64_t n;
  uint32_t bucket;
  uint64_t nb;       // buckets per node
  uint64_t row_bytes;
  uint32_t key0, key1, step;
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

__global__ __launch_bounds__(256) void k_q4(const float* __restrict__ val, uint8_t* __restrict__ codes,
                                            float* __restrict__ scales, Q4Args A) {
  const uint32_t p = blockIdx.y;
  const uint64_t j = (uint64_t)blockIdx.x * 4 + threadIdx.x / kWave;  // bucket
  if (j >= A.nb) return;
  const uint32_t lane = lane_id();
  const float* row = val + (uint64_t)p * A.n;
  uint8_t* crow = codes + (uint64_t)p * A.row_bytes;
  const bool vec_ok = (((uint64_t)p * A.n) & 3u) == 0;
  const bool word_ok = (reinterpret_cast<uintptr_t>(crow) & 3u) == 0;
  const uint64_t b0 = j * A.bucket;
  const uint64_t b1 = std::min<uint64_t>(b0 + A.bucket, A.n);

  float vals[8];
  float m = 0.0f;
  const bool single = (b1 - b0) <= (uint64_t)kChunk;
  for (uint64_t c = b0; c < b1; c += kChunk) {
    float v[8];
    load8(row, c + lane * kPerLane, b1, vec_ok, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m = fmaxf(m, fabsf(v[i]));
      vals[i] = v[i];
    }
  }
  const float scale = wave_max(m);
  if (lane == 0) scales[(uint64_t)p * A.nb + j] = scale;

  for (uint64_t c = b0; c < b1; c += kChunk) {
    const uint64_t e = c + lane * kPerLane;
    float v[8];
    if (single) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = vals[i];
    } else {
      load8(row, e, b1, vec_ok, v);
    }
    if (e >= b1) continue;
    const uint32_t ctr = (uint32_t)(e >> 2);
    const Philox4 r0 = philox4x32_10(ctr, p, A.step, 0u, A.key0, A.key1);
    const Philox4 r1 = philox4x32_10(ctr + 1u, p, A.step, 0u, A.key0, A.key1);
    uint32_t word = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (e + i < b1) {
        const uint32_t rnd = i < 4 ? r0.w[i] : r1.w[i - 4];
        word |= quantize_one(v[i], scale, rnd) << (4 * i);
      }
    }
    const uint64_t byte = e >> 1;
    if (word_ok && e + 8 <= A.n) {
      *reinterpret_cast<uint32_t*>(crow + byte) = word;
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (byte + b < A.row_bytes) crow[byte + b] = (uint8_t)(word >> (8 * b));
    }
  }
}

__global__ __launch_bounds__(256) void k_dq4(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                                             float* __restrict__ val, Q4Args A) {
  const uint32_t p = blockIdx.y;
  const uint64_t e = ((uint64_t)blockIdx.x * 256 + threadIdx.x) * kPerLane;
  if (e >= A.n) return;
  const uint8_t* crow = codes + (uint64_t)p * A.row_bytes;
  float* row = val + (uint64_t)p * A.n;
  const uint64_t byte = e >> 1;
  uint32_t word = 0u;
  if ((reinterpret_cast<uintptr_t>(crow) & 3u) == 0 && byte + 4 <= A.row_bytes) {
    word = *reinterpret_cast<const uint32_t*>(crow + byte);
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (byte + b < A.row_bytes) word |= (uint32_t)crow[byte + b] << (8 * b);
  }
  const float st = scales[(uint64_t)p * A.nb + e / A.bucket] / 7.0f;
  float out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = (word >> (4 * i)) & 0xFu;
    const float mag = (float)(code & 7u) * st;
    out[i] = (code & 8u) ? -mag : mag;
  }
  if ((((uint64_t)p * A.n) & 3u) == 0 && e + 8 <= A.n) {
    *reinterpret_cast<float4*>(row + e) = make_float4(out[0], out[1], out[2], out[3]);
    *reinterpret_cast<float4*>(row + e + 4) = make_float4(out[4], out[5], out[6], out[7]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (e + i < A.n) row[e + i] = out[i];
  }
}

Q4Args make_args(uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step) {
  Q4Args A;
  A.P = P;
  A.n = n;
  A.bucket = bucket;
  A.nb = (n + bucket - 1) / bucket;
  A.row_bytes = (n + 1) / 2;
  A.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  A.key1 = (uint32_t)(seed >> 32);
  A.step = step;
  return A;
}

}  // namespace

hipError_t q4_launch(uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                     const float* val, uint8_t* codes, float* scales, hipStream_t stream) {
  const Q4Args A = make_args(P, n, bucket, seed, step);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_q4, dim3((uint32_t)((A.nb + 3) / 4), P), dim3(256), 0, stream, val, codes, scales, A);
  return hipGetLastError();
}

hipError_t dq4_launch(uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes, const float* scales,
                      float* val, hipStream_t stream) {
  const Q4Args A = make_args(P, n, bucket, 0, 0);
  if (n == 0) return hipSuccess;
  const uint64_t lanes = (n + kPerLane - 1) / kPerLane;
  hipLaunchKernelGGL(k_dq4, dim3((uint32_t)((lanes + 255) / 256), P), dim3(256), 0, stream, codes, scales, val, A);
  return hipGetLastError();
}

}  // namespace sparcml
