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
    // three-way xors, one v_bitop3_b32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi_b, c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi_a, c3, k1, 0x96);
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

// Code of value v whose ratio |v| / scale (correctly rounded fp32) is given:
// level floor(x) + [u < x - floor(x)] with x = ratio * s and u the top 24
// bits of the random word over 2^24, under the sign bit.
template <int BITS>
__device__ __forceinline__ uint32_t quantize_one(float v, float ratio, uint32_t word) {
  using F = Qsgd<BITS>;
  const float x = ratio * (float)F::kLevels;
  const float l = floorf(x);
  const float f = x - l;
  const float u = (float)(word >> 8) * (1.0f / 16777216.0f);
  const uint32_t level = (uint32_t)l + (u < f ? 1u : 0u);
  return (v < 0.0f ? F::kSign : 0u) | level;
}

// Smallest ratio the fp64 route below takes: its results lie in the normal
// fp32 range, where the bound of its proof holds. A nonnegative fp32 ratio r
// is in (0, kTinyRatio) iff bits(r) - 1 < kTinyBits - 1 as unsigned.
constexpr float kTinyRatio = 0x1p-100f;
constexpr uint32_t kTinyBits = 27u << 23;  // bits of 2^-100

// ratio[i] = |v[i]| / scale, correctly rounded to fp32, for a bucket scale
// (scale = max |v| over the bucket, so every ratio is in [0, 1]). The fp32
// quotient is taken as RN32(RN64(|v| * rs)) with rs = RN64(1 / scale): that
// approximation is within 2^-52 (relative) of the exact quotient, while an
// exact quotient of two fp32 numbers lies at least 2^-49 (relative) from
// every rounding boundary of fp32 (it is never a midpoint, and its distance
// to one is a nonzero integer over B * 2^(24 - e), B < 2^24 the divisor's
// significand), so both round to the same fp32 number. Ratios below
// kTinyRatio (none in practice) take the plain division instead. A scale of
// 0 gives ratio 0 (all values are zero).
template <int K>
__device__ __forceinline__ void ratios(const float (&v)[K], float scale, float (&ratio)[K]) {
  if (scale == 0.0f) {
#pragma unroll
    for (int i = 0; i < K; ++i) ratio[i] = 0.0f;
    return;
  }
  const double rs = 1.0 / (double)scale;
  bool tiny = false;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    ratio[i] = (float)((double)fabsf(v[i]) * rs);
    tiny |= __float_as_uint(ratio[i]) - 1u < kTinyBits - 1u;
  }
  if (__builtin_expect(__ballot(tiny) != 0ull, 0)) {
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (ratio[i] < kTinyRatio) ratio[i] = fabsf(v[i]) / scale;
  }
}

struct QArgs {
  uint32_t P;
  uint64_t n;
  uint32_t bucket;
  uint64_t nb;  // buckets per node
  uint64_t row_bytes;
  uint32_t key0, key1, step, node0;
};

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

// values off .. off+7 of a bucket of `len` values at `bp` (zeros past the end)
__device__ __forceinline__ void load8_rel(const float* bp, uint32_t off, uint32_t len, bool vec_ok, float v[8]) {
  if (vec_ok && off + 8 <= len) {
    const float4 a = *reinterpret_cast<const float4*>(bp + off);
    const float4 b = *reinterpret_cast<const float4*>(bp + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (off + i < len) ? bp[off + i] : 0.0f;
  }
}

// One wave per bucket: a wave-wide max gives the scale, then each lane turns
// 8 consecutive values into BITS bytes of codes (two Philox blocks). Buckets
// of up to HELD chunks of 512 values stay in registers between the max and
// the quantization (HELD = 0: read twice).
template <int BITS, int HELD>
__global__ __launch_bounds__(256) void k_qsgd(const float* __restrict__ val, uint8_t* __restrict__ codes,
                                              float* __restrict__ scales, QArgs A, const uint32_t* gate) {
  if (gate != nullptr && *gate == 0u) return;  // the result this would quantize is not dense
  const uint32_t p = blockIdx.y;
  const uint32_t lane = lane_id();
  const uint32_t node = A.node0 + p;
  const float* row = val + (uint64_t)p * A.n;
  uint8_t* crow = codes + (uint64_t)p * A.row_bytes;
  // bucket starts are multiples of 8 positions: 16-byte aligned when the row is
  const bool vec_ok = (((uint64_t)p * A.n) & 3u) == 0;
  const uint32_t lo = lane * kPerLane;  // the lane's first position in a chunk
  for (uint64_t j = (uint64_t)blockIdx.x * 4 + threadIdx.x / kWave; j < A.nb; j += (uint64_t)gridDim.x * 4) {
    const uint64_t b0 = j * A.bucket;
    const uint32_t len = (uint32_t)std::min<uint64_t>(A.bucket, A.n - b0);
    const float* bp = row + b0;
    float held[HELD ? HELD : 1][8];
    float m = 0.0f;
    if constexpr (HELD > 0) {
#pragma unroll
      for (int h = 0; h < HELD; ++h) {
        load8_rel(bp, h * kChunk + lo, len, vec_ok, held[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(held[h][i]));
      }
    } else {
      for (uint32_t c = 0; c < len; c += kChunk) {
        float v[8];
        load8_rel(bp, c + lo, len, vec_ok, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
      }
    }
    const float scale = wave_max(m);
    if (lane == 0) scales[(uint64_t)p * A.nb + j] = scale;

    auto quantize_chunk = [&](uint32_t c, const float (&v)[8]) {
      float ratio[8];
      ratios(v, scale, ratio);  // all lanes: it takes a wave-wide vote
      const uint32_t off = c + lo;
      if (off >= len) return;
      const uint64_t e = b0 + off;
      const uint32_t ctr = (uint32_t)(e >> 2);
      const Philox4 r0 = philox4x32_10(ctr, node, A.step, 0u, A.key0, A.key1);
      const Philox4 r1 = philox4x32_10(ctr + 1u, node, A.step, 0u, A.key0, A.key1);
      uint64_t packed = 0u;
      if (off + 8 <= len) {  // a whole group of eight
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t rnd = i < 4 ? r0.w[i] : r1.w[i - 4];
          packed |= (uint64_t)quantize_one<BITS>(v[i], ratio[i], rnd) << (BITS * i);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (off + i < len) {
            const uint32_t rnd = i < 4 ? r0.w[i] : r1.w[i - 4];
            packed |= (uint64_t)quantize_one<BITS>(v[i], ratio[i], rnd) << (BITS * i);
          }
        }
      }
      store_lane<BITS>(crow, e / 8 * BITS, A.row_bytes, packed, e + 8 <= A.n);
    };
    if constexpr (HELD > 0) {
#pragma unroll
      for (int h = 0; h < HELD; ++h)
        if ((uint32_t)h * kChunk < len) quantize_chunk(h * kChunk, held[h]);
    } else {
      for (uint32_t c = 0; c < len; c += kChunk) {
        float v[8];
        load8_rel(bp, c + lo, len, vec_ok, v);
        quantize_chunk(c, v);
      }
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
  // buckets of one or two chunks stay in registers
  const int held = bucket <= (uint32_t)kChunk ? 1 : bucket <= 2u * kChunk ? 2 : 0;
  auto go = [&](auto k) { return launch_ev(k, grid, dim3(256), stream, e0, e1, val, codes, scales, A, gate); };
  switch (bits * 4 + held) {
    case 2 * 4 + 0: return go(k_qsgd<2, 0>);
    case 2 * 4 + 1: return go(k_qsgd<2, 1>);
    case 2 * 4 + 2: return go(k_qsgd<2, 2>);
    case 4 * 4 + 0: return go(k_qsgd<4, 0>);
    case 4 * 4 + 1: return go(k_qsgd<4, 1>);
    case 4 * 4 + 2: return go(k_qsgd<4, 2>);
    case 8 * 4 + 0: return go(k_qsgd<8, 0>);
    case 8 * 4 + 1: return go(k_qsgd<8, 1>);
    case 8 * 4 + 2: return go(k_qsgd<8, 2>);
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
