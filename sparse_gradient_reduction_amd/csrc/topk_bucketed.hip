// Bucketed error-feedback Top-k for gfx950.
//
// SparCML (paperlayer.ai digest of arXiv 1802.08021v3), section 8.3: the
// CIFAR-10 runs keep k entries out of every 512 (16/512 and 8/512); section
// 2.2: the kept entries are the largest in magnitude, the rest accumulate;
// section 4: the unapplied part is carried as residual error.
//
// Per node, the N positions form buckets of B consecutive positions (the
// last one partial); bucket j keeps k_j = min(k, len_j) positions, the first
// under (key descending, index ascending), key = bits(a) & 0x7FFFFFFF with
// a = grad + residual. Output rows concatenate the buckets' selections in
// index order (bucket j's pairs start at j * min(k, B)); the residual is a
// with +0 at the selected positions.
//
// One wave per bucket of B = 64 * E positions, held in registers: one HBM
// pass, 12 bytes per element plus 8 per kept pair. The bucket's threshold is
// found by binary search over key values, counting with wave ballots (a
// vector compare and a scalar popcount per element slot), first within a
// factor of four below the bucket's largest magnitude; it stops as soon as
// some threshold has exactly k_j keys at or above it, else it ends on the
// k_j-th largest key itself and ties at it go to the lowest indices. Ranks of
// ties and output positions are mbcnt prefixes in index order.
#include "device_common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace sparcml {
namespace {

constexpr int kBucketThreads = 256;
constexpr int kBucketWaves = kBucketThreads / kWave;

struct BArgs {
  uint64_t N;
  uint64_t nb;             // buckets per node
  uint64_t total_buckets;  // P * nb
  uint64_t K;              // pairs per node
  uint32_t kb;             // pairs kept per whole bucket, min(k, B)
  uint32_t pad;
};

// wave-uniform value held in a scalar register
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// ballot straight from a vector compare
__device__ __forceinline__ uint64_t ballot_cmp(bool c) { return __builtin_amdgcn_ballot_w64(c); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v = max(v, (uint32_t)__shfl_xor(v, d, kWave));
  return uniform(v);
}

// Lane l holds, for chunk c < E/V and q < V, position c*64*V + l*V + q: with
// V = 4 (buckets of 256 and more) every lane moves 16 bytes per instruction,
// with V = 1 each instruction moves 64 consecutive floats.
template <int E>
__global__ __launch_bounds__(kBucketThreads) void k_topk_bucketed(const float* __restrict__ g,
                                                                  float* __restrict__ r,
                                                                  uint32_t* __restrict__ out_idx,
                                                                  float* __restrict__ out_val, BArgs A) {
  constexpr uint32_t B = (uint32_t)kWave * E;
  constexpr int V = E >= 4 ? 4 : 1;
  constexpr int C = E / V;
  const uint32_t lane = lane_id();
  const uint64_t stride = (uint64_t)gridDim.x * kBucketWaves;
  for (uint64_t w = (uint64_t)blockIdx.x * kBucketWaves + uniform(threadIdx.x / kWave); w < A.total_buckets;
       w += stride) {
    const uint64_t p = w / A.nb, j = w % A.nb;
    const uint64_t lo = j * B;
    const uint32_t len = (uint32_t)std::min<uint64_t>(B, A.N - lo);
    const float* gb = g + p * A.N + lo;
    float* rb = r + p * A.N + lo;
    const bool vec = V == 4 && ((reinterpret_cast<uintptr_t>(gb) | reinterpret_cast<uintptr_t>(rb)) & 15u) == 0;

    // positions past the bucket get key 0 and are masked wherever 0 can count
    float a[C][V];
    uint32_t key[C][V];
    uint64_t vmask[C][V];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint32_t pos0 = (uint32_t)c * kWave * V + lane * V;
      if (vec && pos0 + V <= len) {
        const f32x4 x = load_nt(reinterpret_cast<const f32x4*>(gb + pos0));
        const f32x4 y = load_nt(reinterpret_cast<const f32x4*>(rb + pos0));
#pragma unroll
        for (int q = 0; q < V; ++q) a[c][q] = x[q] + y[q];
      } else {
#pragma unroll
        for (int q = 0; q < V; ++q)
          a[c][q] = pos0 + q < len ? __builtin_nontemporal_load(gb + pos0 + q) + __builtin_nontemporal_load(rb + pos0 + q)
                                   : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const bool in = pos0 + q < len;
        vmask[c][q] = ballot_cmp(in);
        key[c][q] = in ? mag_key(a[c][q]) : 0u;
      }
    }
    const uint32_t kj = std::min<uint32_t>(A.kb, len);
    auto count_ge = [&](uint32_t t) {  // keys >= t, for t >= 1
      uint32_t n = 0;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int q = 0; q < V; ++q) n += popc64(ballot_cmp(key[c][q] >= t));
      return n;
    };

    uint64_t sel_mask[C][V];
    if (kj == 0) {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int q = 0; q < V; ++q) sel_mask[c][q] = 0ull;
    } else {
      // T = the kj-th largest key, by binary search over [lo_t, hi_t) with
      // count(key >= lo_t) >= kj > count(key >= hi_t); it stops early at a
      // threshold with exactly kj keys at or above it. The first bracket is
      // [M - 2^24, M]: a factor of about four below the largest key M, which
      // usually holds the kj-th largest; otherwise the whole key range.
      uint32_t mloc = 0;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int q = 0; q < V; ++q) mloc = max(mloc, key[c][q]);
      const uint32_t M = wave_max_u32(mloc);
      uint32_t lo_t = 0u, hi_t = M + 1u;  // count(key >= 0) = len >= kj; none is above M
      bool exact = (len == kj);
      if (!exact && M > (1u << 24)) {
        const uint32_t guess = M - (1u << 24);
        const uint32_t n = count_ge(guess);
        if (n >= kj) {
          lo_t = guess;
          exact = (n == kj);
        } else {
          hi_t = guess;
        }
      }
      while (!exact && hi_t - lo_t > 1u) {
        const uint32_t mid = lo_t + ((hi_t - lo_t) >> 1);  // >= 1
        const uint32_t n = count_ge(mid);
        if (n >= kj) {
          lo_t = mid;
          exact = (n == kj);
        } else {
          hi_t = mid;
        }
      }
      const uint32_t T = lo_t;
      if (exact) {  // exactly kj keys are >= T: they are the selection (T = 0 only if the bucket is kept whole)
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int q = 0; q < V; ++q) sel_mask[c][q] = ballot_cmp(key[c][q] >= T) & vmask[c][q];
      } else {      // T is the kj-th largest key; m ties at T go to the lowest positions
        uint32_t gt = 0;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int q = 0; q < V; ++q) gt += popc64(ballot_cmp(key[c][q] > T));
        const uint32_t m = kj - gt;
        uint32_t eq_before = 0;  // ties in earlier chunks
#pragma unroll
        for (int c = 0; c < C; ++c) {
          uint64_t em[V];
          uint32_t below = 0, chunk = 0;  // ties of this chunk in lower lanes / in all lanes
#pragma unroll
          for (int q = 0; q < V; ++q) {
            em[q] = ballot_cmp(key[c][q] == T) & vmask[c][q];
            below += lanes_below(em[q]);
            chunk += popc64(em[q]);
          }
          uint32_t rank = eq_before + below;  // ties at lower positions than this lane's first
#pragma unroll
          for (int q = 0; q < V; ++q) {
            const bool eq = (em[q] >> lane) & 1ull;
            const bool take = eq && rank < m;
            sel_mask[c][q] = ballot_cmp(key[c][q] > T) | ballot_cmp(take);
            rank += eq ? 1u : 0u;
          }
          eq_before += chunk;
        }
      }
    }

    const uint64_t out0 = p * A.K + j * A.kb;
    uint32_t sel_before = 0;  // selected in earlier chunks
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint32_t pos0 = (uint32_t)c * kWave * V + lane * V;
      uint32_t rank = sel_before, chunk = 0;
#pragma unroll
      for (int q = 0; q < V; ++q) {
        rank += lanes_below(sel_mask[c][q]);
        chunk += popc64(sel_mask[c][q]);
      }
      float o[V];
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const bool sel = (sel_mask[c][q] >> lane) & 1ull;
        if (sel) {
          out_idx[out0 + rank] = (uint32_t)(lo + pos0 + q);
          out_val[out0 + rank] = a[c][q];
          ++rank;
        }
        o[q] = sel ? 0.0f : a[c][q];
      }
      if (vec && pos0 + V <= len) {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < V; ++q) v[q] = o[q];
        store_nt(v, reinterpret_cast<f32x4*>(rb + pos0));
      } else {
#pragma unroll
        for (int q = 0; q < V; ++q)
          if (pos0 + q < len) __builtin_nontemporal_store(o[q], rb + pos0 + q);
      }
      sel_before += chunk;
    }
  }  // buckets of this wave
}

}  // namespace

uint64_t topk_bucketed_count(uint64_t N, uint32_t bucket, uint32_t k) {
  if (N == 0) return 0;
  const uint64_t nb = (N + bucket - 1) / bucket;
  const uint64_t last = N - (nb - 1) * bucket;
  return (nb - 1) * std::min<uint64_t>(k, bucket) + std::min<uint64_t>(k, last);
}

hipError_t topk_bucketed_launch(uint32_t P, uint64_t N, uint32_t bucket, uint32_t k, const float* grad,
                                float* residual, uint32_t* out_idx, float* out_val, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  BArgs A;
  A.N = N;
  A.nb = (N + bucket - 1) / bucket;
  A.total_buckets = (uint64_t)P * A.nb;
  A.K = topk_bucketed_count(N, bucket, k);
  A.kb = std::min<uint32_t>(k, bucket);
  A.pad = 0;
  // one bucket per wave, up to the 2^32 work-items a grid dimension allows;
  // beyond that the waves loop
  const dim3 grid((uint32_t)std::min<uint64_t>((A.total_buckets + kBucketWaves - 1) / kBucketWaves, 1u << 23));
  const dim3 block(kBucketThreads);
  switch (bucket) {
    case 64: hipLaunchKernelGGL(k_topk_bucketed<1>, grid, block, 0, stream, grad, residual, out_idx, out_val, A); break;
    case 128: hipLaunchKernelGGL(k_topk_bucketed<2>, grid, block, 0, stream, grad, residual, out_idx, out_val, A); break;
    case 256: hipLaunchKernelGGL(k_topk_bucketed<4>, grid, block, 0, stream, grad, residual, out_idx, out_val, A); break;
    case 512: hipLaunchKernelGGL(k_topk_bucketed<8>, grid, block, 0, stream, grad, residual, out_idx, out_val, A); break;
    case 1024: hipLaunchKernelGGL(k_topk_bucketed<16>, grid, block, 0, stream, grad, residual, out_idx, out_val, A); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sparcml
