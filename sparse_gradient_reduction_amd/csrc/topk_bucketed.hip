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
// One wave per bucket, B = 64 * E: lane l holds positions i*64 + l (i < E),
// so every load and store instruction moves 64 consecutive floats. The
// bucket's threshold is found by bisection over the key bits, counting with
// wave ballots (a vector compare and a scalar popcount per element slot); it
// stops as soon as some threshold has exactly k_j keys at or above it, which
// random data reaches after about half the bits. Otherwise the bisection
// ends on the k_j-th largest key itself and ties at it go to the lowest
// indices. Ranks of ties and output positions are mbcnt prefixes in index
// order. The whole bucket lives in registers: one HBM pass, 12 bytes per
// element plus 8 per kept pair.
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

template <int E>
__global__ __launch_bounds__(kBucketThreads) void k_topk_bucketed(const float* __restrict__ g,
                                                                  float* __restrict__ r,
                                                                  uint32_t* __restrict__ out_idx,
                                                                  float* __restrict__ out_val, BArgs A) {
  constexpr uint32_t B = (uint32_t)kWave * E;
  const uint64_t w = (uint64_t)blockIdx.x * kBucketWaves + uniform(threadIdx.x / kWave);
  if (w >= A.total_buckets) return;
  const uint64_t p = w / A.nb, j = w % A.nb;
  const uint64_t lo = j * B;
  const uint32_t len = (uint32_t)std::min<uint64_t>(B, A.N - lo);
  const uint64_t base = p * A.N + lo;
  const uint32_t lane = lane_id();

  // positions past the bucket get key 0 and are masked wherever 0 can count
  float a[E];
  uint32_t key[E];
  uint64_t vmask[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const uint32_t pos = (uint32_t)i * kWave + lane;
    const bool in = pos < len;
    vmask[i] = ballot_cmp(in);
    a[i] = in ? __builtin_nontemporal_load(g + base + pos) + __builtin_nontemporal_load(r + base + pos) : 0.0f;
    key[i] = in ? mag_key(a[i]) : 0u;
  }
  const uint32_t kj = std::min<uint32_t>(A.kb, len);

  uint64_t sel_mask[E];
  if (kj == 0) {
#pragma unroll
    for (int i = 0; i < E; ++i) sel_mask[i] = 0ull;
  } else {
    // largest T with count(key >= T) >= kj; stop early at an exact count.
    // Candidates are >= 1, so the zero keys of absent positions never count.
    uint32_t T = 0u;
    bool exact = (len == kj);
    for (int bit = 30; bit >= 0 && !exact; --bit) {
      const uint32_t cand = T | (1u << bit);
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < E; ++i) cnt += popc64(ballot_cmp(key[i] >= cand));
      if (cnt >= kj) {
        T = cand;
        exact = (cnt == kj);
      }
    }
    if (exact) {  // exactly kj keys are >= T: they are the selection (T = 0 only if the bucket is kept whole)
#pragma unroll
      for (int i = 0; i < E; ++i) sel_mask[i] = ballot_cmp(key[i] >= T) & vmask[i];
    } else {      // T is the kj-th largest key; m ties at T, lowest indices first
      uint32_t gt = 0;
#pragma unroll
      for (int i = 0; i < E; ++i) gt += popc64(ballot_cmp(key[i] > T));
      const uint32_t m = kj - gt;
      uint32_t eq_before = 0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const uint64_t em = ballot_cmp(key[i] == T) & vmask[i];
        const uint64_t gm = ballot_cmp(key[i] > T);
        // the first (m - eq_before) ties of this slot, in lane order
        const uint32_t take = m > eq_before ? m - eq_before : 0u;
        const bool tie_in = ((em >> lane) & 1ull) && lanes_below(em) < take;
        sel_mask[i] = gm | ballot_cmp(tie_in);
        eq_before += popc64(em);
      }
    }
  }

  const uint64_t out0 = p * A.K + j * A.kb;
  uint32_t sel_before = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const uint32_t pos = (uint32_t)i * kWave + lane;
    const bool sel = (sel_mask[i] >> lane) & 1ull;
    if (sel) {
      const uint64_t o = out0 + sel_before + lanes_below(sel_mask[i]);
      out_idx[o] = (uint32_t)(lo + pos);
      out_val[o] = a[i];
    }
    if (pos < len) __builtin_nontemporal_store(sel ? 0.0f : a[i], r + base + pos);
    sel_before += popc64(sel_mask[i]);
  }
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
  const dim3 grid((uint32_t)((A.total_buckets + kBucketWaves - 1) / kBucketWaves));
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
