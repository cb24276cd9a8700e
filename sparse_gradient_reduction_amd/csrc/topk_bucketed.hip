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
// vector compare and a scalar popcount per element slot), first bracketed
// below the bucket's largest magnitude (within half a binade when at most one
// in 16 is kept, else within a factor of about four); it stops as soon as
// some threshold has exactly k_j keys at or above it, else it ends on the
// k_j-th largest key itself and ties at it go to the lowest indices. Ranks of
// ties and output positions are mbcnt prefixes in index order. Buckets of 64
// and 128 share a wave (see k_topk_bucketed_small).
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
      // [M - 2^22, M] or [M - 2^24, M] below the largest key M, which usually
      // holds the kj-th largest; otherwise the whole key range.
      uint32_t mloc = 0;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int q = 0; q < V; ++q) mloc = max(mloc, key[c][q]);
      const uint32_t M = wave_max_u32(mloc);
      uint32_t lo_t = 0u, hi_t = M + 1u;  // count(key >= 0) = len >= kj; none is above M
      bool exact = (len == kj);
      // keeping at most 1 in 16, first try half a binade below M (2^22 key
      // units); then, or otherwise, about a factor of four (2^24)
      if (!exact && kj * 16u <= len && M > (1u << 22)) {
        const uint32_t guess = M - (1u << 22);
        const uint32_t n = count_ge(guess);
        if (n >= kj) {
          lo_t = guess;
          exact = (n == kj);
        } else {
          hi_t = guess;
        }
      }
      if (!exact && lo_t == 0u && M > (1u << 24)) {  // not tried, or held too few keys
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

// Sum / max over aligned groups of LG = 16 or 32 lanes, the result in every
// lane of the group: DPP within each row of 16 lanes (quad swaps, then row
// rotations by 4 and 8), and for 32-lane groups a swap of rows 0<->1 and
// 2<->3. Every lane of the group must be active.
template <uint32_t LG>
__device__ __forceinline__ uint32_t group_sum(uint32_t v) {
  static_assert(LG == 16 || LG == 32, "group of 16 or 32 lanes");
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);  // row_ror:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  if constexpr (LG == 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = s[0] + s[1];
  }
  return v;
}
template <uint32_t LG>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  static_assert(LG == 16 || LG == 32, "group of 16 or 32 lanes");
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  if constexpr (LG == 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(s[0], s[1]);
  }
  return v;
}

// Buckets of 64 and 128: a wave takes 256 consecutive positions, G = 256 / B
// buckets at once, lane l holding positions 4l..4l+3 (one float4 of each
// array). The lanes of one bucket form a group of 64 / G; each group runs its
// own threshold search, with counts summed across the group, and ranks come
// from ballots restricted to the group's lanes. Every cross-lane step runs
// with the whole wave active: the search loop runs while any group is still
// searching, and a finished group's lanes join its counts without using them.
template <int G>
__global__ __launch_bounds__(kBucketThreads) void k_topk_bucketed_small(const float* __restrict__ g,
                                                                        float* __restrict__ r,
                                                                        uint32_t* __restrict__ out_idx,
                                                                        float* __restrict__ out_val, BArgs A,
                                                                        uint64_t chunks_per_node,
                                                                        uint64_t total_chunks) {
  constexpr uint32_t B = 256 / G;     // bucket size
  constexpr uint32_t LG = kWave / G;  // lanes per bucket
  const uint32_t lane = lane_id();
  const uint32_t grp = lane / LG;
  const uint64_t gmask = ((1ull << LG) - 1ull) << (grp * LG);
  const uint64_t stride = (uint64_t)gridDim.x * kBucketWaves;
  for (uint64_t w = (uint64_t)blockIdx.x * kBucketWaves + uniform(threadIdx.x / kWave); w < total_chunks;
       w += stride) {
    const uint64_t p = w / chunks_per_node, c = w % chunks_per_node;
    const uint64_t j = c * G + grp;  // this lane's bucket
    const uint64_t cpos = c * 256;   // chunk start within the node
    const uint32_t clen = (uint32_t)std::min<uint64_t>(256, A.N - cpos);
    const float* gb = g + p * A.N + cpos;
    float* rb = r + p * A.N + cpos;
    const bool vec = ((reinterpret_cast<uintptr_t>(gb) | reinterpret_cast<uintptr_t>(rb)) & 15u) == 0;
    const uint32_t pos0 = lane * 4;  // within the chunk
    float a[4];
    uint32_t key[4];
    bool in[4];
    if (vec && pos0 + 4 <= clen) {
      const f32x4 x = load_nt(reinterpret_cast<const f32x4*>(gb + pos0));
      const f32x4 y = load_nt(reinterpret_cast<const f32x4*>(rb + pos0));
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = x[q] + y[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        a[q] = pos0 + q < clen ? __builtin_nontemporal_load(gb + pos0 + q) + __builtin_nontemporal_load(rb + pos0 + q)
                               : 0.0f;
    }
    uint32_t lmax = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      in[q] = pos0 + q < clen;
      key[q] = in[q] ? mag_key(a[q]) : 0u;
      lmax = max(lmax, key[q]);
    }
    // the group's bucket: its length (0 past the node's end) and kept count
    const uint64_t bstart = j * B;
    const uint32_t len = bstart < A.N ? (uint32_t)std::min<uint64_t>(B, A.N - bstart) : 0u;
    const uint32_t kj = std::min<uint32_t>(A.kb, len);
    auto count_ge = [&](uint32_t t) {  // keys >= t in the group; t >= 1 leaves out padding
      uint32_t n = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) n += key[q] >= t ? 1u : 0u;
      return group_sum<LG>(n);
    };
    const uint32_t M = group_max<LG>(lmax);
    // T = the kj-th largest key of the group, by binary search over [lo_t,
    // hi_t) with count(>= lo_t) >= kj > count(>= hi_t), first bracketed by
    // M - 2^24 (about a factor of four below the largest magnitude); it
    // stops at a threshold with exactly kj keys at or above it
    uint32_t lo_t = 0u, hi_t = M + 1u;
    bool exact = kj == 0u || len == kj;
    // a group keeping at most 1 in 16 first tries half a binade below M
    // (2^22 key units), then about a factor of four (2^24) if that holds
    // too few keys
    const uint32_t span1 = kj * 16u <= len ? (1u << 22) : (1u << 24);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const uint32_t span = pass == 0 ? span1 : (1u << 24);
      const bool try_guess = !exact && M > span && (pass == 0 || (span1 < span && hi_t == M - span1));
      if (pass == 1 && ballot(try_guess) == 0ull) break;  // no group's first guess held too few keys
      const uint32_t guess = try_guess ? M - span : 1u;
      const uint32_t n = count_ge(guess);
      if (try_guess) {
        if (n >= kj) {
          lo_t = guess;
          exact = n == kj;
        } else {
          hi_t = guess;
        }
      }
    }
    bool done = exact || hi_t - lo_t <= 1u;
    while (ballot(!done) != 0ull) {
      const uint32_t mid = lo_t + ((hi_t - lo_t) >> 1);  // >= 1 while searching
      const uint32_t n = count_ge(done ? 1u : mid);
      // a finished group keeps its bracket (no branch: the wave stays converged)
      const bool up = !done && n >= kj, down = !done && n < kj;
      lo_t = up ? mid : lo_t;
      hi_t = down ? mid : hi_t;
      exact = exact || (up && n == kj);
      done = exact || hi_t - lo_t <= 1u;
    }
    const uint32_t T = lo_t;
    // kept: with an exact count every key >= T (all of the bucket when T = 0);
    // otherwise T is the kj-th largest key, every key above it is kept and
    // the m ties at T at the lowest positions (a group ends that way only on
    // ties, so the wave usually skips that part)
    const uint64_t ex_lanes = ballot(exact);  // lanes of the groups with an exact count
    uint64_t sel[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sel[q] = ballot(kj > 0u && in[q] && key[q] >= T) & ex_lanes & gmask;
    if (ex_lanes != ~0ull) {
      uint32_t ngt = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) ngt += key[q] > T ? 1u : 0u;
      const uint32_t m = kj - std::min(kj, group_sum<LG>(ngt));
      uint64_t em[4];
      uint32_t tie_rank = 0;  // ties at T in lower lanes of the group
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        em[q] = ballot(in[q] && key[q] == T) & gmask;
        tie_rank += lanes_below(em[q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool eq = (em[q] >> lane) & 1ull;
        sel[q] |= ballot(key[q] > T || (eq && tie_rank < m)) & ~ex_lanes & gmask;
        tie_rank += eq ? 1u : 0u;
      }
    }
    uint32_t rank = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) rank += lanes_below(sel[q]);
    const uint64_t out0 = p * A.K + j * A.kb;
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool s_q = (sel[q] >> lane) & 1ull;
      if (s_q) {
        out_idx[out0 + rank] = (uint32_t)(cpos + pos0 + q);
        out_val[out0 + rank] = a[q];
        ++rank;
      }
      o[q] = s_q ? 0.0f : a[q];
    }
    if (vec && pos0 + 4 <= clen) {
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = o[q];
      store_nt(v, reinterpret_cast<f32x4*>(rb + pos0));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (in[q]) __builtin_nontemporal_store(o[q], rb + pos0 + q);
    }
  }  // chunks of this wave
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
  // buckets of 64 and 128: one wave per 256 positions
  const uint64_t cpn = (N + 255) / 256, chunks = (uint64_t)P * cpn;
  const dim3 grid_small((uint32_t)std::min<uint64_t>((chunks + kBucketWaves - 1) / kBucketWaves, 1u << 23));
  switch (bucket) {
    case 64:
      hipLaunchKernelGGL(k_topk_bucketed_small<4>, grid_small, block, 0, stream, grad, residual, out_idx, out_val, A,
                         cpn, chunks);
      break;
    case 128:
      hipLaunchKernelGGL(k_topk_bucketed_small<2>, grid_small, block, 0, stream, grad, residual, out_idx, out_val, A,
                         cpn, chunks);
      break;
    case 256: hipLaunchKernelGGL(k_topk_bucketed<4>, grid, block, 0, stream, grad, residual, out_idx, out_val, A); break;
    case 512: hipLaunchKernelGGL(k_topk_bucketed<8>, grid, block, 0, stream, grad, residual, out_idx, out_val, A); break;
    case 1024: hipLaunchKernelGGL(k_topk_bucketed<16>, grid, block, 0, stream, grad, residual, out_idx, out_val, A); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sparcml
