// Device helpers shared by the gfx950 kernels: wave64 ballots and prefix
// counts, block-wide scans through LDS, and the magnitude key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparcml {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load and store: the data is touched once.
__device__ __forceinline__ f32x4 load_nt(const f32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(f32x4 v, f32x4* p) { __builtin_nontemporal_store(v, p); }

// MI355X spreads consecutive workgroups of a launch round-robin over its 8
// XCDs, each with its own L2. For kernels whose neighbouring work items share
// cache lines at their edges, this maps the launch-order block id b (of B) to
// a work item so that each XCD walks one contiguous range of work items.
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t b, uint32_t B) {
  const uint32_t xcd = b % kXcds, i = b / kXcds;
  const uint32_t per = B / kXcds, rem = B % kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + i;
}

// |a| ordering key: the IEEE bit pattern with the sign cleared. For finite
// values it is monotone in |a|, and -0 and +0 share key 0.
__device__ __forceinline__ uint32_t mag_key(float a) {
  return __float_as_uint(a) & 0x7FFFFFFFu;
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool pred) { return __ballot(pred); }

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

// The value of the lane below (0 in lane 0), by a DPP whole-wave shift right
// by one lane: one VALU instruction, no LDS permute.
__device__ __forceinline__ uint32_t from_lane_below(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xF, 0xF, false);  // wave_shr:1
}

// Inclusive prefix sum across the 64 lanes of a wave (all lanes active):
// shifts by 1, 2, 4 and 8 lanes within each row of 16 (DPP row_shr, lanes
// without a source add 0), then each row adds the totals of the rows below,
// read from lanes 15, 31 and 47.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t row = lane_id() >> 4;
  return v + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

// Sum over the 64 lanes of a wave (all lanes active), the same in every lane:
// DPP sums within each row of 16, then the four row sums.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);  // row_ror:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// Maximum over the 64 lanes of a wave (all lanes active), the same in every
// lane: DPP maxima within each row of 16, then the four row maxima.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));  // quad_perm [1,0,3,2]
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));  // quad_perm [2,3,0,1]
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));  // row_ror:4
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));  // row_ror:8
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// hist[bin] += 1 for every active lane with `valid`. The bins of the first
// CAP distinct bins met (lowest lanes first) take one LDS atomic each for all
// their lanes; the lanes left over add one by one. Keys near a selection
// threshold crowd into a few bins, where per-lane atomics would serialise;
// where they spread, a leader loop over every distinct bin would cost more.
template <int CAP>
__device__ __forceinline__ void wave_hist_add_capped(uint32_t* hist, uint32_t bin, bool valid) {
  uint64_t todo = ballot(valid);
#pragma unroll
  for (int i = 0; i < CAP; ++i) {
    if (!todo) return;
    const int leader = __ffsll((long long)todo) - 1;
    const uint32_t b = __builtin_amdgcn_readlane(bin, leader);  // leader is wave-uniform
    const uint64_t same = ballot(valid && bin == b) & todo;
    if (lane_id() == (uint32_t)leader) atomicAdd(&hist[b], popc64(same));
    todo &= ~same;
  }
  if ((todo >> lane_id()) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Sum of (a, b) over the block. `scratch` holds 2 * NT/64 words of LDS.
// Contains barriers: all threads of the block must call it.
template <int NT>
__device__ __forceinline__ void block_sum2(uint32_t a, uint32_t b, uint32_t* scratch, uint32_t& sa, uint32_t& sb) {
  constexpr int NW = NT / kWave;
  a = wave_sum(a);
  b = wave_sum(b);
  const uint32_t wid = threadIdx.x / kWave;
  if (lane_id() == 0) {
    scratch[wid] = a;
    scratch[NW + wid] = b;
  }
  __syncthreads();
  sa = 0;
  sb = 0;
  for (int w = 0; w < NW; ++w) {
    sa += scratch[w];
    sb += scratch[NW + w];
  }
  __syncthreads();
}

// Exclusive prefix sum over the threads of a block (thread order), with the
// block total. `scratch` holds NT/64 + 1 words of LDS. Contains barriers: all
// threads of the block must call it. Every wave adds up the wave totals
// itself, so one barrier separates their writes from the reads, and one more
// lets the caller reuse `scratch` right away.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
  constexpr int NW = NT / kWave;
  const uint32_t wid = threadIdx.x / kWave;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane_id() == kWave - 1) scratch[wid] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = scratch[w];
    before += (uint32_t)w < wid ? t : 0u;
    all += t;
  }
  total = all;
  __syncthreads();
  return before + inc - v;
}

// 64-bit exclusive prefix sum across a workgroup of NT threads; every
// thread gets `total`. scratch holds NT / kWave + 1 values.
template <int NT>
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* scratch, uint64_t& total) {
  constexpr int NW = NT / kWave;
  const uint32_t lane = lane_id();
  const uint32_t wid = threadIdx.x / kWave;
  uint64_t inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint64_t t = __shfl_up(inc, d, kWave);
    if (lane >= (uint32_t)d) inc += t;
  }
  if (lane == kWave - 1) scratch[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t run = 0;
    for (int w = 0; w < NW; ++w) {
      const uint64_t t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[NW] = run;
  }
  __syncthreads();
  const uint64_t excl = scratch[wid] + inc - v;
  total = scratch[NW];
  __syncthreads();
  return excl;
}

// Radix-select step over a histogram of NB bins whose counts each thread
// holds: c[i] is bin NB-1-t*per-i for thread t (per = NB/NT), the layout
// load_suffix_bins reads. Finds the highest bin b such that the count of items
// in bins >= b reaches `rank` (1-based, rank >= 1), and the count in bins
// strictly above b. If the histogram holds fewer than `rank` items, returns
// bin 0 with `above` = total of bins > 0. `scratch` holds NT/64 + 3 words of
// LDS. All threads call it; all receive the result.
template <int NT, int NB>
__device__ __forceinline__ void block_find_suffix_held(const uint32_t (&c)[NB / NT], uint32_t rank,
                                                       uint32_t* scratch, uint32_t& bin, uint32_t& above) {
  static_assert(NB % NT == 0, "whole bins per thread");
  constexpr int per = NB / NT;
  const int top = NB - 1 - (int)threadIdx.x * per;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) s += c[i];
  uint32_t total;
  const uint32_t before = block_exclusive_scan<NT>(s, scratch, total);
  constexpr int NW = NT / kWave;
  if (threadIdx.x == NT - 1) {  // holds bin 0 as c[per - 1]
    scratch[NW + 1] = 0u;
    scratch[NW + 2] = total - c[per - 1];
  }
  __syncthreads();
  if (before < rank && before + s >= rank) {
    uint32_t run = before;
    bool found = false;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (!found && run + c[i] >= rank) {
        scratch[NW + 1] = (uint32_t)(top - i);
        scratch[NW + 2] = run;
        found = true;
      }
      run += c[i];
    }
  }
  __syncthreads();
  bin = scratch[NW + 1];
  above = scratch[NW + 2];
  __syncthreads();
}

// This thread's bins of an NB-bin histogram in the block_find_suffix_held
// layout (all loads issued at once).
template <int NT, int NB>
__device__ __forceinline__ void load_suffix_bins(const uint32_t* hist, uint32_t (&c)[NB / NT]) {
  constexpr int per = NB / NT;
  const int top = NB - 1 - (int)threadIdx.x * per;
#pragma unroll
  for (int i = 0; i < per; ++i) c[i] = hist[top - i];
}

// block_find_suffix_held over a histogram in memory (LDS or global).
template <int NT, int NB>
__device__ __forceinline__ void block_find_suffix(const uint32_t* hist, uint32_t rank, uint32_t* scratch,
                                                  uint32_t& bin, uint32_t& above) {
  uint32_t c[NB / NT];
  load_suffix_bins<NT, NB>(hist, c);
  block_find_suffix_held<NT, NB>(c, rank, scratch, bin, above);
}

}  // namespace sparcml
