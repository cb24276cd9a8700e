// Sparse reduction with the dense switch, for gfx950.
//
// SparCML (paperlayer.ai digest of arXiv 1802.08021v3): section 5.1, sparse
// streams of index-value pairs that switch to a dense layout past delta;
// section 5.2, a coordinate-wise sum with neutral element 0; section 5.3, a
// rough estimate of the result size K picks the algorithm and the result is
// dense once K reaches delta; section 5.3.2, the split phase gives each owner
// one index range; Appendix B, K is the size of the union of the index sets.
//
// One GPU holds all P contributions. The index space is cut into segments of
// 8192 indices, the one-GPU analogue of the split phase's index-range owners;
// a workgroup owns one segment, takes each node's sub-run of pairs falling in
// it, and merges them by scatter-adding into an LDS-resident fp64 tile of the
// segment with an occupancy bitmap beside it (ds_add_f64 makes the sums
// independent of arrival order up to fp64 rounding; the result is rounded to
// fp32 once). An ordered compaction of the bitmap then emits the segment's
// part of the sorted sparse result, or the tile is written densely.
//
//   setup    offsets into the workspace (passed inline, 256 nodes per launch),
//            state cleared
//   bounds   node-major streaming pass over the indices: where each node's
//            run crosses a segment boundary; checks range and order
//   count    (count-first) per segment: union size from the LDS bitmap
//   decide   exclusive scan of segment counts, K, dense iff K >= T
//   write    per segment: fp64 LDS accumulate, then dense tile or compacted
//            sparse pairs at the segment's offset
// Dense-first (estimate >= T): write<dense> also counts; decide; a sparse
// rewrite runs only if the exact K turned out below T.
#include "device_common.hpp"
#include "kernels.hpp"
#include "sparcml.h"

#include <algorithm>

namespace sparcml {
namespace {

constexpr int kSegBits = 13;
constexpr uint32_t kSeg = 1u << kSegBits;  // 8192 indices per segment
constexpr int kThreads = 256;              // bounds / count kernels
constexpr int kWriteThreads = 1024;        // write kernel: 16 waves hide the load latency
constexpr int kWords = kSeg / 32;          // bitmap words per segment (== kThreads)
constexpr uint32_t kMaxP = 1024;
constexpr int kInlineOffsets = 256;

static_assert(kWords == kThreads, "one bitmap word per thread");

struct State {
  uint32_t flags;
  uint32_t is_dense;
  uint64_t K;
};

struct Layout {
  uint64_t S;  // segments
  size_t state, offs, bounds, cnt, off, total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout make_layout(uint32_t P, uint64_t N) {
  Layout L{};
  L.S = (N + kSeg - 1) / kSeg;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.state = take(sizeof(State));
  L.offs = take(8ull * (P + 1));
  L.bounds = take(4ull * P * (L.S + 1));
  L.cnt = take(4ull * L.S);
  L.off = take(4ull * L.S);
  L.total = o;
  return L;
}

struct RDev {
  uint32_t P;
  uint32_t N;
  uint64_t S;
  uint64_t T;
  uint64_t out_idx_cap;
  State* state;
  uint64_t* offs;
  uint32_t* bounds;
  uint32_t* cnt;
  uint32_t* off;
  ReduceResultDev* result;
};

struct InlineOffsets {
  uint64_t v[kInlineOffsets];
};

__global__ void k_setup(RDev R, uint32_t first, uint32_t count, InlineOffsets in, int clear) {
  for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) R.offs[first + i] = in.v[i];
  if (clear && threadIdx.x == 0) {
    R.state->flags = 0u;
    R.state->is_dense = 0u;
    R.state->K = 0ull;
  }
}

// Node-major pass: bounds[p][s] = number of node p's pairs with index < s*8192
// (s = S stands for N), written by the pair where the run crosses into s.
// Each thread takes 4 consecutive pairs, so every index is loaded once by the
// thread that owns it and once more as the left neighbour of the next group.
__global__ __launch_bounds__(kThreads) void k_bounds(const uint32_t* __restrict__ idx, RDev R) {
  constexpr int kPer = 4;
  const uint32_t p = blockIdx.y;
  const uint64_t o0 = R.offs[p];
  const uint64_t nnz = R.offs[p + 1] - o0;
  const uint64_t S = R.S;
  uint32_t* b = R.bounds + (uint64_t)p * (S + 1);
  uint32_t bad = 0u;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads * kPer;
  for (uint64_t j0 = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * kPer; j0 < nnz; j0 += stride) {
    uint32_t v[kPer + 1];
    v[0] = j0 > 0 ? idx[o0 + j0 - 1] : 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) v[u + 1] = j0 + u < nnz ? idx[o0 + j0 + u] : 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint64_t j = j0 + u;
      if (j >= nnz) break;
      const uint32_t i = v[u + 1];
      const uint64_t s_cur = i >= R.N ? S : (i >> kSegBits);
      if (i >= R.N) bad |= SPARCML_FLAG_INDEX_RANGE;
      int64_t s_prev = -1;
      if (j > 0) {
        const uint32_t ip = v[u];
        if (ip >= i) bad |= SPARCML_FLAG_NOT_ASCENDING;
        s_prev = ip >= R.N ? (int64_t)S : (int64_t)(ip >> kSegBits);
      }
      for (int64_t s = s_prev + 1; s <= (int64_t)s_cur; ++s) b[s] = (uint32_t)j;
      if (j + 1 == nnz)
        for (uint64_t s = s_cur + 1; s <= S; ++s) b[s] = (uint32_t)nnz;
    }
  }
  if (bad) atomicOr(&R.state->flags, bad);
}

// Node sub-runs of segment s: pre[p] = exclusive prefix of their lengths,
// start[p] = absolute index of the first pair. Returns the segment's pair count.
template <int NT>
__device__ __forceinline__ uint32_t load_runs(const RDev& R, uint64_t s, uint32_t* pre, uint32_t* start,
                                              uint32_t* scr) {
  uint32_t carry = 0;
  for (uint32_t p0 = 0; p0 < R.P; p0 += NT) {
    const uint32_t p = p0 + threadIdx.x;
    uint32_t len = 0;
    if (p < R.P) {
      const uint64_t o0 = R.offs[p];
      const uint64_t nnz = R.offs[p + 1] - o0;
      const uint32_t* b = R.bounds + (uint64_t)p * (R.S + 1);
      const uint64_t b0 = std::min<uint64_t>(b[s], nnz);
      const uint64_t b1 = std::min<uint64_t>(b[s + 1], nnz);
      len = b1 > b0 ? (uint32_t)(b1 - b0) : 0u;
      start[p] = (uint32_t)(o0 + b0);
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<NT>(len, scr, tot);
    if (p < R.P) pre[p] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) pre[R.P] = carry;
  __syncthreads();
  return carry;
}

// largest p with pre[p] <= f (pre is nondecreasing, pre[0] = 0, f < pre[P])
__device__ __forceinline__ uint32_t find_node(const uint32_t* pre, uint32_t P, uint32_t f) {
  uint32_t lo = 0, hi = P;  // invariant: pre[lo] <= f < pre[hi]
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (pre[mid] <= f) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void k_count(const uint32_t* __restrict__ idx, RDev R) {
  __shared__ uint32_t bits[kWords];
  __shared__ uint32_t pre[kMaxP + 1];
  __shared__ uint32_t start[kMaxP];
  __shared__ uint32_t scr[kThreads / kWave + 3];
  const uint64_t s = blockIdx.x;
  const uint32_t seg_lo = (uint32_t)(s << kSegBits);
  const uint32_t seg_len = std::min<uint32_t>(kSeg, R.N - seg_lo);
  bits[threadIdx.x] = 0u;
  const uint32_t total = load_runs<kThreads>(R, s, pre, start, scr);
  constexpr int kBatch = 16;
  for (uint32_t f0 = 0; f0 < total; f0 += kThreads * kBatch) {
    uint32_t ii[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint32_t f = f0 + b * kThreads + threadIdx.x;
      ii[b] = 0xFFFFFFFFu;
      if (f < total) {
        const uint32_t p = find_node(pre, R.P, f);
        ii[b] = idx[start[p] + (f - pre[p])];
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint32_t local = ii[b] - seg_lo;
      if (ii[b] != 0xFFFFFFFFu && local < seg_len) atomicOr(&bits[local >> 5], 1u << (local & 31));
    }
  }
  __syncthreads();
  uint32_t tot;
  block_exclusive_scan<kThreads>((uint32_t)__popc(bits[threadIdx.x]), scr, tot);
  if (threadIdx.x == 0) R.cnt[s] = tot;
}

__global__ __launch_bounds__(1024) void k_decide(RDev R) {
  __shared__ uint32_t scr[1024 / kWave + 3];
  uint64_t carry = 0;
  for (uint64_t s0 = 0; s0 < R.S; s0 += 1024) {
    const uint64_t s = s0 + threadIdx.x;
    const uint32_t c = s < R.S ? R.cnt[s] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<1024>(c, scr, tot);
    if (s < R.S) R.off[s] = (uint32_t)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) {
    const uint32_t dense = carry >= R.T ? 1u : 0u;
    R.state->K = carry;
    R.state->is_dense = dense;
    ReduceResultDev res;
    res.nnz = carry;
    res.is_dense = dense;
    res.flags = R.state->flags;
    *R.result = res;
  }
}

enum WriteMode { kDecided = 0, kDenseFirst = 1, kSparseOnly = 2 };

template <int MODE>
__global__ __launch_bounds__(kWriteThreads) void k_write(const uint32_t* __restrict__ idx,
                                                         const float* __restrict__ val,
                                                         uint32_t* __restrict__ out_idx, float* __restrict__ out_val,
                                                         RDev R) {
  __shared__ double acc[kSeg];
  __shared__ uint32_t bits[kWords];
  __shared__ uint32_t pre[kMaxP + 1];
  __shared__ uint32_t start[kMaxP];
  __shared__ uint32_t scr[kWriteThreads / kWave + 3];
  const uint64_t s = blockIdx.x;
  bool dense;
  if (MODE == kDenseFirst) {
    dense = true;
  } else {
    dense = R.state->is_dense != 0u;
    if (MODE == kSparseOnly && dense) return;
    if (!dense && R.cnt[s] == 0u) return;
  }
  const uint32_t seg_lo = (uint32_t)(s << kSegBits);
  const uint32_t seg_len = std::min<uint32_t>(kSeg, R.N - seg_lo);
  for (uint32_t i = threadIdx.x; i < kSeg; i += kWriteThreads) acc[i] = 0.0;
  if (threadIdx.x < kWords) bits[threadIdx.x] = 0u;
  const uint32_t total = load_runs<kWriteThreads>(R, s, pre, start, scr);

  constexpr int kBatch = 8;
  for (uint32_t f0 = 0; f0 < total; f0 += kWriteThreads * kBatch) {
    uint32_t ii[kBatch];
    float vv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint32_t f = f0 + b * kWriteThreads + threadIdx.x;
      ii[b] = 0xFFFFFFFFu;
      vv[b] = 0.0f;
      if (f < total) {
        const uint32_t p = find_node(pre, R.P, f);
        const uint32_t j = start[p] + (f - pre[p]);
        ii[b] = idx[j];
        vv[b] = val[j];
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint32_t local = ii[b] - seg_lo;
      if (ii[b] != 0xFFFFFFFFu && local < seg_len) {
        atomicAdd(&acc[local], (double)vv[b]);
        atomicOr(&bits[local >> 5], 1u << (local & 31));
      }
    }
  }
  __syncthreads();

  // one bitmap word (32 indices) per thread for the first kWords threads
  const uint32_t word = threadIdx.x < kWords ? bits[threadIdx.x] : 0u;
  uint32_t seg_total;
  const uint32_t ex = block_exclusive_scan<kWriteThreads>((uint32_t)__popc(word), scr, seg_total);
  if (MODE == kDenseFirst && threadIdx.x == 0) R.cnt[s] = seg_total;

  if (dense) {
    float* out = out_val + seg_lo;
    if (seg_len == kSeg) {
      for (uint32_t q = threadIdx.x; q < kSeg / 4; q += kWriteThreads) {
        const float4 o = make_float4((float)acc[4 * q], (float)acc[4 * q + 1], (float)acc[4 * q + 2],
                                     (float)acc[4 * q + 3]);
        reinterpret_cast<float4*>(out)[q] = o;
      }
    } else {
      for (uint32_t i = threadIdx.x; i < seg_len; i += kWriteThreads) out[i] = (float)acc[i];
    }
  } else {
    uint64_t pos = (uint64_t)R.off[s] + ex;
    uint32_t w = word;
    while (w) {
      const uint32_t b = __ffs(w) - 1;
      w &= w - 1;
      const uint32_t local = threadIdx.x * 32 + b;
      if (pos < R.out_idx_cap) {
        out_idx[pos] = seg_lo + local;
        out_val[pos] = (float)acc[local];
      }
      ++pos;
    }
  }
}

}  // namespace

size_t reduce_workspace_bytes(uint32_t P, uint64_t N, uint64_t /*total_nnz*/) { return make_layout(P, N).total; }

hipError_t sparse_reduce_launch(uint32_t P, uint64_t N, uint64_t T, const uint64_t* h_offsets,
                                const uint32_t* idx, const float* val, bool dense_first,
                                uint32_t* out_idx, uint64_t out_idx_cap, float* out_val,
                                ReduceResultDev* d_result, void* ws, hipStream_t stream) {
  const Layout L = make_layout(P, N);
  char* w = static_cast<char*>(ws);
  RDev R;
  R.P = P;
  R.N = (uint32_t)N;
  R.S = L.S;
  R.T = T;
  R.out_idx_cap = out_idx_cap;
  R.state = reinterpret_cast<State*>(w + L.state);
  R.offs = reinterpret_cast<uint64_t*>(w + L.offs);
  R.bounds = reinterpret_cast<uint32_t*>(w + L.bounds);
  R.cnt = reinterpret_cast<uint32_t*>(w + L.cnt);
  R.off = reinterpret_cast<uint32_t*>(w + L.off);
  R.result = d_result;

  uint64_t max_nnz = 0;
  for (uint32_t p = 0; p < P; ++p) max_nnz = std::max<uint64_t>(max_nnz, h_offsets[p + 1] - h_offsets[p]);

  for (uint32_t first = 0; first < P + 1; first += kInlineOffsets) {
    InlineOffsets in;
    const uint32_t count = std::min<uint32_t>(kInlineOffsets, P + 1 - first);
    for (uint32_t i = 0; i < count; ++i) in.v[i] = h_offsets[first + i];
    hipLaunchKernelGGL(k_setup, dim3(1), dim3(256), 0, stream, R, first, count, in, first == 0 ? 1 : 0);
  }
  const uint32_t bx = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((max_nnz + 4095) / 4096, 4096));
  hipLaunchKernelGGL(k_bounds, dim3(bx, P), dim3(kThreads), 0, stream, idx, R);
  const dim3 segs((uint32_t)L.S);
  if (dense_first) {
    hipLaunchKernelGGL(k_write<kDenseFirst>, segs, dim3(kWriteThreads), 0, stream, idx, val, out_idx, out_val, R);
    hipLaunchKernelGGL(k_decide, dim3(1), dim3(1024), 0, stream, R);
    hipLaunchKernelGGL(k_write<kSparseOnly>, segs, dim3(kWriteThreads), 0, stream, idx, val, out_idx, out_val, R);
  } else {
    hipLaunchKernelGGL(k_count, segs, dim3(kThreads), 0, stream, idx, R);
    hipLaunchKernelGGL(k_decide, dim3(1), dim3(1024), 0, stream, R);
    hipLaunchKernelGGL(k_write<kDecided>, segs, dim3(kWriteThreads), 0, stream, idx, val, out_idx, out_val, R);
  }
  return hipGetLastError();
}

}  // namespace sparcml
