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
// 4096 indices, the one-GPU analogue of the split phase's index-range owners;
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
//            sparse pairs (staged in LDS, stored coalesced) at the segment's
//            offset
// Dense-first (estimate >= T): write<dense> also counts; decide; a sparse
// rewrite runs only if the exact K turned out below T.
#include "device_common.hpp"
#include "kernels.hpp"
#include "qsgd_format.hpp"
#include "sparcml.h"

#include <algorithm>
#include <cmath>

namespace sparcml {
namespace {

constexpr int kSegBits = 12;
constexpr uint32_t kSeg = 1u << kSegBits;  // 4096 indices per segment
constexpr int kThreads = 256;              // bounds kernel
constexpr int kWords = kSeg / 32;          // bitmap words per segment
constexpr uint32_t kMaxP = 1024;
constexpr int kInlineOffsets = 256;

struct State {
  uint32_t flags;
  uint32_t is_dense;
  uint64_t K;
};

struct Layout {
  uint64_t S;  // segments
  size_t state, offs, qoffs, bounds, cnt, off, bitmaps, total;
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
  L.qoffs = take(16ull * (P + 1));  // code-byte and scale offsets per node (quantized input)
  L.bounds = take(4ull * P * (L.S + 1));
  L.cnt = take(4ull * L.S);
  L.off = take(4ull * L.S);
  L.bitmaps = take(4ull * kWords * L.S);  // union bitmap of every segment
  L.total = o;
  return L;
}

struct RDev {
  uint32_t P;
  uint32_t N;
  uint32_t total;  // pairs over all nodes
  uint32_t pad;
  uint64_t S;
  uint64_t T;
  uint64_t out_idx_cap;
  State* state;
  uint64_t* offs;
  uint32_t* bounds;
  uint32_t* cnt;
  uint32_t* off;
  uint32_t* bitmaps;  // [S][128]: bit i of segment s set iff s * 4096 + i is in the union
  ReduceResultDev* result;
  // quantized input only: node p's codes start at byte coffs[p], its
  // scales at soffs[p]
  uint32_t bits;
  uint32_t bucket;
  uint64_t bucket_recip;  // ceil(2^64 / bucket) for bucket >= 2, else 0: e / bucket = mulhi(e, bucket_recip)
  const uint8_t* codes;
  const float* scales;
  uint64_t* coffs;
  uint64_t* soffs;
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

// Quantized input: code-byte and scale offsets of every node, exclusive
// prefix sums of ceil(nnz_p * bits / 8) and ceil(nnz_p / bucket) over the
// nodes (one workgroup; P <= 1024).
__global__ __launch_bounds__(1024) void k_qoffsets(RDev R) {
  __shared__ uint64_t wc[1024 / kWave], wsc[1024 / kWave];
  const uint32_t p = threadIdx.x;
  uint64_t c = 0, q = 0;
  if (p < R.P) {
    const uint64_t nnz = R.offs[p + 1] - R.offs[p];
    c = (nnz * R.bits + 7) / 8;
    q = (nnz + R.bucket - 1) / R.bucket;
  }
  uint64_t ic = c, iq = q;  // inclusive scans within the wave
  for (int d = 1; d < kWave; d <<= 1) {
    const uint64_t xc = __shfl_up(ic, d), xq = __shfl_up(iq, d);
    if (lane_id() >= (uint32_t)d) {
      ic += xc;
      iq += xq;
    }
  }
  const uint32_t wid = threadIdx.x / kWave;
  if (lane_id() == kWave - 1) {
    wc[wid] = ic;
    wsc[wid] = iq;
  }
  __syncthreads();
  uint64_t bc = 0, bq = 0;
  for (uint32_t w = 0; w < wid; ++w) {
    bc += wc[w];
    bq += wsc[w];
  }
  if (p < R.P) {
    R.coffs[p] = bc + ic - c;
    R.soffs[p] = bq + iq - q;
  }
}

// Node-major pass: start[p][s] = absolute index of node p's first pair with
// index >= s*4096 (s = S stands for N), written by the pair where the run
// crosses into segment s. The table is node-major, so the entries one node
// writes are consecutive words (a segment's workgroup later gathers its P
// run starts, one word per node).
// Each lane loads four consecutive pairs as one 16-byte-aligned quad (quad q
// holds elements 4q - shift .. 4q - shift + 3, shift placing the quads on
// 16-byte boundaries of the index array); a quad's left neighbour comes from
// the lane below through a cross-lane shift, and only lane 0 loads its own.
__global__ __launch_bounds__(kThreads) void k_bounds(const uint32_t* __restrict__ idx, RDev R, uint32_t shift) {
  constexpr int kQuads = 4;  // quads per thread and pass
  const uint32_t p = blockIdx.y;
  // positions fit in 32 bits (total < 2^32) and so do segment numbers
  const uint32_t o0 = (uint32_t)R.offs[p], o1 = (uint32_t)R.offs[p + 1];
  const uint32_t S = (uint32_t)R.S, N = R.N;
  uint32_t* b = R.bounds + (uint64_t)p * (S + 1);
  uint32_t bad = 0u;
  if (o1 == o0) {  // an empty node starts every segment at its offset
    if (blockIdx.x == 0)
      for (uint32_t s = threadIdx.x; s <= S; s += kThreads) b[s] = o0;
    return;
  }
  const uint32_t q0 = (uint32_t)(((uint64_t)o0 + shift) >> 2);
  const uint32_t nq = (uint32_t)((((uint64_t)o1 + shift + 3) >> 2) - q0);  // quads meeting [o0, o1)
  const bool lane0 = lane_id() == 0;
  const uint32_t stride = gridDim.x * kThreads * kQuads;
  for (uint32_t j0 = blockIdx.x * kThreads * kQuads; j0 < nq; j0 += stride) {
    uint32_t v[kQuads][4], w[kQuads];
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const uint32_t jq = j0 + u * kThreads + threadIdx.x;
      // first element of the quad; below 0 (wrapped) only for the array's first quad
      const uint32_t e0 = 4u * (q0 + jq) - shift;
      const bool first_quad = q0 + jq == 0u && shift != 0u;
      w[u] = 0u;
      if (jq < nq) {
        if (!first_quad && (uint64_t)e0 + 4u <= R.total) {
          const uint4 x = *reinterpret_cast<const uint4*>(idx + e0);
          v[u][0] = x.x;
          v[u][1] = x.y;
          v[u][2] = x.z;
          v[u][3] = x.w;
        } else {  // a quad at either end of the array: elements inside it only
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t e = e0 + t;
            const bool in = (!first_quad || (uint32_t)t >= shift) && e < R.total;
            v[u][t] = in ? idx[e] : 0u;
          }
        }
        if (lane0 && !first_quad && e0 > o0) w[u] = idx[e0 - 1];
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[u][t] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const uint32_t up = __shfl_up(v[u][3], 1);
      const uint32_t jq = j0 + u * kThreads + threadIdx.x;
      if (jq >= nq) continue;
      const uint32_t e0 = 4u * (q0 + jq) - shift;
      const bool first_quad = q0 + jq == 0u && shift != 0u;
      uint32_t ip = lane0 ? w[u] : up;  // the element before the current one
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t e = e0 + t;
        const uint32_t i = v[u][t];
        const bool live = (!first_quad || (uint32_t)t >= shift) && e >= o0 && e < o1;
        if (live) {
          const uint32_t s_cur = i < N ? i >> kSegBits : S;
          uint32_t s_first = 0u;  // first segment whose run starts here
          if (e > o0) {
            if (ip >= i) bad |= SPARCML_FLAG_NOT_ASCENDING;
            s_first = (ip < N ? ip >> kSegBits : S) + 1u;
          }
          if (i >= N) bad |= SPARCML_FLAG_INDEX_RANGE;
          for (uint32_t sx = s_first; sx <= s_cur; ++sx) b[sx] = e;
          if (e + 1u == o1)
            for (uint32_t sx = s_cur + 1u; sx <= S; ++sx) b[sx] = o1;
        }
        ip = i;
      }
    }
  }
  if (bad) atomicOr(&R.state->flags, bad);
}

// Per-node tables of a quantized segment, in LDS: node-relative position of
// the run's first pair and the node's code-byte and scale offsets. Offsets
// fit in 32 bits (at most 2^32 - 16 pairs of at most 8-bit codes, and fewer
// scales than pairs plus nodes), which keeps the writer within four
// workgroups per compute unit.
template <int MAXP>
struct QRuns {
  uint32_t rel[MAXP];
  uint32_t cb[MAXP];
  uint32_t sb[MAXP];
};

// Run of node p in segment s: (absolute position of the node's first pair
// in the segment, number of its pairs there). Run ends are clamped to the
// node's own pairs, which keeps every later load inside them even for input
// whose order check failed.
__device__ __forceinline__ uint2 node_run(const RDev& R, uint64_t s, uint32_t p) {
  const uint32_t* b = R.bounds + p * (R.S + 1) + s;  // node-major run-start table
  const uint32_t lo = (uint32_t)R.offs[p], hi = (uint32_t)R.offs[p + 1];
  const uint32_t b0 = std::min<uint32_t>(std::max<uint32_t>(b[0], lo), hi);
  const uint32_t b1 = std::min<uint32_t>(std::max<uint32_t>(b[1], lo), hi);
  return make_uint2(b0, b1 > b0 ? b1 - b0 : 0u);
}

// The run table of segment s in LDS (node p's run at runs[p]), and for
// quantized input the node's code tables. All loads of a thread go out
// before it waits; the caller's barrier publishes the table.
template <int NT, int MAXP>
__device__ __forceinline__ void store_run_table(const RDev& R, uint64_t s, uint2* runs, QRuns<MAXP>* q) {
  for (uint32_t p = threadIdx.x; p < R.P; p += NT) {
    const uint2 rn = node_run(R, s, p);
    runs[p] = rn;
    if (q != nullptr) {
      q->rel[p] = rn.x - (uint32_t)R.offs[p];
      q->cb[p] = (uint32_t)R.coffs[p];
      q->sb[p] = (uint32_t)R.soffs[p];
    }
  }
}

// Slots of a pass: the threads are cut into groups of `lanes` consecutive
// lanes (lanes = 2^lane_bits); group g of NT / lanes takes nodes
// p0 + b * (NT / lanes) + g for b < B, lane l of the group the node's pair
// l. Each node's pairs are consecutive in memory, so a group's loads are
// contiguous and no thread searches for its node. Pairs past the first
// `lanes` of a run are taken by a later loop.
struct Slots {
  uint32_t lane;     // l
  uint32_t group;    // g
  uint32_t groups;   // NT / lanes: nodes per row of the pass
};

__device__ __forceinline__ Slots make_slots(uint32_t lane_bits, int NT) {
  Slots sl;
  sl.lane = threadIdx.x & ((1u << lane_bits) - 1u);
  sl.group = threadIdx.x >> lane_bits;
  sl.groups = (uint32_t)NT >> lane_bits;
  return sl;
}

constexpr int kCountThreads = 128;
constexpr int kWriteThreads = 512;
constexpr int kWordWaves = kWords / kWave;  // 2
static_assert(kWords % kWave == 0 && kWords <= kCountThreads, "bitmap words cover whole waves");

// One workgroup per segment: short, independent workgroups kept more
// segments in flight than long ones walking several segments (measured).
// Counting needs only the bitmap's 128 words, held by the first two waves;
// the others leave once the merge is done.
template <int MAXP>
__global__ __launch_bounds__(kCountThreads) void k_count(const uint32_t* __restrict__ idx, RDev R,
                                                         uint32_t lane_bits) {
  constexpr int NT = kCountThreads;
  constexpr int kB = 16;  // node rows per pass: 16 index loads in flight per thread
  __shared__ uint32_t bits[kWords];
  __shared__ uint2 runs[MAXP];
  __shared__ uint32_t scr[NT / kWave];
  const uint64_t s = xcd_contiguous(blockIdx.x, gridDim.x);  // neighbours share run-edge lines
  const uint32_t seg_lo = (uint32_t)(s << kSegBits);
  const uint32_t seg_len = std::min<uint32_t>(kSeg, R.N - seg_lo);
  if (threadIdx.x < kWords) bits[threadIdx.x] = 0u;
  const Slots sl = make_slots(lane_bits, NT);
  store_run_table<NT, MAXP>(R, s, runs, nullptr);
  __syncthreads();
  auto mark = [&](uint32_t i) {
    const uint32_t local = i - seg_lo;
    if (local < seg_len) atomicOr(&bits[local >> 5], 1u << (local & 31));
  };
  for (uint32_t p0 = 0; p0 < R.P; p0 += sl.groups * kB) {
    uint2 rn[kB];
    uint32_t ii[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const uint32_t p = p0 + b * sl.groups + sl.group;
      rn[b] = p < R.P ? runs[p] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (sl.lane < rn[b].y) ii[b] = idx[rn[b].x + sl.lane];
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (sl.lane < rn[b].y) mark(ii[b]);
    const uint32_t step = 1u << lane_bits;  // the rest of runs longer than the group
    for (int b = 0; b < kB; ++b)
      for (uint32_t j = sl.lane + step; j < rn[b].y; j += step) mark(idx[rn[b].x + j]);
  }
  __syncthreads();
  const uint32_t wid = threadIdx.x / kWave;
  if (wid >= (uint32_t)kWordWaves) return;
  const uint32_t word = bits[threadIdx.x];
  R.bitmaps[s * kWords + threadIdx.x] = word;  // the ranked writer places pairs by it
  const uint32_t c = wave_sum((uint32_t)__popc(word));
  if (lane_id() == 0) scr[wid] = c;
  __syncthreads();  // only the word waves are left
  if (threadIdx.x == 0) {
    uint32_t tot = 0;
    for (int w = 0; w < kWordWaves; ++w) tot += scr[w];
    R.cnt[s] = tot;
  }
}

// Exclusive scan of the segment counts by one workgroup: each thread loads
// 32 consecutive counts at once (one round trip per 32768 segments, 16-byte
// loads where the run is whole), scans them in registers, and the
// per-thread totals are scanned across the block.
__global__ __launch_bounds__(1024) void k_decide(RDev R) {
  constexpr int kPer = 32;
  __shared__ uint32_t scr[1024 / kWave + 3];
  uint64_t carry = 0;
  for (uint64_t s0 = 0; s0 < R.S; s0 += 1024 * kPer) {
    const uint64_t first = s0 + (uint64_t)threadIdx.x * kPer;
    const bool whole = first + kPer <= R.S;  // cnt and off are 256-byte aligned, first % 32 == 0
    uint32_t c[kPer];
    if (whole) {
      const uint4* src = reinterpret_cast<const uint4*>(R.cnt + first);
#pragma unroll
      for (int q = 0; q < kPer / 4; ++q) {
        const uint4 x = src[q];
        c[4 * q] = x.x;
        c[4 * q + 1] = x.y;
        c[4 * q + 2] = x.z;
        c[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kPer; ++u) c[u] = first + u < R.S ? R.cnt[first + u] : 0u;
    }
    uint32_t sum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) sum += c[u];
    uint32_t tot;
    uint32_t run = (uint32_t)carry + block_exclusive_scan<1024>(sum, scr, tot);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t x = c[u];
      c[u] = run;
      run += x;
    }
    if (whole) {
      uint4* dst = reinterpret_cast<uint4*>(R.off + first);
#pragma unroll
      for (int q = 0; q < kPer / 4; ++q) dst[q] = make_uint4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
    } else {
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (first + u < R.S) R.off[first + u] = c[u];
    }
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

// BITS = 0: fp32 values; 2, 4, 8: values decoded from b-bit codes on load
template <int MODE, int MAXP, int BITS>
__global__ __launch_bounds__(kWriteThreads) void k_write(const uint32_t* __restrict__ idx,
                                                         const float* __restrict__ val,
                                                         uint32_t* __restrict__ out_idx, float* __restrict__ out_val,
                                                         RDev R, uint32_t lane_bits) {
  constexpr int NT = kWriteThreads;
  constexpr int kB = 4;  // node rows per pass
  __shared__ double acc[kSeg];
  __shared__ uint32_t bits[kWords];
  __shared__ uint2 runs[MAXP];
  __shared__ uint32_t scr[NT / kWave + 3];
  __shared__ QRuns<BITS ? MAXP : 1> qruns;
  const uint64_t s = xcd_contiguous(blockIdx.x, gridDim.x);  // neighbours share run-edge lines
  // these loads and the run table's go out together: one round trip
  const bool dense = MODE == kDenseFirst ? true : R.state->is_dense != 0u;
  if (MODE == kSparseOnly && dense) return;  // the dense-first pass already wrote the result
  const uint32_t seg_cnt = MODE == kDenseFirst ? 1u : R.cnt[s];
  const uint32_t seg_off = MODE == kDenseFirst ? 0u : R.off[s];
  const uint32_t seg_lo = (uint32_t)(s << kSegBits);
  const uint32_t seg_len = std::min<uint32_t>(kSeg, R.N - seg_lo);
  for (uint32_t i = threadIdx.x; i < kSeg; i += NT) acc[i] = 0.0;
  if (threadIdx.x < kWords) bits[threadIdx.x] = 0u;
  const Slots sl = make_slots(lane_bits, NT);
  store_run_table<NT, BITS ? MAXP : 1>(R, s, runs, BITS ? &qruns : nullptr);
  __syncthreads();
  if (!dense && seg_cnt == 0u) return;  // nothing of this segment in a sparse result

  // value of node p's pair at absolute position j, run-relative position jr
  auto value_at = [&](uint32_t p, uint32_t j, uint32_t jr) -> float {
    if constexpr (BITS == 0) {
      return val[j];
    } else {  // dequantize on load: position e of the node's codes
      using F = Qsgd<BITS>;
      const uint32_t e = qruns.rel[p] + jr;
      const uint32_t bucket_no = R.bucket_recip ? (uint32_t)__umul64hi((uint64_t)e, R.bucket_recip) : e;
      const uint32_t code = F::code_at(R.codes + qruns.cb[p], e);
      return F::value(code, F::step(R.scales[qruns.sb[p] + bucket_no]));
    }
  };
  auto add = [&](uint32_t i, float v) {
    const uint32_t local = i - seg_lo;
    if (local < seg_len) {
      atomicAdd(&acc[local], (double)v);
      atomicOr(&bits[local >> 5], 1u << (local & 31));
    }
  };
  for (uint32_t p0 = 0; p0 < R.P; p0 += sl.groups * kB) {
    uint2 rn[kB];
    uint32_t ii[kB];
    float vv[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const uint32_t p = p0 + b * sl.groups + sl.group;
      rn[b] = p < R.P ? runs[p] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      if (sl.lane < rn[b].y) {
        const uint32_t j = rn[b].x + sl.lane;
        ii[b] = idx[j];
        vv[b] = value_at(p0 + b * sl.groups + sl.group, j, sl.lane);
      }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (sl.lane < rn[b].y) add(ii[b], vv[b]);
    const uint32_t step = 1u << lane_bits;  // the rest of runs longer than the group
    for (int b = 0; b < kB; ++b) {
      const uint32_t p = p0 + b * sl.groups + sl.group;
      for (uint32_t jr = sl.lane + step; jr < rn[b].y; jr += step) {
        const uint32_t j = rn[b].x + jr;
        add(idx[j], value_at(p, j, jr));
      }
    }
  }
  __syncthreads();

  if (dense) {
    float* out = out_val + seg_lo;
    if (seg_len == kSeg) {
      for (uint32_t q = threadIdx.x; q < kSeg / 4; q += NT) {
        const float4 o = make_float4((float)acc[4 * q], (float)acc[4 * q + 1], (float)acc[4 * q + 2],
                                     (float)acc[4 * q + 3]);
        reinterpret_cast<float4*>(out)[q] = o;
      }
    } else {
      for (uint32_t i = threadIdx.x; i < seg_len; i += NT) out[i] = (float)acc[i];
    }
    if (MODE != kDenseFirst) return;
  }
  if (MODE == kDenseFirst) {  // union size, in the word waves
    const uint32_t wid = threadIdx.x / kWave;
    if (wid >= (uint32_t)kWordWaves) return;
    const uint32_t c = wave_sum((uint32_t)__popc(bits[threadIdx.x]));
    if (lane_id() == 0) scr[wid] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kWordWaves; ++w) tot += scr[w];
      R.cnt[s] = tot;
    }
    return;
  }
  // ordered compaction: each thread owns 8 consecutive indices, stages its
  // selected pairs in LDS at their rank, then the block stores them coalesced
  constexpr int kPerT = kSeg / NT;
  static_assert(kPerT == 8, "one bitmap byte per thread");
  double v[kPerT];
#pragma unroll
  for (int r = 0; r < kPerT; ++r) v[r] = acc[kPerT * threadIdx.x + r];
  const uint32_t byte = (bits[threadIdx.x / 4] >> (8 * (threadIdx.x & 3))) & 0xFFu;
  uint32_t tot;
  uint32_t q = block_exclusive_scan<NT>((uint32_t)__popc(byte), scr, tot);
  float* sval = reinterpret_cast<float*>(acc);
  uint32_t* sidx = reinterpret_cast<uint32_t*>(acc) + kSeg;
#pragma unroll
  for (int r = 0; r < kPerT; ++r) {
    if ((byte >> r) & 1u) {
      sval[q] = (float)v[r];
      sidx[q] = seg_lo + kPerT * threadIdx.x + r;
      ++q;
    }
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < tot; i += NT) {
    const uint64_t pos = (uint64_t)seg_off + i;
    if (pos < R.out_idx_cap) {
      out_idx[pos] = sidx[i];
      out_val[pos] = sval[i];
    }
  }
}

// Writer placing pairs by their rank in the segment's union, for results
// expected sparse. The count pass left each segment's union bitmap; a word
// table (ranks before each 32-index word, and the word) gives every pair its
// rank r in the segment with one LDS read and a popcount, so the sums
// accumulate directly in output order and are stored as they stand: no
// clearing or compaction of a 4096-entry tile, and a quarter of its LDS,
// which lets more workgroups share a compute unit.
//
// The vector-memory address unit and the VALU bound this pass, so each
// memory instruction moves 16 bytes per lane where it can: pairs are loaded
// as aligned quads (QUAD: fp32 values, idx and val 16-byte aligned; else one
// pair per lane), and results are stored as aligned quads: rank r of a
// window whose output starts at position P0 sits in slot r + (P0 mod 4), so
// that slot quads are output quads. Ranks come in windows of kRankCap; a
// segment with more union entries takes one pass over its pairs per window.
// A dense result (the count crossed T) writes every index of the segment:
// the sum at its rank, or 0 outside the union. For valid input every pair's
// bit is set in the bitmap the count pass built from the same pairs; input
// that failed the checks gives unspecified sums, but every LDS slot touched
// stays inside the window.
constexpr int kRankThreads = 256;
constexpr uint32_t kRankCap = 1536;
constexpr uint32_t kRankSlots = kRankCap + 4;

template <int MAXP, int BITS, bool QUAD>
__global__ __launch_bounds__(kRankThreads) void k_write_ranked(const uint32_t* __restrict__ idx,
                                                               const float* __restrict__ val,
                                                               uint32_t* __restrict__ out_idx,
                                                               float* __restrict__ out_val, RDev R,
                                                               uint32_t lane_bits) {
  static_assert(!QUAD || BITS == 0, "quad loads take fp32 values");
  constexpr int NT = kRankThreads;
  constexpr int kB = QUAD ? 2 : 8;  // node rows per pass
  __shared__ __align__(16) double acc[kRankSlots];
  __shared__ __align__(16) uint16_t sloc[kRankSlots];  // index within the segment
  __shared__ uint2 words[kWords];  // (ranks before the word, the word)
  __shared__ uint2 runs[MAXP];
  __shared__ QRuns<BITS ? MAXP : 1> qruns;
  __shared__ uint32_t head[3];     // is_dense, the segment's union count, its output offset
  const uint64_t s = xcd_contiguous(blockIdx.x, gridDim.x);  // neighbours share run-edge lines
  const uint32_t seg_lo = (uint32_t)(s << kSegBits);
  const uint32_t seg_len = std::min<uint32_t>(kSeg, R.N - seg_lo);
  const Slots sl = make_slots(lane_bits, NT);
  // every load of the prologue goes out before any wait: the bitmap (wave 0),
  // the decision, count and offset, and the run table
  uint2 wpair = make_uint2(0u, 0u);
  if (threadIdx.x < kWords / 2) wpair = reinterpret_cast<const uint2*>(R.bitmaps + s * kWords)[threadIdx.x];
  uint32_t h0 = 0, h1 = 0, h2 = 0;
  if (threadIdx.x == NT - 1) {
    h0 = R.state->is_dense;
    h1 = R.cnt[s];
    h2 = R.off[s];
  }
  for (uint32_t r = threadIdx.x; r < kRankSlots; r += NT) acc[r] = 0.0;
  store_run_table<NT, BITS ? MAXP : 1>(R, s, runs, BITS ? &qruns : nullptr);
  if (threadIdx.x < kWave) {  // word table: wave 0, two words per lane
    const uint32_t c0 = (uint32_t)__popc(wpair.x), c1 = (uint32_t)__popc(wpair.y);
    const uint32_t inc = wave_inclusive_scan(c0 + c1);
    words[2 * threadIdx.x] = make_uint2(inc - c0 - c1, wpair.x);
    words[2 * threadIdx.x + 1] = make_uint2(inc - c1, wpair.y);
  }
  if (threadIdx.x == NT - 1) {
    head[0] = h0;
    head[1] = h1;
    head[2] = h2;
  }
  __syncthreads();
  const bool dense = head[0] != 0u;
  const uint32_t seg_cnt = head[1];
  const uint32_t seg_off = head[2];
  if (!dense && seg_cnt == 0u) return;  // nothing of this segment in a sparse result

  auto value_at = [&](uint32_t p, uint32_t j, uint32_t jr) -> float {
    if constexpr (BITS == 0) {
      return val[j];
    } else {  // dequantize on load: position e of the node's codes
      using F = Qsgd<BITS>;
      const uint32_t e = qruns.rel[p] + jr;
      const uint32_t bucket_no = R.bucket_recip ? (uint32_t)__umul64hi((uint64_t)e, R.bucket_recip) : e;
      const uint32_t code = F::code_at(R.codes + qruns.cb[p], e);
      return F::value(code, F::step(R.scales[qruns.sb[p] + bucket_no]));
    }
  };
  const uint32_t windows = std::max<uint32_t>(1u, (seg_cnt + kRankCap - 1) / kRankCap);
  for (uint32_t w0 = 0, win = 0; win < windows; ++win, w0 += kRankCap) {
    const uint32_t sh = (seg_off + w0) & 3u;  // slot of the window's first rank
    const uint32_t base = w0 - sh;             // rank r sits in slot r - base
    if (win > 0) {  // the previous window is stored: clear for this one
      __syncthreads();
      for (uint32_t r = threadIdx.x; r < kRankSlots; r += NT) acc[r] = 0.0;
      __syncthreads();
    }
    auto add = [&](uint32_t i, float v) {
      const uint32_t local = i & (kSeg - 1u);
      const uint2 wd = words[local >> 5];
      const uint32_t x = wd.x + (uint32_t)__popc(wd.y & ((1u << (local & 31)) - 1u)) - base;
      if (x - sh < kRankCap) {
        atomicAdd(&acc[x], (double)v);
        sloc[x] = (uint16_t)local;
      }
    };
    for (uint32_t p0 = 0; p0 < R.P; p0 += sl.groups * kB) {
      uint2 rn[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const uint32_t p = p0 + b * sl.groups + sl.group;
        rn[b] = p < R.P ? runs[p] : make_uint2(0u, 0u);
      }
      const uint32_t step = 1u << lane_bits;
      if constexpr (QUAD) {
        // node run [a, a + L) covers quads q0 .. q1 - 1; lane l takes quad q0 + l
        uint4 ii[kB];
        float4 vv[kB];
        uint32_t q0[kB], q1[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          q0[b] = rn[b].x >> 2;
          q1[b] = rn[b].y ? (rn[b].x + rn[b].y + 3u) >> 2 : q0[b];
          if (q0[b] + sl.lane < q1[b]) {
            ii[b] = reinterpret_cast<const uint4*>(idx)[q0[b] + sl.lane];
            vv[b] = reinterpret_cast<const float4*>(val)[q0[b] + sl.lane];
          }
        }
        auto add4 = [&](uint32_t q, const uint2& r, const uint4& i4, const float4& v4) {
          const uint32_t e = 4u * q - r.x;  // run position of the quad's first pair (may wrap)
          if (e < r.y) add(i4.x, v4.x);
          if (e + 1u < r.y) add(i4.y, v4.y);
          if (e + 2u < r.y) add(i4.z, v4.z);
          if (e + 3u < r.y) add(i4.w, v4.w);
        };
#pragma unroll
        for (int b = 0; b < kB; ++b)
          if (q0[b] + sl.lane < q1[b]) add4(q0[b] + sl.lane, rn[b], ii[b], vv[b]);
        for (int b = 0; b < kB; ++b) {  // the rest of runs longer than the group's quads
          if (__ballot(q1[b] - q0[b] > step) == 0ull) continue;
          for (uint32_t q = q0[b] + sl.lane + step; q < q1[b]; q += step)
            add4(q, rn[b], reinterpret_cast<const uint4*>(idx)[q], reinterpret_cast<const float4*>(val)[q]);
        }
      } else {
        uint32_t ii[kB];
        float vv[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          if (sl.lane < rn[b].y) {
            const uint32_t j = rn[b].x + sl.lane;
            ii[b] = idx[j];
            vv[b] = value_at(p0 + b * sl.groups + sl.group, j, sl.lane);
          }
        }
#pragma unroll
        for (int b = 0; b < kB; ++b)
          if (sl.lane < rn[b].y) add(ii[b], vv[b]);
        for (int b = 0; b < kB; ++b) {  // the rest of runs longer than the group
          if (__ballot(rn[b].y > step) == 0ull) continue;
          const uint32_t p = p0 + b * sl.groups + sl.group;
          for (uint32_t jr = sl.lane + step; jr < rn[b].y; jr += step) {
            const uint32_t j = rn[b].x + jr;
            add(idx[j], value_at(p, j, jr));
          }
        }
      }
    }
    __syncthreads();
    if (dense) {  // every index of the segment: its sum, or 0 outside the union
      float* out = out_val + seg_lo;
      const bool whole = windows == 1u && seg_len == kSeg;
      for (uint32_t q = threadIdx.x; q < (seg_len + 3) / 4; q += NT) {
        const uint2 wd = words[q >> 3];
        float o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t local = 4 * q + t;
          const uint32_t bit = 1u << (local & 31);
          const uint32_t x = wd.x + (uint32_t)__popc(wd.y & (bit - 1u)) - base;
          const bool in = (wd.y & bit) && x - sh < kRankCap;
          o[t] = in ? (float)acc[x] : 0.0f;
          if (!whole && local < seg_len && (in || (!(wd.y & bit) && win == 0u))) out[local] = o[t];
        }
        if (whole) reinterpret_cast<float4*>(out)[q] = make_float4(o[0], o[1], o[2], o[3]);
      }
    } else {
      // slots [sh, sh + n) hold ranks w0 .. w0 + n - 1, at output positions
      // pos0 + slot with pos0 = seg_off + w0 - sh a multiple of 4, so slot
      // quads are output quads
      const uint32_t n = std::min(seg_cnt - w0, kRankCap);
      const uint64_t pos0 = (uint64_t)seg_off + w0 - sh;  // a multiple of 4
      for (uint32_t k = threadIdx.x; 4 * k < sh + n; k += NT) {
        const double2 a01 = reinterpret_cast<const double2*>(acc)[2 * k];
        const double2 a23 = reinterpret_cast<const double2*>(acc)[2 * k + 1];
        const uint2 lp = reinterpret_cast<const uint2*>(sloc)[k];  // four 16-bit indices
        const uint4 oi = make_uint4(seg_lo + (lp.x & 0xFFFFu), seg_lo + (lp.x >> 16), seg_lo + (lp.y & 0xFFFFu),
                                    seg_lo + (lp.y >> 16));
        const float4 ov = make_float4((float)a01.x, (float)a01.y, (float)a23.x, (float)a23.y);
        const uint64_t pos = pos0 + 4ull * k;
        if (4 * k >= sh && 4 * k + 4 <= sh + n && pos + 4 <= R.out_idx_cap) {
          reinterpret_cast<uint4*>(out_idx)[pos >> 2] = oi;
          reinterpret_cast<float4*>(out_val)[pos >> 2] = ov;
        } else {  // a quad at either end of the window, shared with the neighbours' outputs
          const uint32_t oiv[4] = {oi.x, oi.y, oi.z, oi.w};
          const float ovv[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t x = 4 * k + t;
            if (x >= sh && x < sh + n && pos + t < R.out_idx_cap) {
              out_idx[pos + t] = oiv[t];
              out_val[pos + t] = ovv[t];
            }
          }
        }
      }
    }
  }
}

}  // namespace

size_t reduce_workspace_bytes(uint32_t P, uint64_t N, uint64_t /*total_nnz*/) { return make_layout(P, N).total; }

namespace {

template <int MODE, int MAXP>
void launch_write(uint32_t bits, dim3 grid, hipStream_t stream, const uint32_t* idx, const float* val,
                  uint32_t* out_idx, float* out_val, const RDev& R, uint32_t lb) {
  const dim3 block(kWriteThreads);
  switch (bits) {
    case 0: hipLaunchKernelGGL((k_write<MODE, MAXP, 0>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lb); break;
    case 2: hipLaunchKernelGGL((k_write<MODE, MAXP, 2>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lb); break;
    case 4: hipLaunchKernelGGL((k_write<MODE, MAXP, 4>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lb); break;
    default: hipLaunchKernelGGL((k_write<MODE, MAXP, 8>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lb); break;
  }
}

template <int MODE>
void launch_write(bool small_p, uint32_t bits, dim3 grid, hipStream_t stream, const uint32_t* idx, const float* val,
                  uint32_t* out_idx, float* out_val, const RDev& R, uint32_t lb) {
  // run tables sized for up to 256 nodes keep the write workgroups small
  if (small_p) launch_write<MODE, 256>(bits, grid, stream, idx, val, out_idx, out_val, R, lb);
  else launch_write<MODE, kMaxP>(bits, grid, stream, idx, val, out_idx, out_val, R, lb);
}

template <int MAXP>
void launch_write_ranked(uint32_t bits, bool quad, dim3 grid, hipStream_t stream, const uint32_t* idx,
                         const float* val, uint32_t* out_idx, float* out_val, const RDev& R, uint32_t lb,
                         uint32_t lbq) {
  const dim3 block(kRankThreads);
  switch (bits) {
    case 0:
      if (quad) hipLaunchKernelGGL((k_write_ranked<MAXP, 0, true>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lbq);
      else hipLaunchKernelGGL((k_write_ranked<MAXP, 0, false>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lb);
      break;
    case 2: hipLaunchKernelGGL((k_write_ranked<MAXP, 2, false>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lb); break;
    case 4: hipLaunchKernelGGL((k_write_ranked<MAXP, 4, false>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lb); break;
    default: hipLaunchKernelGGL((k_write_ranked<MAXP, 8, false>), grid, block, 0, stream, idx, val, out_idx, out_val, R, lb); break;
  }
}

// Lanes per node in the count and write passes (as a power of two): about
// 1.5 times the mean run length of a node in a segment, so that few runs
// spill past their lanes while lanes stay mostly busy; 16 to 128.
uint32_t lanes_log2(uint32_t P, uint64_t S, uint64_t total) {
  const double mean = (double)total / ((double)P * (double)S);
  uint32_t lb = 4;
  while (lb < 7 && (double)(1u << lb) < 1.5 * mean) ++lb;
  return lb;
}

// Lanes per node when each lane takes an aligned quad of pairs: the mean
// number of quads a run meets (its length / 4, plus 3/4 for the unaligned
// ends) with room for one standard deviation and more; 2 to 64.
uint32_t quad_lanes_log2(uint32_t P, uint64_t S, uint64_t total) {
  const double mean = (double)total / ((double)P * (double)S);
  const double quads = mean / 4.0 + 0.75 + std::sqrt(mean) / 4.0 + 1.0;
  uint32_t lb = 1;
  while (lb < 6 && (double)(1u << lb) < quads) ++lb;
  return lb;
}

}  // namespace

hipError_t sparse_reduce_launch(uint32_t P, uint64_t N, uint64_t T, const uint64_t* h_offsets,
                                const uint32_t* idx, const float* val, const ReduceQuantized* quant,
                                bool dense_first, uint32_t* out_idx, uint64_t out_idx_cap, float* out_val,
                                ReduceResultDev* d_result, void* ws, hipStream_t stream) {
  const Layout L = make_layout(P, N);
  char* w = static_cast<char*>(ws);
  RDev R;
  R.P = P;
  R.N = (uint32_t)N;
  R.total = (uint32_t)h_offsets[P];
  R.pad = 0;
  R.S = L.S;
  R.T = T;
  R.out_idx_cap = out_idx_cap;
  R.state = reinterpret_cast<State*>(w + L.state);
  R.offs = reinterpret_cast<uint64_t*>(w + L.offs);
  R.bounds = reinterpret_cast<uint32_t*>(w + L.bounds);
  R.cnt = reinterpret_cast<uint32_t*>(w + L.cnt);
  R.off = reinterpret_cast<uint32_t*>(w + L.off);
  R.bitmaps = reinterpret_cast<uint32_t*>(w + L.bitmaps);
  R.result = d_result;
  R.bits = quant ? quant->bits : 0u;
  R.bucket = quant ? quant->bucket : 1u;
  R.bucket_recip = R.bucket >= 2u ? UINT64_MAX / R.bucket + 1u : 0u;
  R.codes = quant ? quant->codes : nullptr;
  R.scales = quant ? quant->scales : nullptr;
  R.coffs = reinterpret_cast<uint64_t*>(w + L.qoffs);
  R.soffs = R.coffs + (P + 1);

  uint64_t max_nnz = 0;
  for (uint32_t p = 0; p < P; ++p) max_nnz = std::max<uint64_t>(max_nnz, h_offsets[p + 1] - h_offsets[p]);

  for (uint32_t first = 0; first < P + 1; first += kInlineOffsets) {
    InlineOffsets in;
    const uint32_t count = std::min<uint32_t>(kInlineOffsets, P + 1 - first);
    for (uint32_t i = 0; i < count; ++i) in.v[i] = h_offsets[first + i];
    hipLaunchKernelGGL(k_setup, dim3(1), dim3(256), 0, stream, R, first, count, in, first == 0 ? 1 : 0);
  }
  if (R.bits) hipLaunchKernelGGL(k_qoffsets, dim3(1), dim3(1024), 0, stream, R);
  const uint32_t bx = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((max_nnz + 4095) / 4096, 4096));
  const uint32_t shift = (uint32_t)((reinterpret_cast<uintptr_t>(idx) >> 2) & 3u);
  hipLaunchKernelGGL(k_bounds, dim3(bx, P), dim3(kThreads), 0, stream, idx, R, shift);
  const dim3 segs((uint32_t)L.S);
  const bool small_p = P <= 256;
  const uint32_t lb = lanes_log2(P, L.S, R.total);
  if (dense_first) {
    launch_write<kDenseFirst>(small_p, R.bits, segs, stream, idx, val, out_idx, out_val, R, lb);
    hipLaunchKernelGGL(k_decide, dim3(1), dim3(1024), 0, stream, R);
    launch_write<kSparseOnly>(small_p, R.bits, segs, stream, idx, val, out_idx, out_val, R, lb);
  } else {
    if (small_p) hipLaunchKernelGGL((k_count<256>), segs, dim3(kCountThreads), 0, stream, idx, R, lb);
    else hipLaunchKernelGGL((k_count<kMaxP>), segs, dim3(kCountThreads), 0, stream, idx, R, lb);
    hipLaunchKernelGGL(k_decide, dim3(1), dim3(1024), 0, stream, R);
    // 16-byte quads of pairs where both arrays allow them
    const bool quad = R.bits == 0 && ((reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(val)) & 15u) == 0;
    const uint32_t lbq = quad_lanes_log2(P, L.S, R.total);
    if (small_p) launch_write_ranked<256>(R.bits, quad, segs, stream, idx, val, out_idx, out_val, R, lb, lbq);
    else launch_write_ranked<kMaxP>(R.bits, quad, segs, stream, idx, val, out_idx, out_val, R, lb, lbq);
  }
  return hipGetLastError();
}

}  // namespace sparcml
