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
  size_t state, offs, qoffs, bounds, cnt, off, total;
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

// Node runs of segment s: pre[p] = exclusive prefix of their lengths,
// start[p] = absolute index of the first pair; returns the segment's pair
// count. pre[P + 1 .. 2P) are set to all ones (room for find_nodes' steps).
// Run ends are clamped to the node's own pairs, which keeps every later load
// inside them even for input whose order check failed. With at most 64 nodes
// one wave builds the table (no block scan).
template <int NT, int MAXP>
__device__ __forceinline__ uint32_t load_runs(const RDev& R, uint64_t s, uint32_t* pre, uint32_t* start,
                                              uint32_t* scr, QRuns<MAXP>* q) {
  const uint64_t rows = R.S + 1;  // entries per node in the run-start table
  auto run = [&](uint32_t p) -> uint32_t {
    const uint32_t* b = R.bounds + p * rows + s;
    const uint32_t lo = (uint32_t)R.offs[p], hi = (uint32_t)R.offs[p + 1];
    const uint32_t b0 = std::min<uint32_t>(std::max<uint32_t>(b[0], lo), hi);
    const uint32_t b1 = std::min<uint32_t>(std::max<uint32_t>(b[1], lo), hi);
    start[p] = b0;
    if (q != nullptr) {
      q->rel[p] = b0 - lo;
      q->cb[p] = (uint32_t)R.coffs[p];
      q->sb[p] = (uint32_t)R.soffs[p];
    }
    return b1 > b0 ? b1 - b0 : 0u;
  };
  for (uint32_t i = R.P + 1u + threadIdx.x; i < 2u * R.P; i += NT) pre[i] = ~0u;
  if (R.P <= (uint32_t)kWave) {
    if (threadIdx.x < kWave) {
      const uint32_t p = threadIdx.x;
      const uint32_t len = p < R.P ? run(p) : 0u;
      const uint32_t inc = wave_inclusive_scan(len);
      if (p < R.P) pre[p] = inc - len;
      if (p == R.P - 1) pre[R.P] = inc;
    }
    __syncthreads();
    return pre[R.P];
  }
  uint32_t carry = 0;
  for (uint32_t p0 = 0; p0 < R.P; p0 += NT) {
    const uint32_t p = p0 + threadIdx.x;
    const uint32_t len = p < R.P ? run(p) : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<NT>(len, scr, tot);
    if (p < R.P) pre[p] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) pre[R.P] = carry;
  __syncthreads();
  return carry;
}

// For every batch slot b with f = f0 + b * NT + threadIdx.x < total: node[b]
// = the largest p with pre[p] <= f (pre is nondecreasing, pre[0] = 0 and
// pre[P] = total > f). Binary lifting with one uniform step sequence for all
// slots and no branches, so the slots' LDS reads overlap instead of forming
// one dependent chain per slot. pre[] holds 2P words, those past P all ones:
// a step reads at most pre[2P - 1] and never moves past P for f < total.
template <int NT, int B>
__device__ __forceinline__ void find_nodes(const uint32_t* pre, uint32_t P, uint32_t f0, uint32_t (&node)[B]) {
#pragma unroll
  for (int b = 0; b < B; ++b) node[b] = 0u;
  const uint32_t top = P > 1u ? 1u << (31 - __clz(P - 1u)) : 0u;  // largest power of two <= P - 1
  for (uint32_t step = top; step != 0u; step >>= 1) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const uint32_t f = f0 + b * NT + threadIdx.x;
      const uint32_t c = node[b] + step;
      node[b] = pre[c] <= f ? c : node[b];
    }
  }
}

// One workgroup per segment: short, independent workgroups kept more
// segments in flight than long ones walking several segments (measured).
// Counting needs only the bitmap's 128 words, held by the first two waves;
// the others leave once the merge is done. The sparse compaction stages the
// segment's pairs in LDS so that its global stores are coalesced.
constexpr int kCountThreads = 128;
constexpr int kWriteThreads = 512;
constexpr int kWordWaves = kWords / kWave;  // 2
static_assert(kWords % kWave == 0 && kWords <= kCountThreads, "bitmap words cover whole waves");

template <int MAXP>
__global__ __launch_bounds__(kCountThreads) void k_count(const uint32_t* __restrict__ idx, RDev R) {
  constexpr int NT = kCountThreads;
  __shared__ uint32_t bits[kWords];
  __shared__ uint32_t pre[2 * MAXP];
  __shared__ uint32_t start[MAXP];
  __shared__ uint32_t scr[NT / kWave + 3];
  const uint64_t s = xcd_contiguous(blockIdx.x, gridDim.x);  // neighbours share run-edge lines
  const uint32_t seg_lo = (uint32_t)(s << kSegBits);
  const uint32_t seg_len = std::min<uint32_t>(kSeg, R.N - seg_lo);
  if (threadIdx.x < kWords) bits[threadIdx.x] = 0u;
  const uint32_t total = load_runs<NT, MAXP>(R, s, pre, start, scr, (QRuns<MAXP>*)nullptr);
  constexpr int kBatch = 12;
  for (uint32_t f0 = 0; f0 < total; f0 += NT * kBatch) {
    uint32_t ii[kBatch], pos[kBatch];
    find_nodes<NT>(pre, R.P, f0, pos);  // each slot's node, replaced below by its position
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {  // positions first, so the LDS reads are not behind branches
      const uint32_t p = std::min(pos[b], R.P - 1u);
      pos[b] = start[p] + (f0 + b * NT + threadIdx.x - pre[p]);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (f0 + b * NT + threadIdx.x < total) ii[b] = idx[pos[b]];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint32_t local = ii[b] - seg_lo;
      if (f0 + b * NT + threadIdx.x < total && local < seg_len) atomicOr(&bits[local >> 5], 1u << (local & 31));
    }
  }
  __syncthreads();
  const uint32_t wid = threadIdx.x / kWave;
  if (wid >= (uint32_t)kWordWaves) return;
  const uint32_t c = wave_sum((uint32_t)__popc(bits[threadIdx.x]));
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
                                                         RDev R) {
  constexpr int NT = kWriteThreads;
  __shared__ double acc[kSeg];
  __shared__ uint32_t bits[kWords];
  __shared__ uint32_t pre[2 * MAXP];
  __shared__ uint32_t start[MAXP];
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
  const uint32_t total = load_runs<NT, BITS ? MAXP : 1>(R, s, pre, start, scr, BITS ? &qruns : nullptr);
  if (!dense && seg_cnt == 0u) return;  // nothing of this segment in a sparse result

  constexpr int kBatch = 4;
  for (uint32_t f0 = 0; f0 < total; f0 += NT * kBatch) {
    uint32_t ii[kBatch], node[kBatch], js[kBatch];
    uint32_t qe[kBatch];              // quantized input: position in the node's code row
    uint32_t qc[kBatch], qs[kBatch];  // ... and the node's code-byte and scale offsets
    float vv[kBatch];
    find_nodes<NT>(pre, R.P, f0, node);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {  // positions first, so the LDS reads are not behind branches
      const uint32_t p = std::min(node[b], R.P - 1u);
      const uint32_t jr = f0 + b * NT + threadIdx.x - pre[p];  // position in the node's run
      js[b] = start[p] + jr;                                   // position in the pair arrays
      if constexpr (BITS != 0) {
        qe[b] = qruns.rel[p] + jr;
        qc[b] = qruns.cb[p];
        qs[b] = qruns.sb[p];
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint32_t f = f0 + b * NT + threadIdx.x;
      if (f < total) {
        const uint32_t j = js[b];
        ii[b] = idx[j];
        if constexpr (BITS == 0) {
          vv[b] = val[j];
        } else {  // dequantize on load: position e of the node's codes
          using F = Qsgd<BITS>;
          const uint32_t e = qe[b];
          const uint32_t bucket_no = R.bucket_recip ? (uint32_t)__umul64hi((uint64_t)e, R.bucket_recip) : e;
          const uint32_t code = F::code_at(R.codes + qc[b], e);
          vv[b] = F::value(code, F::step(R.scales[qs[b] + bucket_no]));
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const uint32_t local = ii[b] - seg_lo;
      if (f0 + b * NT + threadIdx.x < total && local < seg_len) {
        atomicAdd(&acc[local], (double)vv[b]);
        atomicOr(&bits[local >> 5], 1u << (local & 31));
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

}  // namespace

size_t reduce_workspace_bytes(uint32_t P, uint64_t N, uint64_t /*total_nnz*/) { return make_layout(P, N).total; }

namespace {

template <int MODE, int MAXP>
void launch_write(uint32_t bits, dim3 grid, hipStream_t stream, const uint32_t* idx, const float* val,
                  uint32_t* out_idx, float* out_val, const RDev& R) {
  const dim3 block(kWriteThreads);
  switch (bits) {
    case 0: hipLaunchKernelGGL((k_write<MODE, MAXP, 0>), grid, block, 0, stream, idx, val, out_idx, out_val, R); break;
    case 2: hipLaunchKernelGGL((k_write<MODE, MAXP, 2>), grid, block, 0, stream, idx, val, out_idx, out_val, R); break;
    case 4: hipLaunchKernelGGL((k_write<MODE, MAXP, 4>), grid, block, 0, stream, idx, val, out_idx, out_val, R); break;
    default: hipLaunchKernelGGL((k_write<MODE, MAXP, 8>), grid, block, 0, stream, idx, val, out_idx, out_val, R); break;
  }
}

template <int MODE>
void launch_write(bool small_p, uint32_t bits, dim3 grid, hipStream_t stream, const uint32_t* idx, const float* val,
                  uint32_t* out_idx, float* out_val, const RDev& R) {
  // run tables sized for up to 256 nodes keep the write workgroups small
  if (small_p) launch_write<MODE, 256>(bits, grid, stream, idx, val, out_idx, out_val, R);
  else launch_write<MODE, kMaxP>(bits, grid, stream, idx, val, out_idx, out_val, R);
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
  if (dense_first) {
    launch_write<kDenseFirst>(small_p, R.bits, segs, stream, idx, val, out_idx, out_val, R);
    hipLaunchKernelGGL(k_decide, dim3(1), dim3(1024), 0, stream, R);
    launch_write<kSparseOnly>(small_p, R.bits, segs, stream, idx, val, out_idx, out_val, R);
  } else {
    if (small_p) hipLaunchKernelGGL((k_count<256>), segs, dim3(kCountThreads), 0, stream, idx, R);
    else hipLaunchKernelGGL((k_count<kMaxP>), segs, dim3(kCountThreads), 0, stream, idx, R);
    hipLaunchKernelGGL(k_decide, dim3(1), dim3(1024), 0, stream, R);
    launch_write<kDecided>(small_p, R.bits, segs, stream, idx, val, out_idx, out_val, R);
  }
  return hipGetLastError();
}

}  // namespace sparcml
