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
// a workgroup owns a group of consecutive segments and takes each node's run
// of pairs falling in it. Sums accumulate in fp64 in LDS (ds_add_f64:
// independent of arrival order up to fp64 rounding) and are rounded to fp32
// once.
//
//   bounds   node-major streaming pass over the indices: where each node's
//            run crosses a segment boundary; checks range and order. Its
//            first workgroup also stores the node offsets (passed inline).
//            Not launched when the caller gives that run table (the
//            whole-vector Top-k writes it for its own output as it emits).
//   count    per count group of 2^glog segments: union bitmap in LDS, stored
//            for the writer, and the union count of every writer group in it
//            with the group's input-check bits in the word's top bits
//   decide   exclusive scan of the writer-group counts, K, dense iff K >= T,
//            the check bits of all groups (not launched for at most 4096
//            writer groups: every writer adds up the counts itself)
//   write    per writer group of 2^mlog segments: the sums, stored densely or
//            as the group's sorted part of the sparse result at its offset
// Groups of several segments serve inputs with few pairs per segment, where
// one segment per workgroup leaves each workgroup too little to load. The
// estimate of K picks the writer: a full 4096-entry tile per segment when the
// result is expected dense, slots in union-rank order otherwise; both write
// either result. More than 255 nodes take setup launches for the offsets
// first. (Per-group totals added up by atomics in the count pass, to let
// every writer find its own offset without the scan, made the count pass more
// than twice as slow: hundreds of workgroups adding to one word. Finding each
// node's run ends by searching its indices in the count pass, instead of the
// bounds pass, cost more than the pass it saved: every probe is a cache line.)
#include "device_common.hpp"
#include "kernels.hpp"
#include "qsgd_format.hpp"
#include "sparcml.h"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace sparcml {
namespace {

// An aligned quad of indices, plain or non-temporal. The writer, the last
// pass over the indices, loads them non-temporal: streaming them through
// the memory-side cache would evict the values, which the op before the
// reduce (the dequantizer, in a training step) has just written there. The
// bounds and count passes load them plain: the count pass finds in that
// cache what the bounds pass brought in (measured: non-temporal there made
// the count pass 35% slower).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_idx4(const uint32_t* p) {
  const u32x4v v = *reinterpret_cast<const u32x4v*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_idx4_nt(const uint32_t* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kSegBits = 12;
constexpr uint32_t kSeg = 1u << kSegBits;  // 4096 indices per segment
constexpr int kThreads = 256;              // bounds kernel
constexpr int kWordBits = 7;
constexpr int kWords = kSeg / 32;          // bitmap words per segment
static_assert(kWords == 1 << kWordBits, "segment words");
static_assert(kSeg == SPARCML_SEGMENT, "run tables of the C ABI use this segment");
constexpr uint32_t kMaxP = 1024;
// A writer group's count word: the union count (at most 4 segments of 4096)
// below bit kCountBits, the input-check bits of its count group above.
constexpr int kCountBits = 24;
constexpr uint32_t kCountMask = (1u << kCountBits) - 1u;
constexpr int kInlineOffsets = 256;
// Group sizes, measured on MI355X: count workgroups of up to 2048 pairs
// whose node runs stay within about 200 pairs (its lanes take one pair, or
// one quad, of a run each), and rank-order writers of up to 4 segments whose
// expected union fits the rank slots. Both keep at least 512 workgroups. The
// writer is bound by the bytes its workgroups have in flight: five
// workgroups of two 4096-index segments each (2560 rank slots) kept more in
// flight than eight of one, and more than four of two with 3072 slots or
// three of four with 5120.
constexpr uint32_t kMaxCountLog2 = 4;   // at most 16 segments per count workgroup
constexpr uint32_t kMaxWriterLog2 = 2;  // at most 4 segments per rank-order writer
constexpr double kCountPairs = 2048.0;
// With the caller's run table no bounds pass has just read the indices into
// the memory-side cache, and the count pass reads them from HBM: groups of
// up to 6000 pairs (four segments at the wide-ResNet size) then keep more
// bytes in flight (measured: 194 us for the reduce with one segment per
// group, 189 with two, 185 with four, 198-201 with eight).
constexpr double kCountPairsRuns = 6000.0;
constexpr double kCountRun = 200.0;
constexpr uint64_t kCountGroupsWanted = 512;
constexpr uint64_t kWriterGroupsWanted = 512;

// Written by the decide pass for the writers; nothing accumulates into it,
// so it needs no clearing.
struct State {
  uint32_t is_dense;
  uint32_t pad;
  uint64_t K;
};

struct Layout {
  uint64_t S;  // segments
  size_t state, offs, qoffs, flagw, bounds, cnt, off, bitmaps, total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workgroups per node in the bounds pass: one per 4096 pairs of the longest
// node, at most 4096.
uint32_t bounds_blocks(uint64_t max_nnz) {
  return (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((max_nnz + 4095) / 4096, 4096));
}

Layout make_layout(uint32_t P, uint64_t N, uint64_t total_nnz) {
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
  L.flagw = take(4ull * P * bounds_blocks(total_nnz));  // input-check bits of every bounds workgroup
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
  uint32_t glog;   // segments per count group: 2^glog
  uint32_t mlog;   // segments per writer group: 2^mlog (mlog <= glog)
  uint32_t pad;
  uint64_t S;      // segments
  uint64_t W;      // writer groups
  uint64_t T;
  uint64_t out_idx_cap;
  State* state;
  uint64_t* offs;
  uint32_t* flagw;  // [P * bx]: input-check bits found by each bounds workgroup
  uint64_t nflagw;
  uint32_t* bounds;   // [P][S+1] run starts: the bounds pass's, or the caller's table
  uint32_t* cnt;      // [W] union count per writer group, with its count group's check bits above kCountBits
  uint32_t* off;      // [W] its offset in the sparse result
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

// More than 255 nodes: offsets stored by launches of 256.
__global__ void k_setup(RDev R, uint32_t first, uint32_t count, InlineOffsets in) {
  for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) R.offs[first + i] = in.v[i];
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
// writes are consecutive words (a group's workgroup later gathers two words
// per node, at the group's first segment and the next group's). Checks range
// and order: each workgroup
// stores the bits it found in its own word, which the count pass folds into
// its groups' check words.
// Each lane loads four consecutive pairs as one 16-byte-aligned quad (quad q
// holds elements 4q - shift .. 4q - shift + 3, shift placing the quads on
// 16-byte boundaries of the index array); a quad's left neighbour comes from
// the lane below through a cross-lane shift, and only lane 0 loads its own.
// With up to 255 nodes the offsets come inline (`in`), and workgroup (0, 0)
// stores them for the later passes and, for quantized input, lays out the
// code and scale offsets.
__global__ __launch_bounds__(kThreads) void k_bounds(const uint32_t* __restrict__ idx, RDev R, uint32_t shift,
                                                     InlineOffsets in, int inline_offs) {
  constexpr int kQuads = 4;  // quads per thread and pass
  const uint32_t p = blockIdx.y;
  if (inline_offs && blockIdx.x == 0 && blockIdx.y == 0) {
    __shared__ uint64_t scr[kThreads / kWave + 1];
    for (uint32_t i = threadIdx.x; i <= R.P; i += kThreads) R.offs[i] = in.v[i];
    if (R.bits) {  // code-byte and scale offsets: exclusive prefix sums over the nodes (P <= 256)
      const uint32_t q = threadIdx.x;
      const uint64_t nnz = q < R.P ? in.v[q + 1] - in.v[q] : 0ull;
      uint64_t tc, ts;
      const uint64_t c = block_exclusive_scan_u64<kThreads>((nnz * R.bits + 7) / 8, scr, tc);
      const uint64_t sc = block_exclusive_scan_u64<kThreads>((nnz + R.bucket - 1) / R.bucket, scr, ts);
      if (q < R.P) {
        R.coffs[q] = c;
        R.soffs[q] = sc;
      }
    }
  }
  // positions fit in 32 bits (total < 2^32) and so do segment numbers
  const uint32_t o0 = (uint32_t)(inline_offs ? in.v[p] : R.offs[p]);
  const uint32_t o1 = (uint32_t)(inline_offs ? in.v[p + 1] : R.offs[p + 1]);
  const uint32_t S = (uint32_t)R.S, N = R.N;
  uint32_t* b = R.bounds + (uint64_t)p * (S + 1);
  uint32_t* flag = R.flagw + (uint64_t)p * gridDim.x + blockIdx.x;
  uint32_t bad = 0u;
  if (o1 == o0) {  // an empty node starts every segment at its offset
    if (blockIdx.x == 0)
      for (uint32_t s = threadIdx.x; s <= S; s += kThreads) b[s] = o0;
    if (threadIdx.x == 0) *flag = 0u;
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
          const uint4 x = ld_idx4(idx + e0);
          v[u][0] = x.x;
          v[u][1] = x.y;
          v[u][2] = x.z;
          v[u][3] = x.w;
        } else {  // a quad at either end of the array: elements inside it only
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t e = e0 + t;
            const bool inside = (!first_quad || (uint32_t)t >= shift) && e < R.total;
            v[u][t] = inside ? idx[e] : 0u;
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
      if (!first_quad && e0 >= o0 && e0 + 4u <= o1) {
        // a quad inside the node's pairs (all but its two ends): segments
        // (s_{t-1}, s_t] start at element t, s_{-1} the predecessor's segment
        // (or below 0 for the node's first element); the node's last element
        // also starts every later segment (at o1)
        const uint32_t i0 = v[u][0], i1 = v[u][1], i2 = v[u][2], i3 = v[u][3];
        const bool has_prev = e0 > o0;
        if ((has_prev && ip >= i0) || i0 >= i1 || i1 >= i2 || i2 >= i3) bad |= SPARCML_FLAG_NOT_ASCENDING;
        if (std::max(std::max(i0, i1), std::max(i2, i3)) >= N) bad |= SPARCML_FLAG_INDEX_RANGE;
        auto seg = [&](uint32_t i) { return i < N ? i >> kSegBits : S; };
        const uint32_t s0 = seg(i0), s1 = seg(i1), s2 = seg(i2), s3 = seg(i3);
        const uint32_t from = has_prev ? seg(ip) + 1u : 0u;
        if (from <= s3 || from <= s0) {
          for (uint32_t sx = from; sx <= s0; ++sx) b[sx] = e0;
          for (uint32_t sx = std::max(s0 + 1u, from); sx <= s1; ++sx) b[sx] = e0 + 1u;
          for (uint32_t sx = std::max(s1 + 1u, from); sx <= s2; ++sx) b[sx] = e0 + 2u;
          for (uint32_t sx = std::max(s2 + 1u, from); sx <= s3; ++sx) b[sx] = e0 + 3u;
        }
        if (e0 + 4u == o1)
          for (uint32_t sx = s3 + 1u; sx <= S; ++sx) b[sx] = o1;
        continue;
      }
      // segments whose run starts in this quad: [lo, hi], each at the quad's
      // first pair whose segment reaches it; the node's last pair also
      // starts every later segment (at o1)
      uint32_t sc[4];
      bool lv[4];
      uint32_t lo = 1u, hi = 0u, last_e = 0u, last_s = 0u;
      bool any = false, ends = false;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t e = e0 + t;
        const uint32_t i = v[u][t];
        lv[t] = (!first_quad || (uint32_t)t >= shift) && e >= o0 && e < o1;
        sc[t] = i < N ? i >> kSegBits : S;
        if (lv[t]) {
          // first segment whose run starts here (none if this pair is below its predecessor)
          const uint32_t s_first = e > o0 ? (ip < N ? ip >> kSegBits : S) + 1u : 0u;
          if (e > o0 && ip >= i) bad |= SPARCML_FLAG_NOT_ASCENDING;
          if (i >= N) bad |= SPARCML_FLAG_INDEX_RANGE;
          if (!any) lo = s_first;
          any = true;
          hi = sc[t];
          last_e = e;
          last_s = sc[t];
          ends |= e + 1u == o1;
        }
        ip = i;
      }
      for (uint32_t sx = lo; sx <= hi; ++sx) {
        uint32_t at = last_e;
#pragma unroll
        for (int t = 3; t >= 0; --t)
          if (lv[t] && sc[t] >= sx) at = e0 + t;
        b[sx] = at;
      }
      if (ends)
        for (uint32_t sx = last_s + 1u; sx <= S; ++sx) b[sx] = o1;
    }
  }
  // every workgroup stores its bits, so no word needs clearing first
  __shared__ uint32_t block_bad;
  if (threadIdx.x == 0) block_bad = 0u;
  __syncthreads();
  if (bad) atomicOr(&block_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) *flag = block_bad;
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

// Values of one aligned quad of pairs decoded from b-bit codes, for the rank
// writer's quad loads of quantized input (codes 4-byte aligned). The quad's
// elements inside its node's run, t0 .. t0 + nv - 1, have consecutive
// node-relative positions rel .. rel + nv - 1, so their codes are one span of
// at most 32 bits: two aligned words hold it (the same word when it fits in
// one; each holds a code of the node, so neither lies past the array's last
// word). Their buckets are at most two, each with its scale. A quad with no
// element in the run loads the arrays' first word and scale. The decode is
// the op sequence of the pair-by-pair loader, so the sums are the same.
template <int BITS>
struct QuadCodes {
  uint32_t lo, hi, bit, t0, split;  // split: the first t of the second bucket (4: one bucket)
  float s_lo, s_hi;

  // quad q of node p's run r (absolute start, length), whose first pair is
  // at node-relative position rel_run; cb, sb: the node's code byte and
  // scale offsets
  __device__ __forceinline__ void load(const RDev& R, uint32_t q, uint2 r, uint32_t rel_run, uint32_t cb,
                                       uint32_t sb) {
    const uint32_t e = 4u * q - r.x;                 // run position of the quad's first pair (may wrap)
    const uint32_t lead = e > 0xFFFFFFFCu ? 0u - e : 0u;  // pairs before the run's start
    const bool any = lead < 4u && e + lead < r.y;
    const uint32_t nv = any ? std::min(4u - lead, r.y - (e + lead)) : 1u;
    const uint32_t rel = any ? rel_run + e + lead : 0u;
    const uint64_t b0 = any ? (uint64_t)cb * 8u + (uint64_t)rel * BITS : 0u;
    const uint64_t b1 = b0 + nv * BITS - 1u;
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(R.codes);
    lo = cw[b0 >> 5];
    hi = cw[b1 >> 5];
    bit = (uint32_t)(b0 & 31u);
    t0 = lead;
    auto bucket = [&](uint32_t x) { return R.bucket_recip ? (uint32_t)__umul64hi((uint64_t)x, R.bucket_recip) : x; };
    const uint32_t k0 = bucket(rel), k1 = bucket(rel + nv - 1u);
    s_lo = R.scales[any ? sb + k0 : 0u];
    s_hi = R.scales[any ? sb + k1 : 0u];
    split = k1 != k0 ? lead + (k1 * R.bucket - rel) : 4u;
  }

  __device__ __forceinline__ float4 values() const {
    using F = Qsgd<BITS>;
    const uint64_t win = ((((uint64_t)hi) << 32) | lo) >> bit;
    const float st_lo = F::step(s_lo), st_hi = F::step(s_hi);
    float v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t code = t >= (int)t0 ? (uint32_t)(win >> ((t - t0) * BITS)) & F::kMask : 0u;
      v[t] = F::value(code, (uint32_t)t < split ? st_lo : st_hi);
    }
    return make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Run of node p in segments [s0, s1): (absolute position of the node's
// first pair there, number of its pairs there). Run ends are clamped to the
// node's own pairs, which keeps every later load inside them even for input
// whose order check failed.
__device__ __forceinline__ uint2 node_run(const RDev& R, uint64_t s0, uint64_t s1, uint32_t p) {
  const uint32_t* b = R.bounds + p * (R.S + 1);  // node-major run-start table
  const uint32_t lo = (uint32_t)R.offs[p], hi = (uint32_t)R.offs[p + 1];
  const uint32_t b0 = std::min<uint32_t>(std::max<uint32_t>(b[s0], lo), hi);
  const uint32_t b1 = std::min<uint32_t>(std::max<uint32_t>(b[s1], lo), hi);
  return make_uint2(b0, b1 > b0 ? b1 - b0 : 0u);
}

// The run table of segments [s0, s1) in LDS (node p's run at runs[p]), and
// for quantized input the node's code tables. All loads of a thread go out
// before it waits; the caller's barrier publishes the table.
template <int NT, int MAXP>
__device__ __forceinline__ void store_run_table(const RDev& R, uint64_t s0, uint64_t s1, uint2* runs,
                                                QRuns<MAXP>* q) {
  for (uint32_t p = threadIdx.x; p < R.P; p += NT) {
    const uint2 rn = node_run(R, s0, s1, p);
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
static_assert(2 * kCountThreads >= kInlineOffsets, "two nodes' code offsets per count thread");
constexpr uint32_t kMaxWritersPerCount = 1u << kMaxCountLog2;

// One workgroup per count group g, segments [s0, s1) = [g 2^glog, ...):
// short, independent workgroups kept more segments in flight than long ones
// walking several groups (measured), and a group of several segments gives
// each workgroup enough pairs where a segment holds few. Builds the group's
// union bitmap in LDS, stores it with the union count of each writer group
// in the group, and folds a share of the bounds pass's check words into the
// state. (The checks themselves cost the count pass 14 us at 64 x 671088
// pairs, the bounds pass, which compares every pair with its predecessor
// anyway, about 4 us.) The pass is bound by its VALU work per index, so
// where the index array is 16-byte aligned (QUAD) each lane loads an
// aligned quad of indices: node run [a, a + L) meets quads a / 4 ..
// (a + L + 3) / 4 - 1, lane l of the node's group takes quad a / 4 + l.
//
// RUNS: the run table is the caller's (no bounds pass ran). The offsets then
// come inline (`in`, up to 255 nodes; workgroup 0 stores them for the
// writer) or from the setup launches, and the pass checks the table as it
// reads it: each node's entries at the group's two edges lie within the
// node's pairs and in order, the first segment's entry is the node's first
// pair and the last segment's the node's end, and every pair of a run lies
// in the run's segments. A table that passes these checks covers every pair
// exactly once, in its own segment.
struct NoOffsets {};

template <int MAXP, bool QUAD, bool RUNS>
__global__ __launch_bounds__(kCountThreads) void k_count(const uint32_t* __restrict__ idx, RDev R,
                                                         uint32_t lane_bits,
                                                         std::conditional_t<RUNS, InlineOffsets, NoOffsets> in,
                                                         int inline_offs) {
  constexpr int NT = kCountThreads;
  constexpr int kB = QUAD ? 4 : 16;  // node rows per pass: 64 bytes of index loads in flight per thread
  static_assert(kWords % NT == 0 || NT % kWords == 0, "bitmap words cover whole waves");
  __shared__ uint2 runs[MAXP];
  __shared__ uint32_t wc[kMaxWritersPerCount];
  __shared__ uint32_t s_bad;
  extern __shared__ uint32_t bits[];  // [128 << glog]: the group's bitmap
  const uint64_t g = xcd_contiguous(blockIdx.x, gridDim.x);  // neighbours share run-edge lines
  const uint64_t s0 = g << R.glog;
  const uint64_t s1 = std::min<uint64_t>(s0 + (1u << R.glog), R.S);
  const uint32_t segs = (uint32_t)(s1 - s0);
  const uint32_t glo = (uint32_t)(s0 << kSegBits);
  const uint32_t glen = std::min<uint32_t>(segs << kSegBits, R.N - glo);
  for (uint32_t i = threadIdx.x; i < segs * kWords; i += NT) bits[i] = 0u;
  if (threadIdx.x < kMaxWritersPerCount) wc[threadIdx.x] = 0u;
  if (threadIdx.x == 0) s_bad = 0u;
  const Slots sl = make_slots(lane_bits, NT);
  uint32_t bad = 0u;
  if constexpr (RUNS) {
    auto off_at = [&](uint32_t p) -> uint32_t { return (uint32_t)(inline_offs ? in.v[p] : R.offs[p]); };
    if (inline_offs && blockIdx.x == 0) {
      for (uint32_t i = threadIdx.x; i <= R.P; i += NT) R.offs[i] = in.v[i];
      if (R.bits) {  // quantized input: the code-byte and scale offsets, two nodes per thread (P <= 255)
        __shared__ uint64_t qscr[NT / kWave + 1];
        const uint32_t pa = 2u * threadIdx.x, pb = pa + 1u;
        auto nnz = [&](uint32_t q) -> uint64_t { return q < R.P ? in.v[q + 1] - in.v[q] : 0ull; };
        const uint64_t ca = (nnz(pa) * R.bits + 7) / 8, cb = (nnz(pb) * R.bits + 7) / 8;
        const uint64_t sa = (nnz(pa) + R.bucket - 1) / R.bucket, sb = (nnz(pb) + R.bucket - 1) / R.bucket;
        uint64_t tc, ts;
        const uint64_t xc = block_exclusive_scan_u64<NT>(ca + cb, qscr, tc);
        const uint64_t xs = block_exclusive_scan_u64<NT>(sa + sb, qscr, ts);
        if (pa < R.P) {
          R.coffs[pa] = xc;
          R.soffs[pa] = xs;
        }
        if (pb < R.P) {
          R.coffs[pb] = xc + ca;
          R.soffs[pb] = xs + sa;
        }
      }
    }
    for (uint32_t p = threadIdx.x; p < R.P; p += NT) {
      const uint32_t lo = off_at(p), hi = off_at(p + 1);
      const uint32_t* b = R.bounds + p * (R.S + 1);
      const uint32_t a0 = b[s0], a1 = b[s1];
      if (a0 < lo || a1 > hi || a1 < a0 || (s0 == 0u && a0 != lo) || (s1 == R.S && a1 != hi))
        bad |= SPARCML_FLAG_RUN_TABLE;
      const uint32_t b0 = std::min(std::max(a0, lo), hi), b1 = std::min(std::max(a1, lo), hi);
      runs[p] = make_uint2(b0, b1 > b0 ? b1 - b0 : 0u);
    }
  } else {
    store_run_table<NT, MAXP>(R, s0, s1, runs, nullptr);
  }
  __syncthreads();
  auto mark = [&](uint32_t i) {
    const uint32_t local = i - glo;
    if (local < glen) atomicOr(&bits[local >> 5], 1u << (local & 31));
    else if (RUNS) bad |= i >= R.N ? SPARCML_FLAG_INDEX_RANGE : SPARCML_FLAG_RUN_TABLE;
  };
  const uint32_t step = 1u << lane_bits;  // lanes per node
  // Every lane loads, whether its position is in a run or not, from a
  // position clamped into the array (the last quad, the last index), so that
  // a thread's loads of all its rows are in flight together: loads under a
  // per-lane condition were each waited for before the next was issued.
  // With no pairs at all (the index array may then be null) nothing loads.
  const uint32_t jlast = R.total - 1u, qlast = jlast >> 2;
  for (uint32_t p0 = 0; p0 < (R.total ? R.P : 0u); p0 += sl.groups * kB) {
    uint2 rn[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const uint32_t p = p0 + b * sl.groups + sl.group;
      rn[b] = p < R.P ? runs[p] : make_uint2(0u, 0u);
    }
    if constexpr (QUAD) {
      uint32_t q0[kB], q1[kB];
      uint4 ii[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        q0[b] = rn[b].x >> 2;
        q1[b] = rn[b].y ? (rn[b].x + rn[b].y + 3u) >> 2 : q0[b];
        ii[b] = ld_idx4(idx + 4u * std::min(q0[b] + sl.lane, qlast));
      }
      auto mark4 = [&](uint32_t q, const uint2& r, const uint4& i4) {
        const uint32_t e = 4u * q - r.x;  // run position of the quad's first index (may wrap)
        if (e < r.y) mark(i4.x);
        if (e + 1u < r.y) mark(i4.y);
        if (e + 2u < r.y) mark(i4.z);
        if (e + 3u < r.y) mark(i4.w);
      };
#pragma unroll
      for (int b = 0; b < kB; ++b)
        if (q0[b] + sl.lane < q1[b]) mark4(q0[b] + sl.lane, rn[b], ii[b]);
      for (int b = 0; b < kB; ++b) {  // the rest of runs longer than the group's quads
        if (__ballot(q1[b] - q0[b] > step) == 0ull) continue;
        for (uint32_t q = q0[b] + sl.lane + step; q < q1[b]; q += step) mark4(q, rn[b], ld_idx4(idx + 4u * q));
      }
    } else {
      uint32_t ii[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) ii[b] = idx[std::min(rn[b].x + sl.lane, jlast)];
#pragma unroll
      for (int b = 0; b < kB; ++b)
        if (sl.lane < rn[b].y) mark(ii[b]);
      for (int b = 0; b < kB; ++b) {  // the rest of runs longer than the group
        if (__ballot(rn[b].y > step) == 0ull) continue;
        for (uint32_t j = sl.lane + step; j < rn[b].y; j += step) mark(idx[rn[b].x + j]);
      }
    }
  }
  // the group's check bits: its own, and the bounds pass's words g,
  // g + groups, ... (none when the run table is the caller's)
  if (threadIdx.x == 0)
    for (uint64_t w = g; w < R.nflagw; w += gridDim.x) bad |= R.flagw[w];
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  // the bitmaps, whole waves at a time (the words come in multiples of 128),
  // and the union count of every writer group
  uint32_t* gb = R.bitmaps + s0 * kWords;
  for (uint32_t k = threadIdx.x; k < segs * kWords; k += NT) {
    const uint32_t word = bits[k];
    gb[k] = word;
    const uint32_t c = wave_sum((uint32_t)__popc(word));
    if (lane_id() == 0u) atomicAdd(&wc[k >> (kWordBits + R.mlog)], c);
  }
  __syncthreads();
  const uint64_t wfirst = g << (R.glog - R.mlog);
  const uint64_t wn = std::min<uint64_t>(1u << (R.glog - R.mlog), R.W - wfirst);
  if (threadIdx.x < wn) R.cnt[wfirst + threadIdx.x] = wc[threadIdx.x] | (s_bad << kCountBits);
}

// Exclusive scan of the writer-group counts by one workgroup, into offsets,
// K, the dense decision and the result record. Each thread loads 32
// consecutive counts at once (one round trip per 32768 groups, 16-byte loads
// where the run is whole), scans them in registers, and the per-thread totals
// are scanned across the block.
__global__ __launch_bounds__(1024) void k_decide(RDev R) {
  constexpr int kPer = 32;
  __shared__ uint32_t scr[1024 / kWave + 3];
  __shared__ uint32_t s_flags;
  if (threadIdx.x == 0) s_flags = 0u;
  uint32_t f = 0u;  // the count groups' check bits, from the count words' top bits
  uint64_t carry = 0;
  for (uint64_t s0 = 0; s0 < R.W; s0 += 1024 * kPer) {
    const uint64_t first = s0 + (uint64_t)threadIdx.x * kPer;
    const bool whole = first + kPer <= R.W;  // cnt and off are 256-byte aligned, first % 32 == 0
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
      for (int u = 0; u < kPer; ++u) c[u] = first + u < R.W ? R.cnt[first + u] : 0u;
    }
    uint32_t sum = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      f |= c[u] >> kCountBits;
      c[u] &= kCountMask;
      sum += c[u];
    }
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
        if (first + u < R.W) R.off[first + u] = c[u];
    }
    carry += tot;
  }
  if (f) atomicOr(&s_flags, f);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t dense = carry >= R.T ? 1u : 0u;
    R.state->K = carry;
    R.state->is_dense = dense;
    ReduceResultDev res;
    res.nnz = carry;
    res.is_dense = dense;
    res.flags = s_flags;
    *R.result = res;
  }
}

// What a writer workgroup needs of its group w before merging: whether the
// result is dense, the group's union count and its output offset. After the
// decide pass the last thread loads them (its wave has no run-table loads to
// hold back while it waits). Without it (SCAN, for at most kScanMaxW groups,
// where one more launch costs more than the scan), every workgroup adds up
// the group counts itself: all of them for K, those before w for its offset;
// the workgroup of group 0 stores the result record. load() goes out with the
// other prologue loads; finish() follows the caller's barrier and is called
// by every thread.
constexpr uint64_t kScanMaxW = 4096;  // LSTM-sized reduce, 4096 writer groups: 41.3 -> 39.3 us cold

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

template <int NT, bool SCAN>
struct WriterHead {
  uint32_t before = 0u, all = 0u, flags = 0u;

  __device__ __forceinline__ void load(const RDev& R, uint64_t w, uint32_t* head) {
    if constexpr (!SCAN) {
      if (threadIdx.x == NT - 1) {
        const uint32_t dense = R.state->is_dense, cnt = R.cnt[w] & kCountMask, off = R.off[w];
        head[0] = dense;
        head[1] = cnt;
        head[2] = off;
      }
    } else {
      constexpr int kPer = (int)(kScanMaxW / NT);
      static_assert(kPer % 4 == 0, "whole 16-byte loads");
      const uint64_t first = (uint64_t)threadIdx.x * kPer;  // cnt is 256-byte aligned
      uint32_t c[kPer];
      if (first + kPer <= R.W) {
#pragma unroll
        for (int q = 0; q < kPer / 4; ++q) {
          const uint4 x = reinterpret_cast<const uint4*>(R.cnt + first)[q];
          c[4 * q] = x.x;
          c[4 * q + 1] = x.y;
          c[4 * q + 2] = x.z;
          c[4 * q + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kPer; ++u) c[u] = first + u < R.W ? R.cnt[first + u] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        flags |= c[u] >> kCountBits;  // the result record's check bits (group 0 stores them)
        c[u] &= kCountMask;
        all += c[u];
        before += first + u < w ? c[u] : 0u;
        if (first + u == w) head[1] = c[u];
      }
    }
  }

  // The values are the same in every thread; readfirstlane keeps them in
  // scalar registers and the branches on them uniform.
  __device__ __forceinline__ uint3 finish(const RDev& R, uint64_t w, const uint32_t* head, uint32_t* scratch) {
    if constexpr (!SCAN) {
      return make_uint3(uniform(head[0]), uniform(head[1]), uniform(head[2]));
    } else {
      uint32_t K, off;
      block_sum2<NT>(all, before, scratch, K, off);
      const uint32_t dense = K >= R.T ? 1u : 0u;
      if (w == 0) {  // uniform over the block
        __shared__ uint32_t s_flags;
        if (threadIdx.x == 0) s_flags = 0u;
        __syncthreads();
        if (flags) atomicOr(&s_flags, flags);
        __syncthreads();
        if (threadIdx.x == 0) {
          ReduceResultDev res;
          res.nnz = K;
          res.is_dense = dense;
          res.flags = s_flags;
          *R.result = res;
        }
      }
      return make_uint3(uniform(dense), uniform(head[1]), uniform(off));
    }
  }
};

constexpr int kWriteThreads = 512;
constexpr int kWordWaves = kWords / kWave;  // 2

// Writer for results expected dense: each segment's sums in a 4096-entry
// fp64 LDS tile, written out as float4 when the result is dense; when it
// turns out sparse, each thread stores the union entries of its 8 indices at
// their ranks from the count pass's bitmap.
template <int MAXP, int BITS, bool SCAN>
__global__ __launch_bounds__(kWriteThreads) void k_write_tile(const uint32_t* __restrict__ idx,
                                                              const float* __restrict__ val,
                                                              uint32_t* __restrict__ out_idx,
                                                              float* __restrict__ out_val, RDev R,
                                                              uint32_t lane_bits) {
  constexpr int NT = kWriteThreads;
  constexpr int kB = 4;  // node rows per pass
  __shared__ double acc[kSeg];
  __shared__ uint2 runs[MAXP];
  __shared__ uint32_t scr[3];
  __shared__ uint32_t hscr[SCAN ? 2 * NT / kWave : 1];
  __shared__ QRuns<BITS ? MAXP : 1> qruns;
  const uint64_t s = xcd_contiguous(blockIdx.x, gridDim.x);  // neighbours share run-edge lines
  const uint32_t seg_lo = (uint32_t)(s << kSegBits);
  const uint32_t seg_len = std::min<uint32_t>(kSeg, R.N - seg_lo);
  WriterHead<NT, SCAN> hw;
  hw.load(R, s, scr);
  uint32_t word = 0u;
  if (threadIdx.x < kWords) word = R.bitmaps[s * kWords + threadIdx.x];
  for (uint32_t i = threadIdx.x; i < kSeg; i += NT) acc[i] = 0.0;
  const Slots sl = make_slots(lane_bits, NT);
  store_run_table<NT, BITS ? MAXP : 1>(R, s, s + 1, runs, BITS ? &qruns : nullptr);
  __syncthreads();
  const uint3 hd = hw.finish(R, s, scr, hscr);
  const bool dense = hd.x != 0u;
  const uint32_t seg_cnt = hd.y, seg_off = hd.z;
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
  auto add = [&](uint32_t i, float v) { atomicAdd(&acc[i & (kSeg - 1u)], (double)v); };
  // (loads under the lane's condition, unlike the count pass and the rank
  // writer: clamped loads by every lane measured 3% slower here)
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
      if (__ballot(rn[b].y > step) == 0ull) continue;
      const uint32_t p = p0 + b * sl.groups + sl.group;
      for (uint32_t jr = sl.lane + step; jr < rn[b].y; jr += step) {
        const uint32_t j = rn[b].x + jr;
        add(idx[j], value_at(p, j, jr));
      }
    }
  }
  __shared__ uint32_t wbits[kWords], wrank[kWords], wtot[kWordWaves];  // bitmap words, ranks before them
  if (!dense && threadIdx.x < kWords) {
    const uint32_t c = (uint32_t)__popc(word);
    const uint32_t inc = wave_inclusive_scan(c);
    wbits[threadIdx.x] = word;
    wrank[threadIdx.x] = inc - c;
    if (lane_id() == kWave - 1) wtot[threadIdx.x / kWave] = inc;
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
    return;
  }
  // each thread: indices 8t .. 8t + 7, byte (t mod 4) of word t / 4
  constexpr int kPerT = kSeg / NT;
  static_assert(kPerT == 8 && kWordWaves == 2, "one bitmap byte per thread");
  const uint32_t wi = threadIdx.x / 4;
  const uint32_t wd = wbits[wi];
  const uint32_t sh = 8 * (threadIdx.x & 3);
  const uint32_t byte = (wd >> sh) & 0xFFu;
  uint32_t r = wrank[wi] + (wi >= (uint32_t)kWave ? wtot[0] : 0u) + (uint32_t)__popc(wd & ((1u << sh) - 1u));
#pragma unroll
  for (int t = 0; t < kPerT; ++t) {
    if ((byte >> t) & 1u) {
      const uint64_t pos = (uint64_t)seg_off + r;
      if (pos < R.out_idx_cap) {
        out_idx[pos] = seg_lo + kPerT * threadIdx.x + t;
        out_val[pos] = (float)acc[kPerT * threadIdx.x + t];
      }
      ++r;
    }
  }
}

// Writer placing pairs by their rank in its group's union, for results
// expected sparse; a group is 2^mlog consecutive segments (up to 4, as many
// as keep the group's pairs near the rank slots). The count pass left each
// segment's union bitmap; a word table in LDS (ranks before each 32-index
// word, and the word) gives every pair its rank r in the group with one LDS
// read and a popcount, so the sums accumulate directly in output order and
// are stored as they stand: no clearing or compaction of a dense tile, and
// LDS for the union only.
//
// The pass is bound by the bytes its workgroups have in flight, so each
// memory instruction moves 16 bytes per lane where it can: pairs are loaded
// as aligned quads (QUAD: fp32 values, idx and val 16-byte aligned; else one
// pair per lane), and results are stored as aligned quads: rank r of a
// window whose output starts at position P0 sits in slot r + (P0 mod 4), so
// that slot quads are output quads. Ranks come in windows of kRankCap; a
// group with more union entries takes one pass over its pairs per window.
// A dense result (the count crossed T) writes every index of the group:
// the sum at its rank, or 0 outside the union. For valid input every pair's
// bit is set in the bitmap the count pass built from the same pairs; input
// that failed the checks gives unspecified sums, but every LDS slot touched
// stays inside the window.
constexpr int kRankThreads = 256;
constexpr uint32_t kRankCap = 2560;
// Groups whose expected union leaves room within kRankCapSmall take a writer
// with that many slots: less LDS, more workgroups per compute unit
// (LSTM-sized reduce, 4 segments per group: 39.5 -> 37.2 us cold; with the
// small cap for every call the wide-ResNet reduce, then one segment per
// group, took 234 us instead of 184).
constexpr uint32_t kRankCapSmall = 1536;

template <int MAXP, int BITS, bool QUAD, bool SCAN, uint32_t CAP>
__global__ __launch_bounds__(kRankThreads) void k_write_ranked(const uint32_t* __restrict__ idx,
                                                               const float* __restrict__ val,
                                                               uint32_t* __restrict__ out_idx,
                                                               float* __restrict__ out_val, RDev R,
                                                               uint32_t lane_bits) {
  constexpr int NT = kRankThreads;
  constexpr int kB = QUAD ? 2 : 8;  // node rows per pass
  __shared__ __align__(16) double acc[(CAP + 4)];
  __shared__ __align__(16) uint16_t sloc[(CAP + 4)];  // index within the group
  __shared__ uint2 runs[MAXP];
  __shared__ QRuns<BITS ? MAXP : 1> qruns;
  __shared__ uint32_t scr[3];
  __shared__ uint32_t hscr[SCAN ? 2 * NT / kWave : 1];
  __shared__ uint32_t sscr[NT / kWave + 1];
  extern __shared__ uint2 words[];  // [128 << mlog]: (ranks before the word, the word)
  const uint64_t s = xcd_contiguous(blockIdx.x, gridDim.x);  // neighbours share run-edge lines
  const uint32_t mlog = R.mlog;
  const uint32_t seg_lo = (uint32_t)(s << (kSegBits + mlog));
  const uint32_t span = kSeg << mlog;
  const uint32_t seg_len = std::min<uint32_t>(span, R.N - seg_lo);
  const Slots sl = make_slots(lane_bits, NT);
  // every load of the prologue goes out before any wait: the bitmaps (two
  // words per thread), the counts and totals, and the run table
  const uint32_t npairs = (kWords / 2) << mlog;
  const uint32_t nvalid = (kWords / 2) * (uint32_t)std::min<uint64_t>(1u << mlog, R.S - (s << mlog));
  uint2 wpair = make_uint2(0u, 0u);  // segments past the last (in the last group) hold nothing
  if (threadIdx.x < nvalid) wpair = reinterpret_cast<const uint2*>(R.bitmaps + (s << mlog) * kWords)[threadIdx.x];
  WriterHead<NT, SCAN> hw;
  hw.load(R, s, scr);
  for (uint32_t r = threadIdx.x; r < (CAP + 4); r += NT) acc[r] = 0.0;
  store_run_table<NT, BITS ? MAXP : 1>(R, s << mlog, std::min<uint64_t>((s + 1) << mlog, R.S), runs,
                                       BITS ? &qruns : nullptr);
  const uint32_t c0 = (uint32_t)__popc(wpair.x), c1 = (uint32_t)__popc(wpair.y);
  if (mlog == 0u) {
    if (threadIdx.x < kWave) {  // word table: wave 0
      const uint32_t inc = wave_inclusive_scan(c0 + c1);
      words[2 * threadIdx.x] = make_uint2(inc - c0 - c1, wpair.x);
      words[2 * threadIdx.x + 1] = make_uint2(inc - c1, wpair.y);
    }
  } else {  // word table of several segments: a scan over the block
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<NT>(c0 + c1, sscr, tot);
    if (threadIdx.x < npairs) {
      words[2 * threadIdx.x] = make_uint2(ex, wpair.x);
      words[2 * threadIdx.x + 1] = make_uint2(ex + c0, wpair.y);
    }
  }
  __syncthreads();
  const uint3 hd = hw.finish(R, s, scr, hscr);
  const bool dense = hd.x != 0u;
  const uint32_t seg_cnt = hd.y;
  const uint32_t seg_off = hd.z;
  if (!dense && seg_cnt == 0u) return;  // nothing of this group in a sparse result

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
  const uint32_t lmask = span - 1u;
  const uint32_t windows = std::max<uint32_t>(1u, (seg_cnt + CAP - 1) / CAP);
  for (uint32_t w0 = 0, win = 0; win < windows; ++win, w0 += CAP) {
    const uint32_t sh = (seg_off + w0) & 3u;  // slot of the window's first rank
    const uint32_t base = w0 - sh;             // rank r sits in slot r - base
    if (win > 0) {  // the previous window is stored: clear for this one
      __syncthreads();
      for (uint32_t r = threadIdx.x; r < (CAP + 4); r += NT) acc[r] = 0.0;
      __syncthreads();
    }
    auto add = [&](uint32_t i, float v) {
      const uint32_t local = i & lmask;
      const uint2 wd = words[local >> 5];
      const uint32_t x = wd.x + (uint32_t)__popc(wd.y & ((1u << (local & 31)) - 1u)) - base;
      if (x - sh < CAP) {
        atomicAdd(&acc[x], (double)v);
        sloc[x] = (uint16_t)local;
      }
    };
    // Every lane loads, whether its position is in a run or not, from a
    // position clamped into the arrays (the last quad, the last pair), so
    // that a thread's loads of all its rows are in flight together: loads
    // under the lane's condition were each waited for before the next was
    // issued. With no pairs at all (the arrays may then be null) nothing
    // loads.
    const uint32_t jlast = R.total - 1u, qlast = jlast >> 2;
    for (uint32_t p0 = 0; p0 < (R.total ? R.P : 0u); p0 += sl.groups * kB) {
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
        [[maybe_unused]] QuadCodes<BITS ? BITS : 4> qc[kB];
        uint32_t q0[kB], q1[kB];
        // the quad's values: loaded, or decoded from the node's codes
        auto quad_values = [&](uint32_t q, uint32_t b, uint2 r) -> float4 {
          if constexpr (BITS == 0) {
            return reinterpret_cast<const float4*>(val)[q];
          } else {
            const uint32_t p = p0 + b * sl.groups + sl.group;
            QuadCodes<BITS> c;
            c.load(R, q, r, qruns.rel[p], qruns.cb[p], qruns.sb[p]);
            return c.values();
          }
        };
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          q0[b] = rn[b].x >> 2;
          q1[b] = rn[b].y ? (rn[b].x + rn[b].y + 3u) >> 2 : q0[b];
          const uint32_t q = std::min(q0[b] + sl.lane, qlast);
          ii[b] = ld_idx4_nt(idx + 4u * q);
          if constexpr (BITS == 0) {
            vv[b] = reinterpret_cast<const float4*>(val)[q];
          } else {
            const uint32_t p = std::min(p0 + b * sl.groups + sl.group, R.P - 1u);
            qc[b].load(R, q, rn[b], qruns.rel[p], qruns.cb[p], qruns.sb[p]);
          }
        }
        if constexpr (BITS != 0) {
#pragma unroll
          for (int b = 0; b < kB; ++b) vv[b] = qc[b].values();
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
            add4(q, rn[b], ld_idx4_nt(idx + 4u * q), quad_values(q, b, rn[b]));
        }
      } else {
        uint32_t ii[kB];
        float vv[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          if constexpr (BITS == 0) {
            const uint32_t j = std::min(rn[b].x + sl.lane, jlast);
            ii[b] = idx[j];
            vv[b] = val[j];
          } else if (sl.lane < rn[b].y) {
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
    if (dense) {  // every index of the group: its sum, or 0 outside the union
      float* out = out_val + seg_lo;
      const bool whole = windows == 1u && seg_len == span;
      for (uint32_t q = threadIdx.x; q < (seg_len + 3) / 4; q += NT) {
        const uint2 wd = words[q >> 3];
        float o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t local = 4 * q + t;
          const uint32_t bit = 1u << (local & 31);
          const uint32_t x = wd.x + (uint32_t)__popc(wd.y & (bit - 1u)) - base;
          const bool in = (wd.y & bit) && x - sh < CAP;
          o[t] = in ? (float)acc[x] : 0.0f;
          if (!whole && local < seg_len && (in || (!(wd.y & bit) && win == 0u))) out[local] = o[t];
        }
        if (whole) reinterpret_cast<float4*>(out)[q] = make_float4(o[0], o[1], o[2], o[3]);
      }
    } else {
      // slots [sh, sh + n) hold ranks w0 .. w0 + n - 1, at output positions
      // pos0 + slot with pos0 = seg_off + w0 - sh a multiple of 4, so slot
      // quads are output quads
      const uint32_t n = std::min(seg_cnt - w0, CAP);
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

size_t reduce_workspace_bytes(uint32_t P, uint64_t N, uint64_t total_nnz) {
  return make_layout(P, N, total_nnz).total;
}

namespace {

template <int MAXP, bool SCAN>
hipError_t launch_write_tile(uint32_t bits, dim3 grid, hipStream_t stream, hipEvent_t e0, hipEvent_t e1,
                             const uint32_t* idx, const float* val, uint32_t* out_idx, float* out_val, const RDev& R,
                             uint32_t lb) {
  const dim3 block(kWriteThreads);
  switch (bits) {
    case 0:
      return launch_ev(k_write_tile<MAXP, 0, SCAN>, grid, block, stream, e0, e1, idx, val, out_idx, out_val, R, lb);
    case 2:
      return launch_ev(k_write_tile<MAXP, 2, SCAN>, grid, block, stream, e0, e1, idx, val, out_idx, out_val, R, lb);
    case 4:
      return launch_ev(k_write_tile<MAXP, 4, SCAN>, grid, block, stream, e0, e1, idx, val, out_idx, out_val, R, lb);
    default:
      return launch_ev(k_write_tile<MAXP, 8, SCAN>, grid, block, stream, e0, e1, idx, val, out_idx, out_val, R, lb);
  }
}

template <int MAXP, bool SCAN>
hipError_t launch_write_ranked(uint32_t bits, bool quad, bool small_cap, dim3 grid, hipStream_t stream, hipEvent_t e0,
                               hipEvent_t e1,
                               const uint32_t* idx, const float* val, uint32_t* out_idx, float* out_val,
                               const RDev& R, uint32_t lb, uint32_t lbq) {
  const dim3 block(kRankThreads);
  const size_t lds = sizeof(uint2) * ((size_t)kWords << R.mlog);  // the word table
  auto go = [&](auto kq, auto kp) {
    constexpr int B = decltype(kq)::value;
    constexpr bool Q = decltype(kp)::value;
    return small_cap ? launch_ev_lds(k_write_ranked<MAXP, B, Q, SCAN, kRankCapSmall>, grid, block, lds, stream, e0,
                                     e1, idx, val, out_idx, out_val, R, Q ? lbq : lb)
                     : launch_ev_lds(k_write_ranked<MAXP, B, Q, SCAN, kRankCap>, grid, block, lds, stream, e0, e1, idx,
                                     val, out_idx, out_val, R, Q ? lbq : lb);
  };
  using T = std::true_type;
  using F = std::false_type;
  switch (bits) {
    case 0: return quad ? go(std::integral_constant<int, 0>{}, T{}) : go(std::integral_constant<int, 0>{}, F{});
    case 2: return quad ? go(std::integral_constant<int, 2>{}, T{}) : go(std::integral_constant<int, 2>{}, F{});
    case 4: return quad ? go(std::integral_constant<int, 4>{}, T{}) : go(std::integral_constant<int, 4>{}, F{});
    default: return quad ? go(std::integral_constant<int, 8>{}, T{}) : go(std::integral_constant<int, 8>{}, F{});
  }
}

// The writer for (tile or rank order) x (nodes up to 256 or 1024: the run
// table's LDS) x (its own scan or the decide pass's).
template <bool SCAN>
hipError_t launch_writer(bool tile, bool quad, bool small_cap, dim3 grid, hipStream_t stream, hipEvent_t e0,
                         hipEvent_t e1,
                         const uint32_t* idx, const float* val, uint32_t* out_idx, float* out_val, const RDev& R,
                         uint32_t lb, uint32_t lbq) {
  if (tile)
    return R.P <= 256
               ? launch_write_tile<256, SCAN>(R.bits, grid, stream, e0, e1, idx, val, out_idx, out_val, R, lb)
               : launch_write_tile<kMaxP, SCAN>(R.bits, grid, stream, e0, e1, idx, val, out_idx, out_val, R, lb);
  return R.P <= 256
             ? launch_write_ranked<256, SCAN>(R.bits, quad, small_cap, grid, stream, e0, e1, idx, val, out_idx, out_val, R, lb,
                                              lbq)
             : launch_write_ranked<kMaxP, SCAN>(R.bits, quad, small_cap, grid, stream, e0, e1, idx, val, out_idx, out_val, R, lb,
                                                lbq);
}

// Lanes per node in the write passes (as a power of two): about 1.5 times
// the mean run length of a node in a writer group, so that few runs spill
// past their lanes while lanes stay mostly busy; 16 to 128.
uint32_t lanes_log2(uint32_t P, uint64_t W, uint64_t total) {
  const double mean = (double)total / ((double)P * (double)W);
  uint32_t lb = 4;
  while (lb < 7 && (double)(1u << lb) < 1.5 * mean) ++lb;
  return lb;
}

// Lanes per node when each lane takes an aligned quad of pairs: the mean
// number of quads a run meets (its length / 4, plus 3/4 for the unaligned
// ends) with room for one standard deviation and more; 2 to 64.
uint32_t quad_lanes_log2(uint32_t P, uint64_t W, uint64_t total) {
  const double mean = (double)total / ((double)P * (double)W);
  const double quads = mean / 4.0 + 0.75 + std::sqrt(mean) / 4.0 + 1.0;
  uint32_t lb = 1;
  while (lb < 6 && (double)(1u << lb) < quads) ++lb;
  return lb;
}

// Segments per rank-order writer group (log2): as many as keep the group's
// expected union u (from the estimate) with room for 4 sqrt(u) + 16 more
// within the rank slots, and leave at least kWriterGroupsWanted groups. A
// union past the slots costs one more pass over the group's pairs. The tile
// writer takes one segment.
uint32_t writer_log2(uint64_t S, double union_est, bool tile) {
  if (tile) return 0;
  const double per_seg = union_est / (double)S;
  auto fits = [&](uint32_t m) {
    const double u = (double)(1u << m) * per_seg;
    return u + 4.0 * std::sqrt(u) + 16.0 <= (double)kRankCap;
  };
  uint32_t m = 0;
  while (m < kMaxWriterLog2 && fits(m + 1) && (S >> (m + 1)) >= kWriterGroupsWanted) ++m;
  return m;
}

// Whether groups of 2^mlog segments fit the writer with kRankCapSmall slots
// by the same margin.
bool writer_small_cap(uint64_t S, double union_est, uint32_t mlog) {
  const double u = (double)(1u << mlog) * union_est / (double)S;
  return u + 4.0 * std::sqrt(u) + 16.0 <= (double)kRankCapSmall;
}

// Segments per count group (log2): a multiple of the writer group, doubled
// while its pairs stay below `pairs` (kCountPairs, or kCountPairsRuns with
// the caller's run table), a node's mean run in the doubled
// group within kCountRun, and at least kCountGroupsWanted groups remain.
uint32_t count_log2(uint32_t P, uint64_t S, uint64_t total, uint32_t mlog, double pairs) {
  const double per_seg = (double)total / (double)S;
  uint32_t g = mlog;
  while (g < kMaxCountLog2 && (double)(1u << g) * per_seg < pairs &&
         (double)(2u << g) * per_seg / (double)P <= kCountRun && (S >> (g + 1)) >= kCountGroupsWanted)
    ++g;
  return g;
}

}  // namespace

hipError_t sparse_reduce_launch(uint32_t P, uint64_t N, uint64_t T, const uint64_t* h_offsets,
                                const uint32_t* idx, const float* val, const ReduceQuantized* quant,
                                const uint32_t* runs, bool dense_first, double union_est, uint32_t* out_idx,
                                uint64_t out_idx_cap, float* out_val, ReduceResultDev* d_result, void* ws,
                                hipStream_t stream, const OpEvents* ev, int phase) {
  const Layout L = make_layout(P, N, h_offsets[P]);
  // measurement events: the op's span runs from its first dispatch to the
  // writer's end; the kernel pair times the writer alone. A union phase's
  // span ends at its last kernel; the sums phase is the writer alone, which
  // then carries the op's pair (or else the kernel pair).
  const bool do_union = (phase & kReduceUnion) != 0, do_sums = (phase & kReduceSums) != 0;
  const OpEvents none{};
  const OpEvents& E = ev ? *ev : none;
  char* w = static_cast<char*>(ws);
  RDev R{};
  R.P = P;
  R.N = (uint32_t)N;
  R.total = (uint32_t)h_offsets[P];
  R.mlog = writer_log2(L.S, union_est, dense_first);
  R.glog = count_log2(P, L.S, R.total, R.mlog, runs ? kCountPairsRuns : kCountPairs);
  R.pad = 0;
  R.S = L.S;
  R.W = (L.S + (1u << R.mlog) - 1) >> R.mlog;
  R.T = T;
  R.out_idx_cap = out_idx_cap;
  R.state = reinterpret_cast<State*>(w + L.state);
  R.offs = reinterpret_cast<uint64_t*>(w + L.offs);
  R.flagw = reinterpret_cast<uint32_t*>(w + L.flagw);
  // the caller's run table is only read (by the count pass and the writer)
  R.bounds = runs ? const_cast<uint32_t*>(runs) : reinterpret_cast<uint32_t*>(w + L.bounds);
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

  // offsets inline to the bounds pass for up to 255 nodes, else by setup launches
  InlineOffsets in;
  const bool inline_offs = P + 1 <= (uint32_t)kInlineOffsets;
  const bool scan_in_writer = R.W <= kScanMaxW;
  hipError_t e = hipSuccess;
  if (do_union) {
  if (inline_offs) {
    for (uint32_t i = 0; i <= P; ++i) in.v[i] = h_offsets[i];
  } else {
    for (uint32_t first = 0; first < P + 1; first += kInlineOffsets) {
      InlineOffsets part;
      const uint32_t count = std::min<uint32_t>(kInlineOffsets, P + 1 - first);
      for (uint32_t i = 0; i < count; ++i) part.v[i] = h_offsets[first + i];
      const hipError_t e = launch_ev(k_setup, dim3(1), dim3(256), stream, first == 0 ? E.op_start : nullptr, nullptr,
                                     R, first, count, part);
      if (e != hipSuccess) return e;
    }
    if (R.bits) hipLaunchKernelGGL(k_qoffsets, dim3(1), dim3(1024), 0, stream, R);
  }
  if (runs == nullptr) {
    const uint32_t bx = bounds_blocks(max_nnz);
    R.nflagw = (uint64_t)bx * P;
    const uint32_t shift = (uint32_t)((reinterpret_cast<uintptr_t>(idx) >> 2) & 3u);
    e = launch_ev(k_bounds, dim3(bx, P), dim3(kThreads), stream, inline_offs ? E.op_start : nullptr, nullptr, idx, R,
                  shift, in, inline_offs ? 1 : 0);
    if (e != hipSuccess) return e;
  }
  const bool small_p = P <= 256;
  const uint64_t groups = (L.S + (1u << R.glog) - 1) >> R.glog;  // count workgroups
  const dim3 cgrid((uint32_t)groups);
  const uint32_t lbc = lanes_log2(P, groups, R.total);
  const size_t clds = sizeof(uint32_t) * ((size_t)kWords << R.glog);
  const bool idx_quads = (reinterpret_cast<uintptr_t>(idx) & 15u) == 0;  // the count pass loads aligned quads
  const uint32_t lbcq = std::min<uint32_t>(quad_lanes_log2(P, groups, R.total), 7u);
  const uint32_t lbk = idx_quads ? lbcq : lbc;
  const dim3 cblock(kCountThreads);
  // a union phase ends with the decide pass or, without one, the count pass
  const hipEvent_t c1 = !do_sums && scan_in_writer ? E.op_stop : nullptr;
  if (runs != nullptr) {
    // no bounds pass: the count pass is the op's first kernel (after any setup launches)
    const hipEvent_t c0 = inline_offs ? E.op_start : nullptr;
    const int io = inline_offs ? 1 : 0;
    if (small_p)
      e = idx_quads ? launch_ev_lds(k_count<256, true, true>, cgrid, cblock, clds, stream, c0, c1, idx, R, lbk, in, io)
                    : launch_ev_lds(k_count<256, false, true>, cgrid, cblock, clds, stream, c0, c1, idx, R, lbk, in, io);
    else
      e = idx_quads
              ? launch_ev_lds(k_count<kMaxP, true, true>, cgrid, cblock, clds, stream, c0, c1, idx, R, lbk, in, io)
              : launch_ev_lds(k_count<kMaxP, false, true>, cgrid, cblock, clds, stream, c0, c1, idx, R, lbk, in, io);
  } else {
    const NoOffsets no{};
    if (small_p)
      e = idx_quads ? launch_ev_lds(k_count<256, true, false>, cgrid, cblock, clds, stream, nullptr, c1, idx, R, lbk, no, 0)
                    : launch_ev_lds(k_count<256, false, false>, cgrid, cblock, clds, stream, nullptr, c1, idx, R, lbk, no,
                                    0);
    else
      e = idx_quads
              ? launch_ev_lds(k_count<kMaxP, true, false>, cgrid, cblock, clds, stream, nullptr, c1, idx, R, lbk, no, 0)
              : launch_ev_lds(k_count<kMaxP, false, false>, cgrid, cblock, clds, stream, nullptr, c1, idx, R, lbk, no,
                              0);
  }
  if (e != hipSuccess) return e;
  if (!scan_in_writer) {
    e = launch_ev(k_decide, dim3(1), dim3(1024), stream, nullptr, do_sums ? nullptr : E.op_stop, R);
    if (e != hipSuccess) return e;
  }
  }  // do_union
  if (!do_sums) return hipSuccess;
  // the writer is the op's last kernel: it carries the kernel pair, or the
  // op's stop alone (a sums phase: the op's pair, or else the kernel pair)
  const bool alone = !do_union;
  const hipEvent_t w0 = alone && E.op_start ? E.op_start : E.k_start;
  const hipEvent_t w1 = alone && E.op_start ? E.op_stop : (E.k_stop ? E.k_stop : E.op_stop);
  const dim3 wgrid((uint32_t)R.W);
  const uint32_t lb = lanes_log2(P, R.W, R.total);
  // the estimate expecting a dense result takes the full tile; rank order
  // loads 16-byte quads of pairs where both arrays allow them
  // (quantized input: 16-byte index quads and 4-byte code words)
  const bool quad = R.bits == 0
                        ? ((reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(val)) & 15u) == 0
                        : (reinterpret_cast<uintptr_t>(idx) & 15u) == 0 && (reinterpret_cast<uintptr_t>(R.codes) & 3u) == 0;
  const uint32_t lbq = quad_lanes_log2(P, R.W, R.total);
  const bool small_cap = !dense_first && writer_small_cap(L.S, union_est, R.mlog);
  e = scan_in_writer
          ? launch_writer<true>(dense_first, quad, small_cap, wgrid, stream, w0, w1, idx, val, out_idx, out_val, R, lb,
                                lbq)
          : launch_writer<false>(dense_first, quad, small_cap, wgrid, stream, w0, w1, idx, val, out_idx, out_val, R, lb,
                                 lbq);
  // with both pairs asked for, the op's stop follows the writer's at once
  if (e == hipSuccess && !(alone && E.op_start) && E.k_stop && E.op_stop) e = hipEventRecord(E.op_stop, stream);
  return e;
}

}  // namespace sparcml
