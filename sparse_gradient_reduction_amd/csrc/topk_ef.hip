// Error-feedback Top-k for gfx950.
//
// SparCML (paperlayer.ai digest of arXiv 1802.08021v3), section 2.2: each
// node sends its k largest-magnitude components and accumulates the rest for
// the next iteration; section 4: the unapplied part is the residual error.
//
// Exact selection, HBM-streaming design. The method's work is one pass over
// grad and residual (read 8 B, write 4 B per element); everything after it
// works on a small candidate list:
//
//   predict  one block per node reads a stratified sample (1024 chunks of 64
//            elements) of a = grad + residual and picks two key thresholds:
//            `lo`, that the k-th largest key T* exceeds with high probability
//            (for certain when the sample is the whole node), and `mid`, the
//            sample's estimate of T*. It also resets the node's state.
//   stream   one pass over 1024-element tiles: a = grad + residual; elements
//            with key >= lo are compacted in index order inside the tile
//            (wave ballots and prefix counts) and appended as one run to the
//            node's candidate buffer, reserved with one atomic on one of 256
//            counters (one counter would serialise the tiles; runs of 16
//            neighbouring tiles share a counter, so they land close together,
//            and 256 counters exceed the slot groups in flight, so groups do
//            not interleave inside a region);
//            residual is written back as a, with stored candidates whose key
//            is >= mid written as +0 (they are almost surely selected).
//   tsum     candidate counts summed per group of 1024 tiles.
//   gscan    per node: group offsets, candidate count, and the path: the
//            candidate list when every tile was stored and it holds >= k
//            candidates, else an exact rescan of the whole node.
//   restore  rescan path only: zeroed candidates go back into residual.
//   gather   candidate runs copied into index order; LDS histogram of key
//            bits 30..20 (first radix level) on the way.
//   hist     further radix levels of T* (bits 19..10, 9..0) over the ordered
//            candidates, or all three levels over the residual on the rescan
//            path; each level's digit is picked from the previous histogram.
//   count    per chunk of 4096 candidates: how many have key > T*, == T*.
//   scan     per node: the tie quota m goes to the lowest indices; output
//            offset of every chunk.
//   emit     per chunk, in index order: selected pairs to the output, and the
//            residual fixed where the guess `mid` was wrong (selected below
//            mid: zeroed; not selected at or above mid: restored).
//
// Every element with key >= T* is a candidate whenever the list holds at
// least k of them, so both paths give the same exact result; the sample only
// decides how much the candidate work costs.
#include "device_common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <cmath>

namespace sparcml {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kTile = 4 * kStreamThreads;                 // 1024 elements per tile, one float4 per thread
constexpr int kNW = kStreamThreads / kWave;               // waves per stream block
constexpr int kSub = 256;                                 // reservation counters per node
constexpr int kTilesPerSlot = 16;                         // consecutive tiles sharing a counter
constexpr int kSampleChunks = 1024;
constexpr int kSampleChunk = 64;
constexpr int kSample = kSampleChunks * kSampleChunk;     // 65536
constexpr int kPredictThreads = 1024;
constexpr int kH0 = 2048, kH1 = 1024, kH2 = 1024;         // radix digits: 11 + 10 + 10 bits
constexpr int kGroup = 1024;                              // tiles per gather group
constexpr int kChunkThreads = 256;
constexpr int kChunkIt = 16;
constexpr int kChunk = kChunkThreads * kChunkIt;          // 4096 candidates per chunk
constexpr uint32_t kNotStored = 0xFFFFFFFFu;

struct NodeState {
  uint32_t lo;      // candidate threshold on the key
  uint32_t mid;     // zeroing threshold on the key (estimate of T*)
  uint32_t count;   // candidates of the node
  uint32_t fail;    // some tile did not fit its counter's region
  uint32_t mode;    // 0 candidates, 1 exact rescan
  uint32_t T;       // k-th largest key
  uint32_t m;       // how many elements with key == T are selected
  uint32_t pad;
};

struct Layout {
  uint64_t capS;  // candidate slots per counter region
  uint64_t cap;   // candidate slots per node (kSub * capS)
  uint64_t MT;    // tiles per node (slots)
  uint64_t MG;    // tile groups per node
  uint64_t MC;    // chunks per node (slots, rescan worst case)
  size_t info, err, state, h0, h1, h2, sub, cand, oidx, oval, tmeta, gsum, gbase, cgt, ceq, ceqoff,
      cout, total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout make_layout(uint32_t P, uint64_t N, uint64_t k) {
  Layout L{};
  const uint64_t want = std::min<uint64_t>(N, 2 * k + 65536);
  L.capS = (want + kSub - 1) / kSub + kTile;  // + one whole tile of slack per region
  L.cap = kSub * L.capS;
  L.MT = (N + 3 + kTile - 1) / kTile;
  L.MG = (L.MT + kGroup - 1) / kGroup;
  L.MC = std::max<uint64_t>(1, (N + kChunk - 1) / kChunk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.info = take(8ull * P);  // [P] path per node, then [P] consistency flags
  L.err = L.info + 4ull * P;
  L.state = take(sizeof(NodeState) * P);
  L.h0 = take(4ull * P * kH0);
  L.h1 = take(4ull * P * kH1);
  L.h2 = take(4ull * P * kH2);
  L.sub = take(128ull * P * kSub);  // one counter per 128-byte line
  L.cand = take(8ull * P * L.cap);
  L.oidx = take(4ull * P * L.cap);
  L.oval = take(4ull * P * L.cap);
  L.tmeta = take(8ull * P * L.MT);
  L.gsum = take(4ull * P * L.MG);
  L.gbase = take(4ull * P * L.MG);
  L.cgt = take(4ull * P * L.MC);
  L.ceq = take(4ull * P * L.MC);
  L.ceqoff = take(4ull * P * L.MC);
  L.cout = take(4ull * P * L.MC);
  L.total = o;
  return L;
}

struct Dev {
  uint32_t P;
  uint32_t N;
  uint32_t k;
  uint32_t rs_lo;   // sample rank of the candidate threshold
  uint32_t rs_mid;  // sample rank of the zeroing threshold
  uint32_t pad;
  uint64_t capS;
  uint64_t cap;
  uint64_t MT;
  uint64_t MG;
  uint64_t MC;
  uint32_t* info;
  uint32_t* err;
  NodeState* state;
  uint32_t* h0;
  uint32_t* h1;
  uint32_t* h2;
  uint32_t* sub;
  uint64_t* cand;  // unordered runs: index << 32 | value bits
  uint32_t* oidx;
  float* oval;
  uint64_t* tmeta;  // per tile: candidate count << 32 | run offset (or kNotStored)
  uint32_t* gsum;
  uint32_t* gbase;
  uint32_t* cgt;
  uint32_t* ceq;
  uint32_t* ceqoff;
  uint32_t* cout;
};

__device__ __forceinline__ uint32_t node_tiles(const Dev& D, uint32_t p) {
  const uint32_t phi = (uint32_t)(((uint64_t)p * D.N) & 3u);
  return (uint32_t)(((uint64_t)D.N + phi + kTile - 1) / kTile);
}

// Source of the select, count and emit kernels: the ordered candidate list,
// or the whole node (residual holds a) on the rescan path.
__device__ __forceinline__ uint64_t source_len(const Dev& D, uint32_t p, bool rescan) {
  return rescan ? (uint64_t)D.N : (uint64_t)D.state[p].count;
}

// ---------------------------------------------------------------------------
// predict: reset the node's state and choose the two key thresholds.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPredictThreads) void k_predict(const float* __restrict__ g,
                                                             const float* __restrict__ r, Dev D) {
  __shared__ uint32_t h1[4096];
  __shared__ uint32_t h2lo[2048];
  __shared__ uint32_t h2mid[2048];
  __shared__ uint32_t scr[kPredictThreads / kWave + 3];
  const uint32_t p = blockIdx.x;
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < kH0; i += kPredictThreads) D.h0[(size_t)p * kH0 + i] = 0u;
  for (uint32_t i = tid; i < kH1; i += kPredictThreads) D.h1[(size_t)p * kH1 + i] = 0u;
  for (uint32_t i = tid; i < kH2; i += kPredictThreads) D.h2[(size_t)p * kH2 + i] = 0u;
  for (uint32_t i = tid; i < kSub; i += kPredictThreads) D.sub[((size_t)p * kSub + i) * 32] = 0u;
  for (uint32_t i = tid; i < 4096; i += kPredictThreads) h1[i] = 0u;
  for (uint32_t i = tid; i < 2048; i += kPredictThreads) h2lo[i] = h2mid[i] = 0u;

  uint32_t lo, mid;
  if (D.k == 0) {
    lo = mid = 0xFFFFFFFFu;  // keys are < 2^31: no candidate
  } else if (D.k == D.N) {
    lo = mid = 0u;  // everything is selected
  } else {
    __syncthreads();
    const uint64_t base = (uint64_t)p * D.N;
    const bool whole = D.N <= (uint32_t)kSample;
    uint32_t keys[kSample / kPredictThreads];
#pragma unroll
    for (int j = 0; j < kSample / kPredictThreads; ++j) {
      const uint32_t i = j * kPredictThreads + tid;
      uint32_t key = 0xFFFFFFFFu;  // marks "no sample"
      if (whole) {
        if (i < D.N) key = mag_key(g[base + i] + r[base + i]);
      } else {
        const uint32_t c = i / kSampleChunk, o = i % kSampleChunk;
        const uint64_t start = (uint64_t)c * (D.N - kSampleChunk) / (kSampleChunks - 1);
        key = mag_key(g[base + start + o] + r[base + start + o]);
      }
      keys[j] = key;
    }
#pragma unroll
    for (int j = 0; j < kSample / kPredictThreads; ++j)
      if (keys[j] != 0xFFFFFFFFu) atomicAdd(&h1[keys[j] >> 19], 1u);
    __syncthreads();
    uint32_t b_lo, a_lo, b_mid, a_mid;
    block_find_suffix<kPredictThreads>(h1, 4096, D.rs_lo, scr, b_lo, a_lo);
    block_find_suffix<kPredictThreads>(h1, 4096, D.rs_mid, scr, b_mid, a_mid);
#pragma unroll
    for (int j = 0; j < kSample / kPredictThreads; ++j) {
      const uint32_t key = keys[j];
      if (key == 0xFFFFFFFFu) continue;
      if ((key >> 19) == b_lo) atomicAdd(&h2lo[(key >> 8) & 2047u], 1u);
      if ((key >> 19) == b_mid) atomicAdd(&h2mid[(key >> 8) & 2047u], 1u);
    }
    __syncthreads();
    uint32_t c_lo, x_lo, c_mid, x_mid;
    block_find_suffix<kPredictThreads>(h2lo, 2048, D.rs_lo - a_lo, scr, c_lo, x_lo);
    block_find_suffix<kPredictThreads>(h2mid, 2048, D.rs_mid - a_mid, scr, c_mid, x_mid);
    lo = (b_lo << 19) | (c_lo << 8);
    mid = (b_mid << 19) | (c_mid << 8);
  }
  if (tid == 0) {
    NodeState s{};
    s.lo = lo;
    s.mid = mid;
    D.state[p] = s;
    D.err[p] = 0u;
    D.info[p] = 0u;
  }
}

// ---------------------------------------------------------------------------
// stream: a = g + r, per-tile candidate compaction, residual write-back.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kStreamThreads) void k_stream(const float* __restrict__ g,
                                                           float* __restrict__ r, Dev D) {
  __shared__ uint32_t s_cnt[kNW];
  __shared__ uint32_t s_base;
  __shared__ uint32_t s_stored;
  // each XCD streams one contiguous stretch of tiles (steadier than the
  // default round-robin of consecutive tiles over the 8 XCDs)
  const uint32_t w = xcd_contiguous(blockIdx.x, gridDim.x);
  const uint32_t p = w / (uint32_t)D.MT;
  const uint32_t t = w % (uint32_t)D.MT;
  if (t >= node_tiles(D, p)) return;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = lane_id();
  const uint32_t wid = tid / kWave;
  const uint32_t N = D.N;
  const uint64_t pN = (uint64_t)p * N;
  const int64_t e0 = (int64_t)t * kTile - (int64_t)(pN & 3u) + 4 * (int64_t)tid;  // node-local index
  const uint64_t grp = (pN >> 2) + (uint64_t)t * (kTile / 4) + tid;               // float4 group
  const uint32_t lo = D.state[p].lo;
  const uint32_t mid = D.state[p].mid;
  const bool full = e0 >= 0 && e0 + 4 <= (int64_t)N;

  float a[4];
  uint32_t own = 0xFu;
  if (full) {
    const f32x4 gv = load_nt(reinterpret_cast<const f32x4*>(g) + grp);
    const f32x4 rv = load_nt(reinterpret_cast<const f32x4*>(r) + grp);
    a[0] = gv.x + rv.x;
    a[1] = gv.y + rv.y;
    a[2] = gv.z + rv.z;
    a[3] = gv.w + rv.w;
  } else {
    own = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t e = e0 + c;
      a[c] = 0.0f;
      if (e >= 0 && e < (int64_t)N) {
        a[c] = g[pN + (uint64_t)e] + r[pN + (uint64_t)e];
        own |= 1u << c;
      }
    }
  }

  uint32_t flags = 0, high = 0;  // bit c: candidate / key >= mid
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t key = mag_key(a[c]);
    if (((own >> c) & 1u) && key >= lo) flags |= 1u << c;
    if (key >= mid) high |= 1u << c;
  }
  // index order inside the tile is (wave, lane, c)
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint64_t m = ballot((flags >> c) & 1u);
    pre += lanes_below(m);
    tot += popc64(m);
  }
  if (lane == 0) s_cnt[wid] = tot;
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int i = 0; i < kNW; ++i) {
      const uint32_t c = s_cnt[i];
      s_cnt[i] = run;
      run += c;
    }
    const uint32_t sc = (t / kTilesPerSlot) % kSub;
    uint32_t off = run ? atomicAdd(&D.sub[((size_t)p * kSub + sc) * 32], run) : 0u;
    const bool stored = (uint64_t)off + run <= D.capS;
    D.tmeta[(size_t)p * D.MT + t] = ((uint64_t)run << 32) | (stored ? (uint32_t)(sc * D.capS + off) : kNotStored);
    if (!stored) atomicOr(&D.state[p].fail, 1u);
    s_base = (uint32_t)(sc * D.capS + off);
    s_stored = stored ? 1u : 0u;
  }
  __syncthreads();
  const bool stored = s_stored != 0u;
  if (stored && flags) {
    uint32_t pos = s_base + s_cnt[wid] + pre;
    uint64_t* cd = D.cand + (size_t)p * D.cap;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((flags >> c) & 1u) {
        cd[pos] = ((uint64_t)(uint32_t)(e0 + c) << 32) | __float_as_uint(a[c]);
        ++pos;
      }
    }
  }
  const uint32_t zero = stored ? (flags & high) : 0u;
  if (full) {
    f32x4 o;
    o.x = (zero & 1u) ? 0.0f : a[0];
    o.y = (zero & 2u) ? 0.0f : a[1];
    o.z = (zero & 4u) ? 0.0f : a[2];
    o.w = (zero & 8u) ? 0.0f : a[3];
    store_nt(o, reinterpret_cast<f32x4*>(r) + grp);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if ((own >> c) & 1u) r[pN + (uint64_t)(e0 + c)] = ((zero >> c) & 1u) ? 0.0f : a[c];
  }
}

// ---------------------------------------------------------------------------
// tsum: candidate count of every group of 1024 tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_tsum(Dev D) {
  __shared__ uint32_t scr[256 / kWave + 3];
  const uint32_t p = blockIdx.y;
  const uint64_t gidx = blockIdx.x;
  const uint32_t nt = node_tiles(D, p);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kGroup / 256; ++i) {
    const uint64_t t = gidx * kGroup + (uint64_t)i * 256 + threadIdx.x;
    if (t < nt) s += (uint32_t)(D.tmeta[(size_t)p * D.MT + t] >> 32);
  }
  uint32_t tot;
  block_exclusive_scan<256>(s, scr, tot);
  if (threadIdx.x == 0) D.gsum[(size_t)p * D.MG + gidx] = tot;
}

// ---------------------------------------------------------------------------
// gscan: group offsets, candidate count and the path of the node.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_gscan(Dev D) {
  __shared__ uint32_t scr[1024 / kWave + 3];
  const uint32_t p = blockIdx.x;
  const uint64_t ng = (node_tiles(D, p) + kGroup - 1) / kGroup;
  uint64_t carry = 0;
  for (uint64_t g0 = 0; g0 < ng; g0 += 1024) {
    const uint64_t gi = g0 + threadIdx.x;
    const uint32_t v = gi < ng ? D.gsum[(size_t)p * D.MG + gi] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<1024>(v, scr, tot);
    if (gi < ng) D.gbase[(size_t)p * D.MG + gi] = (uint32_t)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) {
    const bool rescan = D.state[p].fail != 0u || carry < D.k || carry > D.cap;
    D.state[p].count = (uint32_t)std::min<uint64_t>(carry, D.cap);
    D.state[p].mode = rescan ? 1u : 0u;
    D.info[p] = rescan ? 1u : 0u;
  }
}

// ---------------------------------------------------------------------------
// restore: rescan path only - zeroed candidates go back into residual.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_restore(float* __restrict__ r, Dev D) {
  const uint32_t p = blockIdx.y;
  if (D.state[p].mode == 0u) return;
  const uint32_t mid = D.state[p].mid;
  const uint32_t nt = node_tiles(D, p);
  const uint64_t pN = (uint64_t)p * D.N;
  for (uint64_t t = (uint64_t)blockIdx.x * 256 + threadIdx.x; t < nt; t += (uint64_t)gridDim.x * 256) {
    const uint64_t meta = D.tmeta[(size_t)p * D.MT + t];
    const uint32_t off = (uint32_t)meta;
    const uint32_t cnt = (uint32_t)(meta >> 32);
    if (off == kNotStored) continue;
    for (uint32_t j = 0; j < cnt; ++j) {
      const uint64_t c = D.cand[(size_t)p * D.cap + off + j];
      const float v = __uint_as_float((uint32_t)c);
      if (mag_key(v) >= mid) r[pN + (uint32_t)(c >> 32)] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// gather: candidate runs into index order, first radix level on the way.
// A block owns 1024 consecutive tiles, whose runs land contiguously in the
// ordered list; each thread walks output positions and finds its tile by a
// binary search over the block's prefix of run lengths in LDS, so loads and
// stores stay spread over the whole block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGroup) void k_gather(Dev D) {
  constexpr int kU = 8;
  __shared__ uint32_t h[kH0];
  __shared__ uint32_t s_excl[kGroup + 1];
  __shared__ uint32_t s_toff[kGroup];
  __shared__ uint32_t scr[kGroup / kWave + 3];
  const uint32_t p = blockIdx.y;
  if (D.state[p].mode != 0u) return;
  const uint64_t gidx = blockIdx.x;
  const uint32_t nt = node_tiles(D, p);
  if (gidx * kGroup >= nt) return;
  for (uint32_t i = threadIdx.x; i < kH0; i += kGroup) h[i] = 0u;
  const uint64_t t = gidx * kGroup + threadIdx.x;
  const uint64_t meta = t < nt ? D.tmeta[(size_t)p * D.MT + t] : 0ull;
  const uint32_t cnt = (uint32_t)(meta >> 32);
  s_toff[threadIdx.x] = cnt ? (uint32_t)meta : 0u;
  uint32_t tot;
  s_excl[threadIdx.x] = block_exclusive_scan<kGroup>(cnt, scr, tot);
  if (threadIdx.x == 0) s_excl[kGroup] = tot;
  __syncthreads();
  const size_t nbase = (size_t)p * D.cap;
  const size_t out = nbase + D.gbase[(size_t)p * D.MG + gidx];
  for (uint32_t i0 = threadIdx.x; i0 < tot; i0 += kGroup * kU) {
    uint32_t src[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t i = i0 + u * kGroup;
      src[u] = 0xFFFFFFFFu;
      if (i < tot) {
        uint32_t lo = 0, hi = kGroup;  // s_excl[lo] <= i < s_excl[hi]
        while (hi - lo > 1) {
          const uint32_t mid = (lo + hi) >> 1;
          if (s_excl[mid] <= i) lo = mid;
          else hi = mid;
        }
        src[u] = s_toff[lo] + (i - s_excl[lo]);
      }
    }
    uint64_t c[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) c[u] = src[u] != 0xFFFFFFFFu ? D.cand[nbase + src[u]] : 0ull;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool valid = src[u] != 0xFFFFFFFFu;
      const float v = __uint_as_float((uint32_t)c[u]);
      if (valid) {
        const uint32_t i = i0 + u * kGroup;
        D.oval[out + i] = v;
        D.oidx[out + i] = (uint32_t)(c[u] >> 32);
      }
      wave_hist_add(h, mag_key(v) >> 20, valid);
    }
  }
  __syncthreads();
  uint32_t* gh = D.h0 + (size_t)p * kH0;
  for (uint32_t i = threadIdx.x; i < kH0; i += kGroup)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Digits chosen so far, recomputed from the global histograms of the levels
// below `level` (each block does it; they all agree).
template <int NT>
__device__ __forceinline__ void decide(const Dev& D, uint32_t p, int level, uint32_t* scr,
                                       uint32_t& prefix, uint32_t& krem) {
  krem = D.k;
  prefix = 0;
  uint32_t bin, above;
  if (level >= 1) {
    block_find_suffix<NT>(D.h0 + (size_t)p * kH0, kH0, krem, scr, bin, above);
    krem -= above;
    prefix = bin;
  }
  if (level >= 2) {
    block_find_suffix<NT>(D.h1 + (size_t)p * kH1, kH1, krem, scr, bin, above);
    krem -= above;
    prefix = (prefix << 10) | bin;
  }
  if (level >= 3) {
    block_find_suffix<NT>(D.h2 + (size_t)p * kH2, kH2, krem, scr, bin, above);
    krem -= above;
    prefix = (prefix << 10) | bin;
  }
}

// ---------------------------------------------------------------------------
// hist: one radix level of T*. Level 0 runs only on the rescan path (the
// gather kernel builds it for the candidate path).
// ---------------------------------------------------------------------------
template <int LEVEL>
__global__ __launch_bounds__(256) void k_hist(const float* __restrict__ r, Dev D) {
  constexpr int NB = LEVEL == 0 ? kH0 : (LEVEL == 1 ? kH1 : kH2);
  constexpr int kU = 16;
  __shared__ uint32_t h[NB];
  __shared__ uint32_t scr[256 / kWave + 3];
  const uint32_t p = blockIdx.y;
  const bool rescan = D.state[p].mode != 0u;
  if (LEVEL == 0 && !rescan) return;
  for (uint32_t i = threadIdx.x; i < NB; i += 256) h[i] = 0u;
  uint32_t prefix, krem;
  decide<256>(D, p, LEVEL, scr, prefix, krem);
  __syncthreads();
  const uint64_t n = source_len(D, p, rescan);
  const float* src = rescan ? r + (uint64_t)p * D.N : D.oval + (size_t)p * D.cap;
  const uint64_t stride = (uint64_t)gridDim.x * 256 * kU;
  for (uint64_t i0 = (uint64_t)blockIdx.x * 256 * kU + threadIdx.x; i0 < n; i0 += stride) {
    uint32_t key[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint64_t i = i0 + (uint64_t)u * 256;
      key[u] = i < n ? mag_key(src[i]) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t kk = key[u];
      bool hit;
      uint32_t bin;
      if (LEVEL == 0) {
        hit = kk != 0xFFFFFFFFu;
        bin = kk >> 20;
      } else if (LEVEL == 1) {
        hit = kk != 0xFFFFFFFFu && (kk >> 20) == prefix;
        bin = (kk >> 10) & 1023u;
      } else {
        hit = kk != 0xFFFFFFFFu && (kk >> 10) == prefix;
        bin = kk & 1023u;
      }
      // level 0 keys crowd into a few bins: aggregate per wave; the lower
      // digits spread out, where plain LDS atomics are cheaper
      if (LEVEL == 0) {
        wave_hist_add(h, bin, hit);
      } else if (hit) {
        atomicAdd(&h[bin], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = (LEVEL == 0 ? D.h0 : (LEVEL == 1 ? D.h1 : D.h2)) + (size_t)p * NB;
  for (uint32_t i = threadIdx.x; i < NB; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ---------------------------------------------------------------------------
// count: per chunk of the source, elements above and equal to T*.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kChunkThreads) void k_count(const float* __restrict__ r, Dev D) {
  __shared__ uint32_t scr[kChunkThreads / kWave + 3];
  __shared__ uint32_t s_sum[2 * (kChunkThreads / kWave)];
  const uint32_t p = blockIdx.y;
  uint32_t T, m;
  decide<kChunkThreads>(D, p, 3, scr, T, m);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    D.state[p].T = T;
    D.state[p].m = m;
  }
  const bool rescan = D.state[p].mode != 0u;
  const uint64_t n = source_len(D, p, rescan);
  const uint64_t nchunks = (n + kChunk - 1) / kChunk;
  const float* src = rescan ? r + (uint64_t)p * D.N : D.oval + (size_t)p * D.cap;
  for (uint64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    uint32_t gt = 0, eq = 0;
    float v[kChunkIt];
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * kChunkThreads + threadIdx.x;
      v[it] = j < n ? src[j] : 0.0f;
    }
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * kChunkThreads + threadIdx.x;
      const uint32_t key = mag_key(v[it]);
      gt += (j < n && key > T) ? 1u : 0u;
      eq += (j < n && key == T) ? 1u : 0u;
    }
    uint32_t tgt, teq;
    block_sum2<kChunkThreads>(gt, eq, s_sum, tgt, teq);
    if (threadIdx.x == 0) {
      D.cgt[(size_t)p * D.MC + c] = tgt;
      D.ceq[(size_t)p * D.MC + c] = teq;
    }
  }
}

// ---------------------------------------------------------------------------
// scan: tie quota in index order, then each chunk's output offset.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_scan(Dev D) {
  __shared__ uint32_t scr[1024 / kWave + 3];
  const uint32_t p = blockIdx.x;
  const uint32_t m = D.state[p].m;
  const bool rescan = D.state[p].mode != 0u;
  const uint64_t n = source_len(D, p, rescan);
  const uint64_t nchunks = (n + kChunk - 1) / kChunk;
  uint32_t eq_carry = 0, out_carry = 0;
  for (uint64_t c0 = 0; c0 < nchunks; c0 += 1024) {
    const uint64_t c = c0 + threadIdx.x;
    const bool in = c < nchunks;
    const uint32_t gt = in ? D.cgt[(size_t)p * D.MC + c] : 0u;
    const uint32_t eq = in ? D.ceq[(size_t)p * D.MC + c] : 0u;
    uint32_t tot;
    const uint32_t eq_off = eq_carry + block_exclusive_scan<1024>(eq, scr, tot);
    eq_carry += tot;
    const uint32_t quota = eq_off >= m ? 0u : (m - eq_off < eq ? m - eq_off : eq);
    const uint32_t sel = gt + quota;
    const uint32_t out_off = out_carry + block_exclusive_scan<1024>(sel, scr, tot);
    out_carry += tot;
    if (in) {
      D.ceqoff[(size_t)p * D.MC + c] = eq_off;
      D.cout[(size_t)p * D.MC + c] = out_off;
    }
  }
  if (threadIdx.x == 0 && out_carry != D.k) D.err[p] = 1u;
}

// ---------------------------------------------------------------------------
// emit: selected pairs in index order; residual finished.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kChunkThreads) void k_emit(float* __restrict__ r, uint32_t* __restrict__ out_idx,
                                                        float* __restrict__ out_val, Dev D) {
  constexpr int NW = kChunkThreads / kWave;
  __shared__ uint32_t s_eq[kChunkIt * NW];
  __shared__ uint32_t s_sel[kChunkIt * NW];
  const uint32_t p = blockIdx.y;
  const bool rescan = D.state[p].mode != 0u;
  const uint32_t T = D.state[p].T;
  const uint32_t m = D.state[p].m;
  const uint32_t mid = D.state[p].mid;
  const uint32_t lane = lane_id();
  const uint32_t wid = threadIdx.x / kWave;
  const uint64_t n = source_len(D, p, rescan);
  const uint64_t nchunks = (n + kChunk - 1) / kChunk;
  const uint64_t pN = (uint64_t)p * D.N;
  const float* vsrc = rescan ? r + pN : D.oval + (size_t)p * D.cap;
  const uint32_t* isrc = D.oidx + (size_t)p * D.cap;
  uint32_t* oi = out_idx + (uint64_t)p * D.k;
  float* ov = out_val + (uint64_t)p * D.k;
  for (uint64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const uint32_t eq_base = D.ceqoff[(size_t)p * D.MC + c];
    const uint32_t out_base = D.cout[(size_t)p * D.MC + c];
    float v[kChunkIt];
    uint32_t e[kChunkIt];
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * kChunkThreads + threadIdx.x;
      const bool valid = j < n;
      v[it] = valid ? vsrc[j] : 0.0f;
      e[it] = valid ? (rescan ? (uint32_t)j : isrc[j]) : 0u;
    }
    // per (it, wave): ranks of equal keys, then of selected elements
    uint32_t eq_pre[kChunkIt];
    uint32_t eq_bits = 0;
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * kChunkThreads + threadIdx.x;
      const bool is_eq = j < n && mag_key(v[it]) == T;
      const uint64_t em = ballot(is_eq);
      eq_bits |= (is_eq ? 1u : 0u) << it;
      eq_pre[it] = lanes_below(em);
      if (lane == 0) s_eq[it * NW + wid] = popc64(em);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t run = 0;
      for (int i = 0; i < kChunkIt * NW; ++i) {
        const uint32_t x = s_eq[i];
        s_eq[i] = run;
        run += x;
      }
    }
    __syncthreads();
    uint32_t sel_bits = 0;
    uint32_t sel_pre[kChunkIt];
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * kChunkThreads + threadIdx.x;
      const uint32_t key = mag_key(v[it]);
      const bool is_eq = (eq_bits >> it) & 1u;
      const uint32_t eq_rank = eq_base + s_eq[it * NW + wid] + eq_pre[it];
      const bool sel = j < n && (key > T || (is_eq && eq_rank < m));
      sel_bits |= (sel ? 1u : 0u) << it;
      const uint64_t sm = ballot(sel);
      sel_pre[it] = lanes_below(sm);
      if (lane == 0) s_sel[it * NW + wid] = popc64(sm);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t run = 0;
      for (int i = 0; i < kChunkIt * NW; ++i) {
        const uint32_t x = s_sel[i];
        s_sel[i] = run;
        run += x;
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * kChunkThreads + threadIdx.x;
      if (j >= n) continue;
      const bool high = mag_key(v[it]) >= mid;  // written as +0 by the stream kernel
      if ((sel_bits >> it) & 1u) {
        const uint32_t pos = out_base + s_sel[it * NW + wid] + sel_pre[it];
        if (pos < D.k) {
          oi[pos] = e[it];
          ov[pos] = v[it];
        }
        if (rescan || !high) r[pN + e[it]] = 0.0f;
      } else if (!rescan && high) {
        r[pN + e[it]] = v[it];  // zeroed on the guess but not selected: restore
      }
    }
    __syncthreads();  // s_eq / s_sel are reused by the next chunk
  }
}

}  // namespace

size_t topk_workspace_bytes(uint32_t P, uint64_t N, uint64_t k) { return make_layout(P, N, k).total; }

hipError_t topk_ef_launch(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                          uint32_t* out_idx, float* out_val, void* ws, hipStream_t stream,
                          hipEvent_t ev_start, hipEvent_t ev_stop) {
  const Layout L = make_layout(P, N, k);
  char* w = static_cast<char*>(ws);
  Dev D;
  D.P = P;
  D.N = (uint32_t)N;
  D.k = (uint32_t)k;
  if (N <= (uint64_t)kSample) {
    D.rs_lo = D.rs_mid = (uint32_t)k;
  } else {
    const double qs = (double)k / (double)N * kSample;
    D.rs_lo = (uint32_t)std::min<double>(std::ceil(qs + 4.0 * std::sqrt(qs) + 16.0), (double)kSample);
    D.rs_mid = (uint32_t)std::min<double>(std::max<double>(1.0, std::ceil(qs)), (double)kSample);
  }
  D.pad = 0;
  D.capS = L.capS;
  D.cap = L.cap;
  D.MT = L.MT;
  D.MG = L.MG;
  D.MC = L.MC;
  D.info = reinterpret_cast<uint32_t*>(w + L.info);
  D.err = reinterpret_cast<uint32_t*>(w + L.err);
  D.state = reinterpret_cast<NodeState*>(w + L.state);
  D.h0 = reinterpret_cast<uint32_t*>(w + L.h0);
  D.h1 = reinterpret_cast<uint32_t*>(w + L.h1);
  D.h2 = reinterpret_cast<uint32_t*>(w + L.h2);
  D.sub = reinterpret_cast<uint32_t*>(w + L.sub);
  D.cand = reinterpret_cast<uint64_t*>(w + L.cand);
  D.oidx = reinterpret_cast<uint32_t*>(w + L.oidx);
  D.oval = reinterpret_cast<float*>(w + L.oval);
  D.tmeta = reinterpret_cast<uint64_t*>(w + L.tmeta);
  D.gsum = reinterpret_cast<uint32_t*>(w + L.gsum);
  D.gbase = reinterpret_cast<uint32_t*>(w + L.gbase);
  D.cgt = reinterpret_cast<uint32_t*>(w + L.cgt);
  D.ceq = reinterpret_cast<uint32_t*>(w + L.ceq);
  D.ceqoff = reinterpret_cast<uint32_t*>(w + L.ceqoff);
  D.cout = reinterpret_cast<uint32_t*>(w + L.cout);

  hipLaunchKernelGGL(k_predict, dim3(P), dim3(kPredictThreads), 0, stream, grad, residual, D);
  hipError_t e = hipSuccess;
  if (ev_start) e = hipEventRecord(ev_start, stream);
  hipLaunchKernelGGL(k_stream, dim3((uint32_t)(L.MT * P)), dim3(kStreamThreads), 0, stream, grad, residual, D);
  if (ev_stop && e == hipSuccess) e = hipEventRecord(ev_stop, stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess || k == 0) return e;

  // per-node block counts sized for the candidate list; the rescan path
  // loops over more work with the same grids
  const uint64_t per_node = std::max<uint64_t>(1, 8192 / P);
  const uint32_t groups = (uint32_t)L.MG;
  const uint32_t tile_blocks = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((L.MT + 255) / 256, per_node));
  // select / count / emit passes: enough blocks to fill the chip once, each
  // looping over several chunks, so the per-block digit decisions are amortised
  const uint64_t pass_node = std::max<uint64_t>(1, 2048 / P);
  const uint32_t hist_blocks =
      (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((L.cap + 16383) / 16384, pass_node));
  const uint32_t chunk_blocks =
      (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((L.cap + kChunk - 1) / kChunk, pass_node));
  hipLaunchKernelGGL(k_tsum, dim3(groups, P), dim3(256), 0, stream, D);
  hipLaunchKernelGGL(k_gscan, dim3(P), dim3(1024), 0, stream, D);
  hipLaunchKernelGGL(k_restore, dim3(tile_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_gather, dim3(groups, P), dim3(kGroup), 0, stream, D);
  hipLaunchKernelGGL(k_hist<0>, dim3(hist_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_hist<1>, dim3(hist_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_hist<2>, dim3(hist_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_count, dim3(chunk_blocks, P), dim3(kChunkThreads), 0, stream, residual, D);
  hipLaunchKernelGGL(k_scan, dim3(P), dim3(1024), 0, stream, D);
  hipLaunchKernelGGL(k_emit, dim3(chunk_blocks, P), dim3(kChunkThreads), 0, stream, residual, out_idx, out_val,
                     D);
  return hipGetLastError();
}

}  // namespace sparcml
