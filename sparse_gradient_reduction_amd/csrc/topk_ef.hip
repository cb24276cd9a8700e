// Error-feedback Top-k for gfx950.
//
// SparCML (paperlayer.ai digest of arXiv 1802.08021v3), section 2.2: each
// node sends its k largest-magnitude components and accumulates the rest for
// the next iteration; section 4: the unapplied part is the residual error.
//
// Exact selection, HBM-streaming design. The method's work is one pass over
// grad and residual (read 8 B, write 4 B per element); everything else works
// on a small candidate set:
//
//   predict  one block per node reads a stratified sample (512 chunks of 64
//            elements) of a = grad + residual, and picks a key threshold
//            `pred` that the k-th largest key exceeds with high probability
//            (exactly, when the sample is the whole node).
//   stream   one pass per 8192-element tile: a = grad + residual; elements
//            with key >= pred are compacted in index order (wave ballots and
//            prefix counts) into a per-node candidate list, one run per tile
//            reserved with one atomic; residual is written back as a, with
//            stored candidates written as +0.
//   restore  only for a node whose candidate count is below k or above the
//            list capacity: put the stored candidates back into residual, so
//            that the exact rescan below can read a from residual.
//   hist x3  radix select of the k-th largest key over the candidates (or
//            the whole residual on the rescan path): LDS histograms of key
//            bits 30..20, 19..10 and 9..0; each level's digit is chosen from
//            the previous histogram inside the next kernel.
//   count    per tile: candidates with key > T* and key == T*.
//   scan     per node: tie quota m goes to the lowest indices; output offset
//            of each tile.
//   emit     per tile, in index order: selected candidates go to the output;
//            unselected candidates are restored in residual (rescan path:
//            selected positions are zeroed instead).
//
// Every element with key >= T* is a candidate whenever count >= k, so both
// paths give the same, exact result; the sample only decides how much work
// the candidate set costs.
#include "device_common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <cmath>

namespace sparcml {
namespace {

constexpr int kTileGroups = 2048;                // float4 groups per tile
constexpr int kTile = 4 * kTileGroups;           // 8192 elements per tile
constexpr int kStreamThreads = 256;
constexpr int kGPT = kTileGroups / kStreamThreads;  // 8 groups per thread
constexpr int kSampleChunks = 512;
constexpr int kSampleChunk = 64;
constexpr int kSample = kSampleChunks * kSampleChunk;  // 32768
constexpr int kPredictThreads = 1024;
constexpr int kH0 = 2048, kH1 = 1024, kH2 = 1024;  // radix digits: 11 + 10 + 10 bits

struct NodeState {
  uint32_t pred;   // candidate threshold on the key
  uint32_t count;  // candidates reserved by the stream kernel (may exceed cap)
  uint32_t mode;   // 0 candidates, 1 exact rescan
  uint32_t T;      // k-th largest key
  uint32_t m;      // how many elements with key == T are selected
  uint32_t pad[3];
};

struct Layout {
  uint64_t cap;  // candidate list capacity per node
  uint64_t MT;   // tile slots per node
  size_t info, err, state, h0, h1, h2, cidx, cval, toff, tcnt, tgt, teq, teqoff, tout, total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout make_layout(uint32_t P, uint64_t N, uint64_t k) {
  Layout L{};
  L.cap = std::min<uint64_t>(N, 2 * k + 65536);
  L.MT = (N + 3 + kTile - 1) / kTile;
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
  L.cidx = take(4ull * P * L.cap);
  L.cval = take(4ull * P * L.cap);
  L.toff = take(4ull * P * L.MT);
  L.tcnt = take(4ull * P * L.MT);
  L.tgt = take(4ull * P * L.MT);
  L.teq = take(4ull * P * L.MT);
  L.teqoff = take(4ull * P * L.MT);
  L.tout = take(4ull * P * L.MT);
  L.total = o;
  return L;
}

struct Dev {
  uint32_t P;
  uint32_t N;
  uint32_t k;
  uint32_t rs;  // sample rank that sets the threshold
  uint64_t cap;
  uint64_t MT;
  uint32_t* info;
  uint32_t* err;
  NodeState* state;
  uint32_t* h0;
  uint32_t* h1;
  uint32_t* h2;
  uint32_t* cidx;
  float* cval;
  uint32_t* toff;
  uint32_t* tcnt;
  uint32_t* tgt;
  uint32_t* teq;
  uint32_t* teqoff;
  uint32_t* tout;
};

__device__ __forceinline__ uint32_t node_tiles(const Dev& D, uint32_t p) {
  const uint32_t phi = (uint32_t)(((uint64_t)p * D.N) & 3u);
  return (uint32_t)(((uint64_t)D.N + phi + kTile - 1) / kTile);
}

// node-local element range [lo, hi) of tile t of node p
__device__ __forceinline__ void tile_range(const Dev& D, uint32_t p, uint32_t t, uint32_t& lo, uint32_t& hi) {
  const int64_t phi = (int64_t)(((uint64_t)p * D.N) & 3u);
  int64_t a = (int64_t)t * kTile - phi;
  int64_t b = a + kTile;
  lo = (uint32_t)(a < 0 ? 0 : a);
  hi = (uint32_t)(b > (int64_t)D.N ? (int64_t)D.N : b);
}

__device__ __forceinline__ bool needs_rescan(const Dev& D, uint32_t p) {
  const uint32_t c = D.state[p].count;
  return c < D.k || (uint64_t)c > D.cap;
}

// ---------------------------------------------------------------------------
// predict: reset the node's select state and choose the candidate threshold.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPredictThreads) void k_predict(const float* __restrict__ g,
                                                             const float* __restrict__ r, Dev D) {
  __shared__ uint32_t h1[4096];
  __shared__ uint32_t h2[2048];
  __shared__ uint32_t scr[kPredictThreads / kWave + 3];
  const uint32_t p = blockIdx.x;
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < kH0; i += kPredictThreads) D.h0[(size_t)p * kH0 + i] = 0u;
  for (uint32_t i = tid; i < kH1; i += kPredictThreads) D.h1[(size_t)p * kH1 + i] = 0u;
  for (uint32_t i = tid; i < kH2; i += kPredictThreads) D.h2[(size_t)p * kH2 + i] = 0u;
  for (uint32_t i = tid; i < 4096; i += kPredictThreads) h1[i] = 0u;
  for (uint32_t i = tid; i < 2048; i += kPredictThreads) h2[i] = 0u;

  uint32_t pred;
  if (D.k == 0) {
    pred = 0xFFFFFFFFu;  // keys are < 2^31: no candidate
  } else if (D.k == D.N) {
    pred = 0u;  // everything is selected
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
      if (key != 0xFFFFFFFFu) atomicAdd(&h1[key >> 19], 1u);
    }
    __syncthreads();
    uint32_t b1, above1;
    block_find_suffix<kPredictThreads>(h1, 4096, D.rs, scr, b1, above1);
    const uint32_t rank2 = D.rs - above1;
#pragma unroll
    for (int j = 0; j < kSample / kPredictThreads; ++j) {
      const uint32_t key = keys[j];
      if (key != 0xFFFFFFFFu && (key >> 19) == b1) atomicAdd(&h2[(key >> 8) & 2047u], 1u);
    }
    __syncthreads();
    uint32_t b2, above2;
    block_find_suffix<kPredictThreads>(h2, 2048, rank2, scr, b2, above2);
    pred = (b1 << 19) | (b2 << 8);
  }
  if (tid == 0) {
    NodeState s{};
    s.pred = pred;
    s.count = 0;
    s.mode = 0;
    D.state[p] = s;
    D.err[p] = 0u;
    D.info[p] = 0u;
  }
}

// ---------------------------------------------------------------------------
// stream: a = g + r, candidate compaction in index order, residual write-back.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kStreamThreads) void k_stream(const float* __restrict__ g,
                                                           float* __restrict__ r, Dev D) {
  __shared__ uint32_t s_cnt[kGPT * (kStreamThreads / kWave)];
  __shared__ uint32_t s_base;
  __shared__ uint32_t s_stored;
  const uint32_t p = blockIdx.y;
  const uint32_t t = blockIdx.x;
  if (t >= node_tiles(D, p)) return;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = lane_id();
  const uint32_t wid = tid / kWave;
  const uint32_t N = D.N;
  const uint64_t pN = (uint64_t)p * N;
  const int64_t ebase = (int64_t)t * kTile - (int64_t)(pN & 3u);  // node-local index of the tile start
  const uint64_t gbase = (pN >> 2) + (uint64_t)t * kTileGroups;  // float4 group of the tile start
  const uint32_t pred = D.state[p].pred;
  const bool interior = ebase >= 0 && ebase + kTile <= (int64_t)N;

  float a[kGPT][4];
  uint32_t own = 0xFFFFFFFFu;  // bit j*4+c: element belongs to node p
  if (interior) {
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g) + gbase;
    const f32x4* r4 = reinterpret_cast<const f32x4*>(r) + gbase;
    f32x4 gv[kGPT], rv[kGPT];
#pragma unroll
    for (int j = 0; j < kGPT; ++j) gv[j] = load_nt(g4 + j * kStreamThreads + tid);
#pragma unroll
    for (int j = 0; j < kGPT; ++j) rv[j] = load_nt(r4 + j * kStreamThreads + tid);
#pragma unroll
    for (int j = 0; j < kGPT; ++j) {
      a[j][0] = gv[j].x + rv[j].x;
      a[j][1] = gv[j].y + rv[j].y;
      a[j][2] = gv[j].z + rv[j].z;
      a[j][3] = gv[j].w + rv[j].w;
    }
  } else {
    own = 0u;
#pragma unroll
    for (int j = 0; j < kGPT; ++j) {
      const int64_t e0 = ebase + 4 * (int64_t)(j * kStreamThreads + tid);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t e = e0 + c;
        a[j][c] = 0.0f;
        if (e >= 0 && e < (int64_t)N) {
          a[j][c] = g[pN + (uint64_t)e] + r[pN + (uint64_t)e];
          own |= 1u << (j * 4 + c);
        }
      }
    }
  }

  uint32_t flags = 0;  // bit j*4+c: candidate
#pragma unroll
  for (int j = 0; j < kGPT; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (((own >> (j * 4 + c)) & 1u) && mag_key(a[j][c]) >= pred) flags |= 1u << (j * 4 + c);

  // Index order inside the tile is (j, wave, lane, c). Per j: lane prefix from
  // four ballots, wave totals into LDS.
  uint32_t lane_pre[kGPT];
#pragma unroll
  for (int j = 0; j < kGPT; ++j) {
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t m = ballot((flags >> (j * 4 + c)) & 1u);
      pre += lanes_below(m);
      tot += popc64(m);
    }
    lane_pre[j] = pre;
    if (lane == 0) s_cnt[j * (kStreamThreads / kWave) + wid] = tot;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int i = 0; i < kGPT * (kStreamThreads / kWave); ++i) {
      uint32_t c = s_cnt[i];
      s_cnt[i] = run;
      run += c;
    }
    uint32_t base = run ? atomicAdd(&D.state[p].count, run) : 0u;
    D.toff[(size_t)p * D.MT + t] = base;
    D.tcnt[(size_t)p * D.MT + t] = run;
    s_base = base;
    s_stored = ((uint64_t)base + run <= D.cap) ? 1u : 0u;
  }
  __syncthreads();
  const uint32_t base = s_base;
  const bool stored = s_stored != 0u;

  if (stored && flags) {
    uint32_t* ci = D.cidx + (size_t)p * D.cap;
    float* cv = D.cval + (size_t)p * D.cap;
#pragma unroll
    for (int j = 0; j < kGPT; ++j) {
      uint32_t pos = base + s_cnt[j * (kStreamThreads / kWave) + wid] + lane_pre[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((flags >> (j * 4 + c)) & 1u) {
          const int64_t e = ebase + 4 * (int64_t)(j * kStreamThreads + tid) + c;
          ci[pos] = (uint32_t)e;
          cv[pos] = a[j][c];
          ++pos;
        }
      }
    }
  }

  const uint32_t zero_mask = stored ? flags : 0u;
  if (interior) {
    f32x4* r4 = reinterpret_cast<f32x4*>(r) + gbase;
#pragma unroll
    for (int j = 0; j < kGPT; ++j) {
      f32x4 o;
      o.x = ((zero_mask >> (j * 4 + 0)) & 1u) ? 0.0f : a[j][0];
      o.y = ((zero_mask >> (j * 4 + 1)) & 1u) ? 0.0f : a[j][1];
      o.z = ((zero_mask >> (j * 4 + 2)) & 1u) ? 0.0f : a[j][2];
      o.w = ((zero_mask >> (j * 4 + 3)) & 1u) ? 0.0f : a[j][3];
      store_nt(o, r4 + j * kStreamThreads + tid);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kGPT; ++j) {
      const int64_t e0 = ebase + 4 * (int64_t)(j * kStreamThreads + tid);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((own >> (j * 4 + c)) & 1u)
          r[pN + (uint64_t)(e0 + c)] = ((zero_mask >> (j * 4 + c)) & 1u) ? 0.0f : a[j][c];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// restore: rescan path only - stored candidates go back into residual.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_restore(float* __restrict__ r, Dev D) {
  const uint32_t p = blockIdx.y;
  const bool rescan = needs_rescan(D, p);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    D.state[p].mode = rescan ? 1u : 0u;
    D.info[p] = rescan ? 1u : 0u;
  }
  if (!rescan) return;
  const uint32_t lane = lane_id();
  const uint32_t wid = threadIdx.x / kWave;
  const uint32_t nt = node_tiles(D, p);
  const uint64_t pN = (uint64_t)p * D.N;
  for (uint32_t t = blockIdx.x * 4 + wid; t < nt; t += gridDim.x * 4) {
    const uint32_t off = D.toff[(size_t)p * D.MT + t];
    const uint32_t cnt = D.tcnt[(size_t)p * D.MT + t];
    if ((uint64_t)off + cnt > D.cap) continue;  // this tile stored nothing
    for (uint32_t j = lane; j < cnt; j += kWave) {
      const uint32_t e = D.cidx[(size_t)p * D.cap + off + j];
      r[pN + e] = D.cval[(size_t)p * D.cap + off + j];
    }
  }
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
// hist: one radix level of the k-th largest key.
// ---------------------------------------------------------------------------
template <int LEVEL>
__global__ __launch_bounds__(256) void k_hist(const float* __restrict__ r, Dev D) {
  constexpr int NB = LEVEL == 0 ? kH0 : (LEVEL == 1 ? kH1 : kH2);
  __shared__ uint32_t h[NB];
  __shared__ uint32_t scr[256 / kWave + 3];
  const uint32_t p = blockIdx.y;
  for (uint32_t i = threadIdx.x; i < NB; i += 256) h[i] = 0u;
  uint32_t prefix, krem;
  decide<256>(D, p, LEVEL, scr, prefix, krem);
  __syncthreads();
  const bool rescan = D.state[p].mode != 0u;
  const uint64_t n = rescan ? (uint64_t)D.N : (uint64_t)D.state[p].count;
  const float* src = rescan ? r + (uint64_t)p * D.N : D.cval + (size_t)p * D.cap;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256) {
    const uint32_t key = mag_key(src[i]);
    if (LEVEL == 0) {
      atomicAdd(&h[key >> 20], 1u);
    } else if (LEVEL == 1) {
      if ((key >> 20) == prefix) atomicAdd(&h[(key >> 10) & 1023u], 1u);
    } else {
      if ((key >> 10) == prefix) atomicAdd(&h[key & 1023u], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = (LEVEL == 0 ? D.h0 : (LEVEL == 1 ? D.h1 : D.h2)) + (size_t)p * NB;
  for (uint32_t i = threadIdx.x; i < NB; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ---------------------------------------------------------------------------
// count: per tile, candidates above and equal to the k-th largest key.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_count(const float* __restrict__ r, Dev D) {
  __shared__ uint32_t scr[256 / kWave + 3];
  const uint32_t p = blockIdx.y;
  uint32_t T, m;
  decide<256>(D, p, 3, scr, T, m);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    D.state[p].T = T;
    D.state[p].m = m;
  }
  const bool rescan = D.state[p].mode != 0u;
  const uint32_t lane = lane_id();
  const uint32_t wid = threadIdx.x / kWave;
  const uint32_t nt = node_tiles(D, p);
  for (uint32_t t = blockIdx.x * 4 + wid; t < (uint32_t)D.MT; t += gridDim.x * 4) {
    uint32_t gt = 0, eq = 0;
    if (t < nt) {
      const float* src;
      uint32_t cnt;
      if (rescan) {
        uint32_t lo, hi;
        tile_range(D, p, t, lo, hi);
        src = r + (uint64_t)p * D.N + lo;
        cnt = hi - lo;
      } else {
        src = D.cval + (size_t)p * D.cap + D.toff[(size_t)p * D.MT + t];
        cnt = D.tcnt[(size_t)p * D.MT + t];
      }
      for (uint32_t j = lane; j < cnt; j += kWave) {
        const uint32_t key = mag_key(src[j]);
        gt += key > T;
        eq += key == T;
      }
      gt = wave_sum(gt);
      eq = wave_sum(eq);
    }
    if (lane == 0) {
      D.tgt[(size_t)p * D.MT + t] = gt;
      D.teq[(size_t)p * D.MT + t] = eq;
    }
  }
}

// ---------------------------------------------------------------------------
// scan: tie quota in index order, then each tile's output offset.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_scan(Dev D) {
  __shared__ uint32_t scr[1024 / kWave + 3];
  const uint32_t p = blockIdx.x;
  const uint32_t m = D.state[p].m;
  uint32_t eq_carry = 0, out_carry = 0;
  for (uint64_t t0 = 0; t0 < D.MT; t0 += 1024) {
    const uint64_t t = t0 + threadIdx.x;
    const bool in = t < D.MT;
    const uint32_t gt = in ? D.tgt[(size_t)p * D.MT + t] : 0u;
    const uint32_t eq = in ? D.teq[(size_t)p * D.MT + t] : 0u;
    uint32_t tot;
    const uint32_t eq_off = eq_carry + block_exclusive_scan<1024>(eq, scr, tot);
    eq_carry += tot;
    const uint32_t quota = eq_off >= m ? 0u : (m - eq_off < eq ? m - eq_off : eq);
    const uint32_t sel = gt + quota;
    const uint32_t out_off = out_carry + block_exclusive_scan<1024>(sel, scr, tot);
    out_carry += tot;
    if (in) {
      D.teqoff[(size_t)p * D.MT + t] = eq_off;
      D.tout[(size_t)p * D.MT + t] = out_off;
    }
  }
  if (threadIdx.x == 0 && out_carry != D.k) D.err[p] = 1u;
}

// ---------------------------------------------------------------------------
// emit: selected pairs in index order; residual finished.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_emit(float* __restrict__ r, uint32_t* __restrict__ out_idx,
                                              float* __restrict__ out_val, Dev D) {
  const uint32_t p = blockIdx.y;
  const bool rescan = D.state[p].mode != 0u;
  const uint32_t T = D.state[p].T;
  const uint32_t m = D.state[p].m;
  const uint32_t lane = lane_id();
  const uint32_t wid = threadIdx.x / kWave;
  const uint32_t nt = node_tiles(D, p);
  const uint64_t pN = (uint64_t)p * D.N;
  uint32_t* oi = out_idx + (uint64_t)p * D.k;
  float* ov = out_val + (uint64_t)p * D.k;
  for (uint32_t t = blockIdx.x * 4 + wid; t < nt; t += gridDim.x * 4) {
    const size_t ti = (size_t)p * D.MT + t;
    uint32_t eq_seen = D.teqoff[ti];
    uint32_t out_pos = D.tout[ti];
    uint32_t lo = 0, cnt;
    const float* vsrc;
    const uint32_t* isrc = nullptr;
    if (rescan) {
      uint32_t hi;
      tile_range(D, p, t, lo, hi);
      cnt = hi - lo;
      vsrc = r + pN + lo;
    } else {
      const uint32_t off = D.toff[ti];
      cnt = D.tcnt[ti];
      vsrc = D.cval + (size_t)p * D.cap + off;
      isrc = D.cidx + (size_t)p * D.cap + off;
    }
    for (uint32_t j0 = 0; j0 < cnt; j0 += kWave) {
      const uint32_t j = j0 + lane;
      const bool valid = j < cnt;
      const float v = valid ? vsrc[j] : 0.0f;
      const uint32_t e = valid ? (rescan ? lo + j : isrc[j]) : 0u;
      const uint32_t key = mag_key(v);
      const bool is_eq = valid && key == T;
      const uint64_t eq_mask = ballot(is_eq);
      const uint32_t eq_rank = eq_seen + lanes_below(eq_mask);
      const bool sel = valid && (key > T || (is_eq && eq_rank < m));
      const uint64_t sel_mask = ballot(sel);
      if (sel) {
        const uint32_t pos = out_pos + lanes_below(sel_mask);
        if (pos < D.k) {
          oi[pos] = e;
          ov[pos] = v;
        }
        if (rescan) r[pN + e] = 0.0f;
      } else if (valid && !rescan) {
        r[pN + e] = v;  // candidate that was not selected: back into the residual
      }
      eq_seen += popc64(eq_mask);
      out_pos += popc64(sel_mask);
    }
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
    D.rs = (uint32_t)k;
  } else {
    const double qs = (double)k / (double)N * kSample;
    double rs = std::ceil(qs + 4.0 * std::sqrt(qs) + 16.0);
    D.rs = (uint32_t)std::min<double>(rs, (double)kSample);
  }
  D.cap = L.cap;
  D.MT = L.MT;
  D.info = reinterpret_cast<uint32_t*>(w + L.info);
  D.err = reinterpret_cast<uint32_t*>(w + L.err);
  D.state = reinterpret_cast<NodeState*>(w + L.state);
  D.h0 = reinterpret_cast<uint32_t*>(w + L.h0);
  D.h1 = reinterpret_cast<uint32_t*>(w + L.h1);
  D.h2 = reinterpret_cast<uint32_t*>(w + L.h2);
  D.cidx = reinterpret_cast<uint32_t*>(w + L.cidx);
  D.cval = reinterpret_cast<float*>(w + L.cval);
  D.toff = reinterpret_cast<uint32_t*>(w + L.toff);
  D.tcnt = reinterpret_cast<uint32_t*>(w + L.tcnt);
  D.tgt = reinterpret_cast<uint32_t*>(w + L.tgt);
  D.teq = reinterpret_cast<uint32_t*>(w + L.teq);
  D.teqoff = reinterpret_cast<uint32_t*>(w + L.teqoff);
  D.tout = reinterpret_cast<uint32_t*>(w + L.tout);

  hipLaunchKernelGGL(k_predict, dim3(P), dim3(kPredictThreads), 0, stream, grad, residual, D);
  hipError_t e = hipSuccess;
  if (ev_start) e = hipEventRecord(ev_start, stream);
  hipLaunchKernelGGL(k_stream, dim3((uint32_t)L.MT, P), dim3(kStreamThreads), 0, stream, grad, residual, D);
  if (ev_stop && e == hipSuccess) e = hipEventRecord(ev_stop, stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess || k == 0) return e;

  // tile loops: a wave per tile, enough blocks to fill the chip
  const uint32_t tile_blocks =
      (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((L.MT + 3) / 4, std::max<uint64_t>(1, 4096 / P)));
  const uint32_t hist_blocks =
      (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((L.cap + 4095) / 4096, std::max<uint64_t>(8, 8192 / P)));
  hipLaunchKernelGGL(k_restore, dim3(tile_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_hist<0>, dim3(hist_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_hist<1>, dim3(hist_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_hist<2>, dim3(hist_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_count, dim3(tile_blocks, P), dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_scan, dim3(P), dim3(1024), 0, stream, D);
  hipLaunchKernelGGL(k_emit, dim3(tile_blocks, P), dim3(256), 0, stream, residual, out_idx, out_val, D);
  return hipGetLastError();
}

}  // namespace sparcml
