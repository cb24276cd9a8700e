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
//   tsum     candidate counts summed per group of 512 tiles.
//   gscan    per node: group offsets, candidate count, and the path: the
//            candidate list when every tile was stored and it holds >= k
//            candidates, else an exact rescan of the whole node.
//   gather   candidate runs copied into index order; LDS histogram of key
//            bits 30..20 (first radix level) on the way. On the rescan path
//            it puts the zeroed candidates back into residual instead.
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
// A selection row is either a node's whole vector (the [P][N] call) or one
// layer of one node (the per-layer call); every kernel is templated on which,
// the first computing a row's geometry from (P, N, k), the second reading it
// from a per-row table, with a tile-to-row table for the stream kernel.
//
// Every element with key >= T* is a candidate whenever the list holds at
// least k of them, so both paths give the same exact result; the sample only
// decides how much the candidate work costs.
#include "device_common.hpp"
#include "kernels.hpp"
#include "sparcml.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <cmath>

namespace sparcml {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kTile = 4 * kStreamThreads;                 // 1024 elements per tile, one float4 per thread
// A row's tiles start at the 128-byte line holding its first element, so a
// row not aligned to a line shares lines with its neighbours only at its two
// ends, not at every tile boundary.
constexpr uint32_t kTileAlign = 32;
__host__ __device__ inline uint32_t tile_phase(uint64_t base) { return (uint32_t)(base & (kTileAlign - 1)); }
constexpr int kNW = kStreamThreads / kWave;               // waves per stream block
constexpr int kSub = 256;                                 // reservation counters per node
constexpr int kTilesPerSlotLog = 4;
constexpr int kTilesPerSlot = 1 << kTilesPerSlotLog;      // per-layer call: consecutive tiles sharing a counter
constexpr int kNodeTilesPerSlotLog = 2;                   // whole-node call: 4 consecutive tiles per counter
constexpr int kSampleChunks = 1024;
constexpr int kSampleChunk = 64;
constexpr int kSample = kSampleChunks * kSampleChunk;     // 65536
constexpr int kPredictThreads = 1024;
constexpr int kPredictKeys = 64;                            // sample keys per predict thread (registers)
constexpr int kSmallPredictThreads = 256;
constexpr int kSmallSample = kSmallPredictThreads * kPredictKeys;  // 16384
// per-layer call: the largest sample a row gets (512 chunks), held by
// 512-thread blocks, two of which fit a compute unit at once
constexpr int kLayerPredictThreads = 512;
constexpr int kLayerSampleChunks = kLayerPredictThreads * kPredictKeys / kSampleChunk;  // 512
constexpr int kH0 = 2048, kH1 = 1024, kH2 = 1024;         // radix digits: 11 + 10 + 10 bits
constexpr int kDigCap = 32;  // last-digit slots per chunk for the keys that share T*'s upper 21 bits
constexpr uint32_t kEqCounted = 1u << 31;  // ceq word: the count pass counted this chunk (past its digit slots)
// Whole-node call: the gather also counts the second digit of the keys whose
// first digit is one of kSpecBins bins around the prediction `mid`'s; when
// T*'s first digit is among them, that count is the second radix level and
// its pass over the candidates is skipped (the per-layer call, with many
// rows, keeps the pass rather than 12 KB more workspace per row).
constexpr uint32_t kSpecBins = 3;
constexpr int kGroup = 512;                              // tiles per gather group
constexpr int kChunkThreads = 256;
constexpr int kChunkIt = 16;
constexpr int kChunk = kChunkThreads * kChunkIt;          // 4096 candidates per chunk
// The emit pass holds 8 candidates of a chunk per thread (512 threads): with
// 16 (256 threads) it needed 107 VGPRs (4 waves per SIMD), and 161 when it
// also writes the run table (3 waves); with 8, 92 (5 waves), and the table
// then costs nothing measurable.
constexpr int kEmitIt = 8;
constexpr uint32_t kNotStored = 0xFFFFFFFFu;
constexpr uint32_t kSmallLayer = 16384;
constexpr int kSegmentBits = 12;  // run tables: segments of 4096 indices
static_assert((1u << kSegmentBits) == SPARCML_SEGMENT, "run table segment");  // per-layer call: rows this small skip the sampled prediction

struct NodeState {
  uint32_t lo;      // candidate threshold on the key
  uint32_t mid;     // zeroing threshold on the key (estimate of T*)
  uint32_t count;   // candidates of the node
  uint32_t fail;    // some tile did not fit its counter's region
  uint32_t mode;    // 0 candidates, 1 exact rescan
  uint32_t T;       // k-th largest key
  uint32_t m;       // how many elements with key == T are selected
  uint32_t ovf;     // some chunk holds more keys of T*'s 21-bit prefix than its digit slots
};

// Sizes of one row's slices of the workspace arrays (integer formulas shared
// by the host, which sizes the workspace and the grids, and the device, which
// lays out the per-layer row table).
struct RowSize {
  uint64_t nt;      // tiles (stream workgroups)
  uint64_t groups;  // groups of kGroup tiles
  uint64_t chunks;  // chunk slots (rescan worst case)
  uint64_t capS;    // candidate slots per counter region
  uint32_t nsub;    // counter regions
  uint32_t schunks; // sample chunks
  uint32_t npass;   // blocks of the select / count / emit grids
  uint32_t tps_log; // log2 of the consecutive tiles sharing a counter
};
constexpr size_t kRowBytes = 12 * sizeof(uint64_t);

// A whole node: kSub regions with a whole tile of slack each, fed by runs of
// 4 consecutive tiles dealt to the counters in turn (a node of at most
// kSub * kTilesPerSlot tiles deals single tiles), so that candidates crowded in
// one stretch of the node (a layer of larger gradients) spread over many
// regions: with runs of 16 tiles a 2^20-element stretch at 100 times the
// scale fed 64 regions, overflowed them and forced the exact rescan. A layer: as many regions as it
// has runs of kTilesPerSlot tiles (at most kSub), with the slack of its
// largest possible run. Where every element is a candidate (k =
// n, or a layer small enough to skip the prediction), a region takes whole
// slot groups of tiles, and regions may hold one group more than others: each
// holds the most groups any region gets.
__host__ __device__ inline RowSize row_size(uint64_t base, uint64_t n, uint64_t k, bool layer) {
  RowSize z;
  z.nt = (n + tile_phase(base) + kTile - 1) / kTile;
  z.groups = (z.nt + kGroup - 1) / kGroup;
  z.chunks = (n + kChunk - 1) / kChunk;
  if (z.chunks == 0) z.chunks = 1;
  const uint64_t want = n < 2 * k + 65536 ? n : 2 * k + 65536;
  z.tps_log = kTilesPerSlotLog;
  if (!layer) {
    z.nsub = kSub;
    z.tps_log = z.nt <= (uint64_t)kSub * kTilesPerSlot ? 0 : kNodeTilesPerSlotLog;
    z.capS = (want + kSub - 1) / kSub + kTile;
    z.schunks = kSampleChunks;
    z.npass = 0;
  } else {
    uint64_t ns = (z.nt + kTilesPerSlot - 1) / kTilesPerSlot;
    ns = ns < 1 ? 1 : (ns > (uint64_t)kSub ? (uint64_t)kSub : ns);
    z.nsub = (uint32_t)ns;
    z.capS = (want + ns - 1) / ns + (n < (uint64_t)kTile ? n : (uint64_t)kTile);
    // a sample of about one element in 64 (16 to 512 chunks): the wider
    // margin of a small sample costs little, as a layer's candidate list is
    // short next to its stream pass
    uint64_t sc = n / (64 * kSampleChunk);
    z.schunks = (uint32_t)(sc < 16 ? 16 : (sc > (uint64_t)kLayerSampleChunks ? (uint64_t)kLayerSampleChunks : sc));
    // select / count / emit blocks: one per 8192 expected candidates, 1..64
    const uint64_t est = n < 2 * k + 4096 ? n : 2 * k + 4096;
    uint64_t np = (est + 8191) / 8192;
    z.npass = (uint32_t)(np < 1 ? 1 : (np > 64 ? 64 : np));
  }
  if (k >= n || (layer && n <= kSmallLayer)) {
    const uint64_t tps = 1ull << z.tps_log;
    const uint64_t slots = (z.nt + tps - 1) / tps;
    const uint64_t most = (slots + z.nsub - 1) / z.nsub * tps * kTile;
    const uint64_t need = ((most < n ? most : n) + 3) / 4 * 4;
    // (candidate slots are 32-bit: where the total would not fit, such a row
    // takes the exact rescan path instead)
    if (need > z.capS && (uint64_t)z.nsub * need < (1ull << 32) - (1ull << 18)) z.capS = need;
  }
  return z;
}

// Per-layer call: rows whose thresholds come from a sample (the others keep
// no candidate, keep everything, or are small enough to be their own
// candidate list), and among them those whose sample exceeds what a
// 256-thread predict block holds, which get 512-thread blocks.
__host__ __device__ inline bool layer_sampled(uint64_t n, uint64_t k) { return k != 0 && k != n && n > kSmallLayer; }
__host__ __device__ inline bool big_predict(uint64_t n, uint64_t k, uint32_t schunks) {
  return layer_sampled(n, k) && (uint64_t)schunks * kSampleChunk > (uint64_t)kSmallSample;
}

// Totals over the rows: what the workspace holds.
struct Plan {
  uint64_t rows;
  uint64_t cand;    // candidate slots
  uint64_t tiles;   // tile words
  uint64_t groups;  // group words
  uint64_t chunks;  // chunk words
  uint64_t passes;  // per-layer call: select / count / emit blocks
  uint64_t big;     // per-layer call: rows with big_predict
  uint64_t mid;     // per-layer call: sampled rows without big_predict
  bool layers;      // per-layer call: row table and block-to-row tables too
};

struct Layout {
  uint64_t capS;  // whole-node call: candidate slots per counter region
  uint64_t cap;   // whole-node call: candidate slots per node (kSub * capS)
  uint32_t tps_log;  // whole-node call: log2 of the consecutive tiles sharing a counter
  uint64_t MT;    // whole-node call: tiles per node (slots)
  uint64_t MG;    // whole-node call: tile groups per node
  uint64_t MC;    // whole-node call: chunks per node (slots, rescan worst case)
  size_t info, err, state, h0, h1, h2, h1s, sub, cand, oidx, oval, tmeta, gsum, gbase, cgt, ceq, ceqoff,
      cout, cdig, rows, tile_row, group_row, pass_row, big_rows, mid_rows, loff, lk, lkoff, total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout make_layout(const Plan& Q, uint64_t nlayers) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  const uint64_t R = Q.rows;
  L.info = take(8ull * R);  // [rows] path per row, then [rows] consistency flags
  L.err = L.info + 4ull * R;
  L.state = take(sizeof(NodeState) * R);
  L.h0 = take(4ull * R * kH0);
  L.h1 = take(4ull * R * kH1);
  L.h2 = take(4ull * R * kH2);
  L.h1s = take(Q.layers ? 0 : 4ull * R * kSpecBins * kH1);
  L.sub = take(128ull * R * kSub);  // one counter per 128-byte line
  L.cand = take(8ull * Q.cand);
  L.oidx = take(4ull * Q.cand);
  L.oval = take(4ull * Q.cand);
  L.tmeta = take(8ull * Q.tiles);
  L.gsum = take(4ull * Q.groups);
  L.gbase = take(4ull * Q.groups);
  L.cgt = take(4ull * Q.chunks);
  L.ceq = take(4ull * Q.chunks);
  L.ceqoff = take(4ull * Q.chunks);
  L.cout = take(4ull * Q.chunks);
  L.cdig = take(2ull * kDigCap * Q.chunks);
  if (Q.layers) {
    L.rows = take(kRowBytes * R);
    L.tile_row = take(4ull * Q.tiles);
    L.group_row = take(4ull * Q.groups);
    L.pass_row = take(4ull * Q.passes);
    L.big_rows = take(4ull * std::max<uint64_t>(1, Q.big));
    L.mid_rows = take(4ull * std::max<uint64_t>(1, Q.mid));
    L.loff = take(8ull * (nlayers + 1));
    L.lk = take(8ull * nlayers);
    L.lkoff = take(8ull * nlayers);
  }
  L.total = o;
  return L;
}

Layout make_node_layout(uint32_t P, uint64_t N, uint64_t k) {
  const RowSize z = row_size(0, N, k, false);
  Plan Q;
  Q.rows = P;
  Q.cand = (uint64_t)P * kSub * z.capS;
  // tile slots: a node whose first element is not line-aligned may straddle one more tile
  const uint64_t MT = (N + (kTileAlign - 1) + kTile - 1) / kTile;
  const uint64_t MG = (MT + kGroup - 1) / kGroup;
  Q.tiles = (uint64_t)P * MT;
  Q.groups = (uint64_t)P * MG;
  Q.chunks = (uint64_t)P * z.chunks;
  Q.passes = 0;
  Q.big = 0;
  Q.mid = 0;
  Q.layers = false;
  Layout L = make_layout(Q, 0);
  L.capS = z.capS;
  L.cap = kSub * z.capS;
  L.tps_log = z.tps_log;
  L.MT = MT;
  L.MG = MG;
  L.MC = z.chunks;
  return L;
}

// per-layer call: node p, layer l is row p * nlayers + l
struct LayerPlan {
  Plan Q;
  uint64_t max_groups, max_cap, max_tiles, K;
};

LayerPlan plan_layers(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k) {
  LayerPlan lp{};
  lp.Q.rows = (uint64_t)P * nl;
  lp.Q.layers = true;
  for (uint32_t l = 0; l < nl; ++l) lp.K += k[l];
  for (uint32_t p = 0; p < P; ++p)
    for (uint32_t l = 0; l < nl; ++l) {
      const RowSize z = row_size((uint64_t)p * N + off[l], off[l + 1] - off[l], k[l], true);
      lp.Q.cand += (uint64_t)z.nsub * z.capS;
      lp.Q.tiles += z.nt;
      lp.Q.groups += z.groups;
      lp.Q.chunks += z.chunks;
      lp.Q.passes += z.npass;
      const bool big = big_predict(off[l + 1] - off[l], k[l], z.schunks);
      lp.Q.big += big ? 1 : 0;
      lp.Q.mid += layer_sampled(off[l + 1] - off[l], k[l]) && !big ? 1 : 0;
      lp.max_groups = std::max<uint64_t>(lp.max_groups, z.groups);
      lp.max_cap = std::max<uint64_t>(lp.max_cap, (uint64_t)z.nsub * z.capS);
      lp.max_tiles = std::max<uint64_t>(lp.max_tiles, z.nt);
    }
  return lp;
}

struct Dev {
  uint32_t P;
  uint32_t N;
  uint32_t k;
  uint32_t rs_lo;   // sample rank of the candidate threshold
  uint32_t rs_mid;  // sample rank of the zeroing threshold
  uint32_t tps_log; // whole-node call: log2 of the consecutive tiles sharing a counter
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
  uint32_t* h1s;  // [rows][kSpecBins][kH1]: second-digit counts of the gather's speculated bins
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
  uint16_t* cdig;  // [chunk][kDigCap]: last digits of the chunk's keys with T*'s upper 21 bits
  const struct Row* rows;     // per-layer call: row table
  const uint32_t* tile_row;   // per-layer call: row of every stream workgroup
  const uint32_t* group_row;  // per-layer call: row of every tile group
  const uint32_t* pass_row;   // per-layer call: row of every select / count / emit block
  const uint32_t* big_rows;   // per-layer call: the rows with big_predict, in row order
  const uint32_t* mid_rows;   // per-layer call: the other sampled rows, in row order
  uint32_t* runs;             // whole-node call: run table of the output, [P][S+1], or null
  uint32_t S;                 // segments of SPARCML_SEGMENT indices: ceil(N / SPARCML_SEGMENT)
};

// Geometry of one selection row. For the [P][N] call it follows from (P, N,
// k); for the per-layer call it is read from a table in the workspace.
struct Row {
  uint64_t base;    // first element in grad / residual
  uint64_t cand;    // first slot of the row's candidate regions (cand, oidx, oval)
  uint64_t tile0;   // first tile word (tmeta); in the per-layer call also the first stream workgroup
  uint64_t group0;  // first group word (gsum, gbase)
  uint64_t chunk0;  // first chunk word (cgt, ceq, ceqoff, cout)
  uint64_t out0;    // first output pair
  uint32_t n;       // elements
  uint32_t k;       // pairs to select
  uint32_t capS;    // candidate slots per counter region
  uint32_t nsub;    // counter regions in use (<= kSub)
  uint32_t rs_lo;   // sample rank of the candidate threshold
  uint32_t rs_mid;  // sample rank of the zeroing threshold
  uint32_t idx_off; // added to row-local indices in the output
  uint32_t schunks; // sample chunks of kSampleChunk elements
  uint32_t pass0;   // per-layer call: first block of the row in the select / count / emit grids
  uint32_t npass;   // blocks of those grids for the row
  uint32_t tps_log; // log2 of the consecutive tiles sharing a counter
  uint32_t pad;
};

static_assert(sizeof(Row) == kRowBytes, "row table entry size used by the workspace layout");

template <bool ROWS>
__device__ __forceinline__ Row row_of(const Dev& D, uint32_t p) {
  if constexpr (ROWS) {
    return D.rows[p];
  } else {
    Row R;
    R.base = (uint64_t)p * D.N;
    R.cand = (uint64_t)p * D.cap;
    R.tile0 = (uint64_t)p * D.MT;
    R.group0 = (uint64_t)p * D.MG;
    R.chunk0 = (uint64_t)p * D.MC;
    R.out0 = (uint64_t)p * D.k;
    R.n = D.N;
    R.k = D.k;
    R.capS = (uint32_t)D.capS;
    R.nsub = kSub;
    R.rs_lo = D.rs_lo;
    R.rs_mid = D.rs_mid;
    R.idx_off = 0u;
    R.schunks = kSampleChunks;
    R.pass0 = 0u;
    R.npass = 0u;
    R.tps_log = D.tps_log;
    R.pad = 0u;
    return R;
  }
}

// tiles of a row: its first tile starts at the 128-byte line holding its
// first element
__device__ __forceinline__ uint32_t row_tiles(const Row& R) {
  const uint32_t phi = tile_phase(R.base);
  return (uint32_t)(((uint64_t)R.n + phi + kTile - 1) / kTile);
}

// Source of the select, count and emit kernels: the ordered candidate list,
// or the whole row (residual holds a) on the rescan path.
__device__ __forceinline__ uint64_t source_len(const Dev& D, const Row& R, uint32_t p, bool rescan) {
  return rescan ? (uint64_t)R.n : (uint64_t)D.state[p].count;
}

// ---------------------------------------------------------------------------
// predict: reset the node's state and choose the two key thresholds.
// ---------------------------------------------------------------------------
// First of the kSpecBins first-digit bins the gather counts the second digit
// of: the bin of `mid` and its two neighbours.
__device__ __forceinline__ uint32_t spec_first_bin(uint32_t mid) {
  const uint32_t b = mid >> 20;
  return b > 0u ? b - 1u : 0u;
}

// Clears a row's histograms, the reservation counters its stream uses, and
// (with its thresholds) its state and flags.
template <int NT, bool ROWS = false>
__device__ __forceinline__ void reset_row(const Dev& D, uint32_t p, const Row& R) {
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < kH0; i += NT) D.h0[(size_t)p * kH0 + i] = 0u;
  for (uint32_t i = tid; i < kH1; i += NT) D.h1[(size_t)p * kH1 + i] = 0u;
  for (uint32_t i = tid; i < kH2; i += NT) D.h2[(size_t)p * kH2 + i] = 0u;
  if constexpr (!ROWS)
    for (uint32_t i = tid; i < kSpecBins * kH1; i += NT) D.h1s[(size_t)p * kSpecBins * kH1 + i] = 0u;
  for (uint32_t i = tid; i < R.nsub; i += NT) D.sub[((size_t)p * kSub + i) * 32] = 0u;  // the counters in use
}
__device__ __forceinline__ void set_state(const Dev& D, uint32_t p, uint32_t lo, uint32_t mid) {
  NodeState s{};
  s.lo = lo;
  s.mid = mid;
  D.state[p] = s;
  D.err[p] = 0u;
  D.info[p] = 0u;
}
// Thresholds that need no sample; false where the row is sampled.
__device__ __forceinline__ bool fixed_thresholds(const Row& R, bool layer, uint32_t& lo, uint32_t& mid) {
  if (R.k == 0) {
    lo = mid = 0xFFFFFFFFu;  // keys are < 2^31: no candidate
  } else if (R.k == R.n) {
    lo = mid = 0u;  // everything is selected
  } else if (layer && R.n <= kSmallLayer) {
    lo = 0u;            // a small layer is its own candidate list
    mid = 0xFFFFFFFFu;  // and nothing is zeroed before the selection
  } else {
    return false;
  }
  return true;
}

// One block per row, holding kPredictKeys sample keys per thread in
// registers, so a block takes samples of up to NT * kPredictKeys keys. The
// whole-node call runs 1024-thread blocks over the nodes (LIST = 0) and
// resets each node first. The per-layer call, whose rows the tile-table
// kernel has reset, runs 256-thread blocks over the sampled rows without
// big_predict (LIST = 1: block b takes row mid_rows[b]) and 512-thread blocks
// over the big_predict rows (LIST = 2: row big_rows[b]).
template <bool ROWS, int NT, int LIST>
__global__ __launch_bounds__(NT) void k_predict(const float* __restrict__ g,
                                                             const float* __restrict__ r, Dev D) {
  static_assert((LIST != 0) == ROWS, "the row lists exist in the per-layer call only");
  static_assert(NT * kPredictKeys ==
                    (LIST == 0 ? kSample : (LIST == 2 ? kLayerSampleChunks * kSampleChunk : kSmallSample)),
                "a block holds the largest sample of its rows");
  __shared__ uint32_t h1[4096];
  __shared__ uint32_t h2lo[2048];
  __shared__ uint32_t h2mid[2048];
  __shared__ uint32_t scr[NT / kWave + 3];
  const uint32_t p = LIST == 0 ? blockIdx.x : (LIST == 1 ? D.mid_rows[blockIdx.x] : D.big_rows[blockIdx.x]);
  const Row R = row_of<ROWS>(D, p);
  const uint32_t tid = threadIdx.x;
  if constexpr (!ROWS) reset_row<NT>(D, p, R);

  uint32_t lo, mid;
  if (!fixed_thresholds(R, ROWS, lo, mid)) {
    for (uint32_t i = tid; i < 4096; i += NT) h1[i] = 0u;
    for (uint32_t i = tid; i < 2048; i += NT) h2lo[i] = h2mid[i] = 0u;
    __syncthreads();
    const uint64_t base = R.base;
    const uint32_t nsamp = R.schunks * kSampleChunk;  // <= NT * kPredictKeys
    const bool whole = R.n <= nsamp;
    // chunk c starts at c * stride, stride = (n - 64) / (chunks - 1) rounded
    // down: the last chunk ends at most chunks - 1 elements short of the row's
    // end (the sample only guides the thresholds)
    const uint64_t stride = whole ? 0ull : (uint64_t)(R.n - kSampleChunk) / (R.schunks - 1);
    const uint32_t nvalid = whole ? R.n : nsamp;
    // Sample i's element; positions past the sample read element 0 and are
    // masked afterwards. No branch around the loads, so all of a thread's
    // loads are in flight together (a branch per sample made each wait for
    // the previous one).
    auto sample_pos = [&](uint32_t i) -> uint64_t {
      const uint64_t pos = whole ? (uint64_t)i : (uint64_t)(i / kSampleChunk) * stride + i % kSampleChunk;
      return i < nvalid ? pos : 0ull;
    };
    const float* gb = g + base;
    const float* rb = r + base;
    uint32_t keys[kPredictKeys];
#pragma unroll
    for (int j = 0; j < kPredictKeys; ++j) {
      const uint32_t i = j * NT + tid;
      const uint64_t pos = sample_pos(i);
      const uint32_t key = mag_key(gb[pos] + rb[pos]);
      keys[j] = i < nvalid ? key : 0xFFFFFFFFu;  // 0xFFFFFFFF marks "no sample"
    }
#pragma unroll
    for (int j = 0; j < kPredictKeys; ++j)
      if (keys[j] != 0xFFFFFFFFu) atomicAdd(&h1[keys[j] >> 19], 1u);
    __syncthreads();
    uint32_t b_lo, a_lo, b_mid, a_mid;
    block_find_suffix<NT, 4096>(h1, R.rs_lo, scr, b_lo, a_lo);
    block_find_suffix<NT, 4096>(h1, R.rs_mid, scr, b_mid, a_mid);
#pragma unroll
    for (int j = 0; j < kPredictKeys; ++j) {
      const uint32_t key = keys[j];
      if (key == 0xFFFFFFFFu) continue;
      if ((key >> 19) == b_lo) atomicAdd(&h2lo[(key >> 8) & 2047u], 1u);
      if ((key >> 19) == b_mid) atomicAdd(&h2mid[(key >> 8) & 2047u], 1u);
    }
    __syncthreads();
    uint32_t c_lo, x_lo, c_mid, x_mid;
    block_find_suffix<NT, 2048>(h2lo, R.rs_lo - a_lo, scr, c_lo, x_lo);
    block_find_suffix<NT, 2048>(h2mid, R.rs_mid - a_mid, scr, c_mid, x_mid);
    lo = (b_lo << 19) | (c_lo << 8);
    mid = (b_mid << 19) | (c_mid << 8);
  }
  if (tid == 0) set_state(D, p, lo, mid);
}

// ---------------------------------------------------------------------------
// stream: a = g + r, per-tile candidate compaction, residual write-back.
// ---------------------------------------------------------------------------
template <bool ROWS>
__global__ __launch_bounds__(kStreamThreads) void k_stream(const float* __restrict__ g,
                                                           float* __restrict__ r, Dev D) {
  __shared__ uint32_t s_cnt[kNW];
  __shared__ uint32_t s_base;
  __shared__ uint32_t s_stored;
  // each XCD streams one contiguous stretch of tiles (steadier than the
  // default round-robin of consecutive tiles over the 8 XCDs)
  const uint32_t w = xcd_contiguous(blockIdx.x, gridDim.x);
  uint32_t p, t;
  Row R;
  if constexpr (ROWS) {
    p = D.tile_row[w];
    R = row_of<true>(D, p);
    t = w - (uint32_t)R.tile0;
  } else {
    p = w / (uint32_t)D.MT;
    t = w % (uint32_t)D.MT;
    R = row_of<false>(D, p);
    if (t >= row_tiles(R)) return;
  }
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = lane_id();
  const uint32_t wid = tid / kWave;
  const uint32_t N = R.n;
  const uint64_t pN = R.base;
  const uint32_t phi = tile_phase(pN);
  const int64_t e0 = (int64_t)t * kTile - (int64_t)phi + 4 * (int64_t)tid;  // node-local index
  const uint64_t grp = ((pN - phi) >> 2) + (uint64_t)t * (kTile / 4) + tid;   // float4 group
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
    const uint32_t sc = (t >> R.tps_log) % R.nsub;
    uint32_t off = run ? atomicAdd(&D.sub[((size_t)p * kSub + sc) * 32], run) : 0u;
    const bool stored = (uint64_t)off + run <= R.capS;
    D.tmeta[R.tile0 + t] = ((uint64_t)run << 32) | (stored ? (uint32_t)(sc * R.capS + off) : kNotStored);
    if (!stored) atomicOr(&D.state[p].fail, 1u);
    s_base = (uint32_t)(sc * R.capS + off);
    s_stored = stored ? 1u : 0u;
  }
  __syncthreads();
  const bool stored = s_stored != 0u;
  if (stored && flags) {
    uint32_t pos = s_base + s_cnt[wid] + pre;
    uint64_t* cd = D.cand + R.cand;
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
// tsum: candidate count of every group of kGroup tiles.
// ---------------------------------------------------------------------------
template <bool ROWS>
__global__ __launch_bounds__(256) void k_tsum(Dev D) {
  __shared__ uint32_t scr[256 / kWave + 3];
  // per-layer call: one block per group of every row (1D grid)
  const uint32_t p = ROWS ? D.group_row[blockIdx.x] : blockIdx.y;
  const Row R = row_of<ROWS>(D, p);
  const uint64_t gidx = ROWS ? blockIdx.x - R.group0 : blockIdx.x;
  const uint32_t nt = row_tiles(R);
  if (gidx * kGroup >= nt) return;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kGroup / 256; ++i) {
    const uint64_t t = gidx * kGroup + (uint64_t)i * 256 + threadIdx.x;
    if (t < nt) s += (uint32_t)(D.tmeta[R.tile0 + t] >> 32);
  }
  uint32_t tot;
  block_exclusive_scan<256>(s, scr, tot);
  if (threadIdx.x == 0) D.gsum[R.group0 + gidx] = tot;
}

// ---------------------------------------------------------------------------
// gscan: group offsets, candidate count and the path of the node.
// ---------------------------------------------------------------------------
template <bool ROWS>
__global__ __launch_bounds__(1024) void k_gscan(Dev D) {
  __shared__ uint32_t scr[1024 / kWave + 3];
  const uint32_t p = blockIdx.x;
  const Row R = row_of<ROWS>(D, p);
  const uint64_t ng = (row_tiles(R) + kGroup - 1) / kGroup;
  uint64_t carry = 0;
  for (uint64_t g0 = 0; g0 < ng; g0 += 1024) {
    const uint64_t gi = g0 + threadIdx.x;
    const uint32_t v = gi < ng ? D.gsum[R.group0 + gi] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<1024>(v, scr, tot);
    if (gi < ng) D.gbase[R.group0 + gi] = (uint32_t)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) {
    const uint64_t cap = (uint64_t)R.nsub * R.capS;
    const bool rescan = D.state[p].fail != 0u || carry < R.k || carry > cap;
    D.state[p].count = (uint32_t)std::min<uint64_t>(carry, cap);
    D.state[p].mode = rescan ? 1u : 0u;
    D.info[p] = rescan ? 1u : 0u;
  }
}

// ---------------------------------------------------------------------------
// gather: candidate runs into index order, first radix level on the way.
// A block owns kGroup consecutive tiles, whose runs land contiguously in the
// ordered list; each thread walks output positions and finds its tile by a
// binary search over the block's prefix of run lengths in LDS, so loads and
// stores stay spread over the whole block. On the rescan path it restores
// instead: thread t puts the zeroed candidates of the group's tile t back
// into residual (one launch less than a kernel of its own).
// ---------------------------------------------------------------------------
template <bool ROWS>
__global__ __launch_bounds__(kGroup) void k_gather(float* __restrict__ r, Dev D) {
  constexpr int kU = 8;
  __shared__ uint32_t h[kH0];
  __shared__ uint32_t hs[ROWS ? 1 : kSpecBins * kH1];
  __shared__ uint32_t s_excl[kGroup + 1];
  __shared__ uint32_t s_toff[kGroup];
  __shared__ uint32_t scr[kGroup / kWave + 3];
  const uint32_t p = ROWS ? D.group_row[blockIdx.x] : blockIdx.y;  // per-layer call: 1D grid over groups
  const Row R = row_of<ROWS>(D, p);
  const uint64_t gidx = ROWS ? blockIdx.x - R.group0 : blockIdx.x;
  const uint32_t nt = row_tiles(R);
  if (gidx * kGroup >= nt) return;
  if (D.state[p].mode != 0u) {  // rescan path
    const uint64_t t = gidx * kGroup + threadIdx.x;
    const uint64_t meta = t < nt ? D.tmeta[R.tile0 + t] : ((uint64_t)0 << 32 | kNotStored);
    const uint32_t off = (uint32_t)meta, cnt = (uint32_t)(meta >> 32);
    if (off == kNotStored) return;
    const uint32_t mid = D.state[p].mid;
    for (uint32_t j = 0; j < cnt; ++j) {
      const uint64_t c = D.cand[R.cand + off + j];
      const float v = __uint_as_float((uint32_t)c);
      if (mag_key(v) >= mid) r[R.base + (uint32_t)(c >> 32)] = v;
    }
    return;
  }
  for (uint32_t i = threadIdx.x; i < kH0; i += kGroup) h[i] = 0u;
  if constexpr (!ROWS)
    for (uint32_t i = threadIdx.x; i < kSpecBins * kH1; i += kGroup) hs[i] = 0u;
  const uint32_t slo = spec_first_bin(D.state[p].mid);
  const uint64_t t = gidx * kGroup + threadIdx.x;
  const uint64_t meta = t < nt ? D.tmeta[R.tile0 + t] : 0ull;
  const uint32_t cnt = (uint32_t)(meta >> 32);
  s_toff[threadIdx.x] = cnt ? (uint32_t)meta : 0u;
  uint32_t tot;
  s_excl[threadIdx.x] = block_exclusive_scan<kGroup>(cnt, scr, tot);
  if (threadIdx.x == 0) s_excl[kGroup] = tot;
  __syncthreads();
  const size_t nbase = R.cand;
  const size_t out = nbase + D.gbase[R.group0 + gidx];
  for (uint32_t i0 = threadIdx.x; i0 < tot; i0 += kGroup * kU) {
    // Positions past the group's candidates search for (and load) its last
    // one, and only the stores are masked: with the search and the load under
    // the position's condition, the per-layer build kept them as branches and
    // waited for every store to complete before the next.
    uint32_t src[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t i = std::min(i0 + u * kGroup, tot - 1u);
      // the last tile whose run starts at or before i (a fixed number of
      // branch-free steps, so the kU searches interleave)
      uint32_t lo = 0;
#pragma unroll
      for (uint32_t step = kGroup / 2; step > 0; step >>= 1)
        lo = s_excl[lo + step] <= i ? lo + step : lo;
      src[u] = s_toff[lo] + (i - s_excl[lo]);
    }
    uint64_t c[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) c[u] = D.cand[nbase + src[u]];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool valid = i0 + u * kGroup < tot;
      const float v = __uint_as_float((uint32_t)c[u]);
      const uint32_t key = mag_key(v);
      if (valid) {
        const uint32_t i = i0 + u * kGroup;
        D.oval[out + i] = v;
        D.oidx[out + i] = (uint32_t)(c[u] >> 32);
        if constexpr (!ROWS) {
          const uint32_t sb = (key >> 20) - slo;
          if (sb < kSpecBins) atomicAdd(&hs[sb * kH1 + ((key >> 10) & 1023u)], 1u);
        }
      }
      wave_hist_add_capped<2>(h, key >> 20, valid);
    }
  }
  __syncthreads();
  uint32_t* gh = D.h0 + (size_t)p * kH0;
  for (uint32_t i = threadIdx.x; i < kH0; i += kGroup)
    if (h[i]) atomicAdd(&gh[i], h[i]);
  if constexpr (!ROWS) {
    uint32_t* gs = D.h1s + (size_t)p * kSpecBins * kH1;
    for (uint32_t i = threadIdx.x; i < kSpecBins * kH1; i += kGroup)
      if (hs[i]) atomicAdd(&gs[i], hs[i]);
  }
}

// Digits chosen so far, recomputed from the global histograms of the levels
// below `level` (each block does it; they all agree). The bins are loaded
// first (DigitBins::load) and decided on later, so that a kernel can issue
// its first data loads in between and wait for the bins alone.
template <int NT>
struct DigitBins {
  uint32_t c0[kH0 / NT], c1[kH1 / NT], c2[kH2 / NT];
  __device__ __forceinline__ void load(const Dev& D, uint32_t p, int level) {
    if (level >= 1) load_suffix_bins<NT, kH0>(D.h0 + (size_t)p * kH0, c0);
    if (level >= 2) load_suffix_bins<NT, kH1>(D.h1 + (size_t)p * kH1, c1);
    if (level >= 3) load_suffix_bins<NT, kH2>(D.h2 + (size_t)p * kH2, c2);
  }
  __device__ __forceinline__ void decide(uint32_t k, int level, uint32_t* scr, uint32_t& prefix, uint32_t& krem) {
    krem = k;
    prefix = 0;
    uint32_t bin, above;
    if (level >= 1) {
      block_find_suffix_held<NT, kH0>(c0, krem, scr, bin, above);
      krem -= above;
      prefix = bin;
    }
    if (level >= 2) {
      block_find_suffix_held<NT, kH1>(c1, krem, scr, bin, above);
      krem -= above;
      prefix = (prefix << 10) | bin;
    }
    if (level >= 3) {
      block_find_suffix_held<NT, kH2>(c2, krem, scr, bin, above);
      krem -= above;
      prefix = (prefix << 10) | bin;
    }
  }
};

// ---------------------------------------------------------------------------
// hist: one radix level of T*. Level 0 runs only on the rescan path (the
// gather kernel builds it for the candidate path).
//
// The last level also tallies each chunk of kChunk source elements against
// T*'s upper 21 bits, which it knows: cgt[c] = keys above them, ceq[c] = keys
// sharing them, and the last digits of the first kDigCap of those in
// cdig[c]. Once the level's histogram gives the last digit, the scan turns
// these into the chunk's counts above and equal to T*, so no pass over the
// keys is needed for them; a chunk with more such keys than slots (ties, or
// the crowding of error-feedback residuals just under T*) sets the row's
// ovf, and the count pass counts that chunk's keys itself.
// ---------------------------------------------------------------------------
template <int LEVEL, bool ROWS>
__global__ __launch_bounds__(256) void k_hist(const float* __restrict__ r, Dev D) {
  constexpr int NB = LEVEL == 0 ? kH0 : (LEVEL == 1 ? kH1 : kH2);
  constexpr int kU = 16;
  static_assert(256 * kU == kChunk, "a pass of the block is one chunk");
  __shared__ uint32_t h[NB];
  __shared__ uint32_t scr[256 / kWave + 3];
  __shared__ uint32_t s_sum[2 * 256 / kWave];
  __shared__ uint32_t s_eq;  // keys of the chunk sharing T*'s upper bits (last level)
  // per-layer call: a 1D grid, each row owning npass consecutive blocks
  const uint32_t p = ROWS ? D.pass_row[blockIdx.x] : blockIdx.y;
  const bool rescan = D.state[p].mode != 0u;
  if (LEVEL == 0 && !rescan) return;
  const Row R = row_of<ROWS>(D, p);
  if (R.k == 0) return;
  const uint64_t bx = ROWS ? blockIdx.x - R.pass0 : blockIdx.x;
  const uint64_t nbx = ROWS ? R.npass : gridDim.x;
  for (uint32_t i = threadIdx.x; i < NB; i += 256) h[i] = 0u;
  const uint64_t n = source_len(D, R, p, rescan);
  const float* src = rescan ? r + R.base : D.oval + R.cand;
  const uint64_t stride = nbx * 256 * kU;
  // values of the pass starting at i0; positions past the end reread the
  // last element and are masked where the values are used, a pass later.
  // (Masking them here let the compiler put each load under its own branch
  // and wait for it there, one load in flight at a time.)
  const uint64_t last = n ? n - 1 : 0;
  auto load = [&](uint64_t i0, float (&x)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint64_t i = i0 + (uint64_t)u * 256;
      x[u] = src[i < n ? i : last];
    }
  };
  DigitBins<256> bins;
  bins.load(D, p, LEVEL);
  float x[kU];
  load(bx * 256 * kU + threadIdx.x, x);  // in flight while the digits are decided
  uint32_t prefix, krem;
  bins.decide(R.k, LEVEL, scr, prefix, krem);
  if (LEVEL == 1 && !ROWS && !rescan) {
    const uint32_t sb = prefix - spec_first_bin(D.state[p].mid);
    if (sb < kSpecBins) {  // the gather counted this level already
      if (bx == 0) {
        const uint32_t* src = D.h1s + (size_t)p * kSpecBins * kH1 + (size_t)sb * kH1;
        uint32_t* dst = D.h1 + (size_t)p * kH1;
        for (uint32_t i = threadIdx.x; i < kH1; i += 256) dst[i] = src[i];
      }
      return;
    }
  }
  if (LEVEL == 2 && threadIdx.x == 0) s_eq = 0u;
  __syncthreads();
  // passes are whole chunks, block-uniform (the last level's tallies take
  // barriers): pass base c0 = chunk c's first element
  for (uint64_t c0 = bx * 256 * kU; c0 < n; c0 += stride) {
    const uint64_t i0 = c0 + threadIdx.x;
    float nx[kU];
    load(i0 + stride, nx);  // the block's next pass, in flight during this one
    uint32_t above = 0u;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t kk = i0 + (uint64_t)u * 256 < n ? mag_key(x[u]) : 0xFFFFFFFFu;
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
        above += (kk != 0xFFFFFFFFu && (kk >> 10) > prefix) ? 1u : 0u;
      }
      // level 0 keys crowd into a few bins: aggregate per wave; the lower
      // digits spread out, where plain LDS atomics are cheaper
      if (LEVEL == 0) {
        wave_hist_add_capped<2>(h, bin, hit);
      } else if (hit) {
        atomicAdd(&h[bin], 1u);
        if (LEVEL == 2) {
          const uint32_t slot = atomicAdd(&s_eq, 1u);
          if (slot < (uint32_t)kDigCap)
            D.cdig[(R.chunk0 + c0 / kChunk) * kDigCap + slot] = (uint16_t)bin;
        }
      }
    }
    if constexpr (LEVEL == 2) {
      uint32_t tot_above, unused;
      block_sum2<256>(above, 0u, s_sum, tot_above, unused);  // its barriers also order the s_eq adds
      if (threadIdx.x == 0) {
        const uint32_t eq = s_eq;
        D.cgt[R.chunk0 + c0 / kChunk] = tot_above;
        D.ceq[R.chunk0 + c0 / kChunk] = eq;
        if (eq > (uint32_t)kDigCap) atomicOr(&D.state[p].ovf, 1u);
        s_eq = 0u;
      }
      __syncthreads();  // the reset before the next pass's adds
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) x[u] = nx[u];
  }
  __syncthreads();
  uint32_t* gh = (LEVEL == 0 ? D.h0 : (LEVEL == 1 ? D.h1 : D.h2)) + (size_t)p * NB;
  for (uint32_t i = threadIdx.x; i < NB; i += 256)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// ---------------------------------------------------------------------------
// count: per chunk of the source, elements above and equal to T*, for the
// chunks the last histogram pass could not tally (more keys of T*'s upper 21
// bits than digit slots); the count goes out marked kEqCounted. Rows without
// such a chunk (ovf clear) leave at once, and the other chunks are skipped.
// ---------------------------------------------------------------------------
template <bool ROWS>
__global__ __launch_bounds__(kChunkThreads) void k_count(const float* __restrict__ r, Dev D) {
  __shared__ uint32_t scr[kChunkThreads / kWave + 3];
  __shared__ uint32_t s_sum[2 * (kChunkThreads / kWave)];
  const uint32_t p = ROWS ? D.pass_row[blockIdx.x] : blockIdx.y;  // per-layer call: 1D grid
  if (D.state[p].ovf == 0u) return;
  const Row R = row_of<ROWS>(D, p);
  if (R.k == 0) return;
  const uint64_t bx = ROWS ? blockIdx.x - R.pass0 : blockIdx.x;
  const uint64_t nbx = ROWS ? R.npass : gridDim.x;
  const bool rescan = D.state[p].mode != 0u;
  const uint64_t n = source_len(D, R, p, rescan);
  const uint64_t nchunks = (n + kChunk - 1) / kChunk;
  const float* src = rescan ? r + R.base : D.oval + R.cand;
  // chunk c's values; positions past the end reread the last element (no
  // branch around the loads) and are masked where used
  const uint64_t last = n ? n - 1 : 0;
  auto load = [&](uint64_t c, float (&v)[kChunkIt]) {
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * kChunkThreads + threadIdx.x;
      v[it] = src[j < n ? j : last];
    }
  };
  DigitBins<kChunkThreads> bins;
  bins.load(D, p, 3);
  float v[kChunkIt];
  load(bx, v);  // in flight while the digits are decided
  uint32_t T, m;
  bins.decide(R.k, 3, scr, T, m);
  for (uint64_t c = bx; c < nchunks; c += nbx) {
    float nv[kChunkIt];
    load(c + nbx, nv);  // the block's next chunk, in flight during this one
    if (D.ceq[R.chunk0 + c] <= (uint32_t)kDigCap) {  // tallied (block-uniform)
#pragma unroll
      for (int it = 0; it < kChunkIt; ++it) v[it] = nv[it];
      continue;
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * kChunkThreads + threadIdx.x;
      const uint32_t key = mag_key(v[it]);
      gt += (j < n && key > T) ? 1u : 0u;
      eq += (j < n && key == T) ? 1u : 0u;
    }
    uint32_t tgt, teq;
    block_sum2<kChunkThreads>(gt, eq, s_sum, tgt, teq);
    if (threadIdx.x == 0) {  // block_sum2's barriers follow every thread's read of the tally
      D.cgt[R.chunk0 + c] = tgt;
      D.ceq[R.chunk0 + c] = teq | kEqCounted;
    }
#pragma unroll
    for (int it = 0; it < kChunkIt; ++it) v[it] = nv[it];
  }
}

// ---------------------------------------------------------------------------
// scan: T* and its tie quota m from the three radix levels, each chunk's
// counts above and equal to T* (finished from the last histogram pass's
// tallies with T*'s last digit, or the count pass's where the row
// overflowed its digit slots), then the tie quota in index order and each
// chunk's output offset.
// ---------------------------------------------------------------------------
template <bool ROWS>
__global__ __launch_bounds__(1024) void k_scan(Dev D) {
  __shared__ uint32_t scr[1024 / kWave + 3];
  const uint32_t p = blockIdx.x;
  const Row R = row_of<ROWS>(D, p);
  if (R.k == 0) return;
  DigitBins<1024> bins;
  bins.load(D, p, 3);
  uint32_t T, m;
  bins.decide(R.k, 3, scr, T, m);
  if (threadIdx.x == 0) {
    D.state[p].T = T;
    D.state[p].m = m;
  }
  const uint32_t d3 = T & 1023u;
  const bool rescan = D.state[p].mode != 0u;
  const uint64_t n = source_len(D, R, p, rescan);
  const uint64_t nchunks = (n + kChunk - 1) / kChunk;
  uint32_t eq_carry = 0, out_carry = 0;
  for (uint64_t c0 = 0; c0 < nchunks; c0 += 1024) {
    const uint64_t c = c0 + threadIdx.x;
    const bool in = c < nchunks;
    uint32_t gt = in ? D.cgt[R.chunk0 + c] : 0u;
    uint32_t eq = in ? D.ceq[R.chunk0 + c] : 0u;
    if (in && (eq & kEqCounted) == 0u) {  // keys of T*'s upper bits: above T* by their last digit, or equal
      static_assert(kDigCap % 8 == 0, "16-byte loads of digits");
      const uint4* dg = reinterpret_cast<const uint4*>(D.cdig + (R.chunk0 + c) * kDigCap);
      uint32_t w[kDigCap / 2];
#pragma unroll
      for (int q = 0; q < kDigCap / 8; ++q) {
        const uint4 a = dg[q];
        w[4 * q] = a.x;
        w[4 * q + 1] = a.y;
        w[4 * q + 2] = a.z;
        w[4 * q + 3] = a.w;
      }
      uint32_t g2 = 0u, e2 = 0u;
#pragma unroll
      for (int i = 0; i < kDigCap; ++i) {
        const uint32_t dgt = (w[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
        const bool valid = (uint32_t)i < eq;
        g2 += (valid && dgt > d3) ? 1u : 0u;
        e2 += (valid && dgt == d3) ? 1u : 0u;
      }
      gt += g2;
      eq = e2;
    }
    eq &= ~kEqCounted;
    if (in) D.ceq[R.chunk0 + c] = eq;  // the emit's tie test reads the final count
    uint32_t tot;
    const uint32_t eq_off = eq_carry + block_exclusive_scan<1024>(eq, scr, tot);
    eq_carry += tot;
    const uint32_t quota = eq_off >= m ? 0u : (m - eq_off < eq ? m - eq_off : eq);
    const uint32_t sel = gt + quota;
    const uint32_t out_off = out_carry + block_exclusive_scan<1024>(sel, scr, tot);
    out_carry += tot;
    if (in) {
      D.ceqoff[R.chunk0 + c] = eq_off;
      D.cout[R.chunk0 + c] = out_off;
    }
  }
  if (threadIdx.x == 0 && out_carry != R.k) D.err[p] = 1u;
}

// ---------------------------------------------------------------------------
// emit: selected pairs in index order; residual finished.
//
// RUNS (whole-node call): the run table of the output as well, the one the
// sparse reduce would otherwise build with a pass over the indices:
// runs[p][s] = position of node p's first output pair with index >= s * 4096
// (positions count from the start of the [P][k] output; runs[p][S] is the
// node's end). Candidates are in index order and a superset of the output,
// so entry s is the output position of the first candidate with index >=
// s * 4096, which is the number of selected candidates before it: candidate
// j (index e_j) writes the entries s with e_{j-1} < s * 4096 <= e_j, and the
// node's last candidate also the entries past it (the node's end). The
// predecessor's index comes from the lane below (a DPP shift); a wave's
// lane 0 takes it from the last lane of the wave before, through LDS, and the
// chunk's first candidate from memory.
// ---------------------------------------------------------------------------
template <bool ROWS, bool RUNS, int IT>
__global__ __launch_bounds__(kChunk / IT) void k_emit(float* __restrict__ r, uint32_t* __restrict__ out_idx,
                                                        float* __restrict__ out_val, Dev D) {
  static_assert(!(ROWS && RUNS), "run tables of whole-node calls only");
  constexpr int NT = kChunk / IT;  // threads: IT candidates of each chunk per thread
  constexpr int NW = NT / kWave;
  __shared__ uint32_t s_eq[IT * NW];
  __shared__ uint32_t s_sel[IT * NW];
  __shared__ uint32_t s_last[RUNS ? IT * NW : 1];  // index of each (it, wave)'s last candidate
  const uint32_t p = ROWS ? D.pass_row[blockIdx.x] : blockIdx.y;  // per-layer call: 1D grid
  const Row R = row_of<ROWS>(D, p);
  uint32_t* tab = RUNS ? D.runs + (uint64_t)p * (D.S + 1) : nullptr;
  if (R.k == 0) {  // nothing selected: every run of the node is empty
    if constexpr (RUNS)
      for (uint64_t s = (uint64_t)blockIdx.x * NT + threadIdx.x; s <= D.S;
           s += (uint64_t)gridDim.x * NT)
        tab[s] = (uint32_t)R.out0;
    return;
  }
  const uint64_t bx = ROWS ? blockIdx.x - R.pass0 : blockIdx.x;
  const uint64_t nbx = ROWS ? R.npass : gridDim.x;
  const bool rescan = D.state[p].mode != 0u;
  const uint32_t T = D.state[p].T;
  const uint32_t m = D.state[p].m;
  const uint32_t mid = D.state[p].mid;
  const uint32_t lane = lane_id();
  const uint32_t wid = threadIdx.x / kWave;
  const uint64_t n = source_len(D, R, p, rescan);
  const uint64_t nchunks = (n + kChunk - 1) / kChunk;
  const uint64_t pN = R.base;
  const uint32_t K = R.k;
  const float* vsrc = rescan ? r + pN : D.oval + R.cand;
  const uint32_t* isrc = D.oidx + R.cand;
  uint32_t* oi = out_idx + R.out0;
  float* ov = out_val + R.out0;
  // chunk c's values and row-local indices (RUNS: and the index of the
  // candidate before the chunk); positions past the end reread the last
  // element (no branch around the loads) and are masked where used
  const uint64_t last = n ? n - 1 : 0;
  auto load = [&](uint64_t c, float (&v)[IT], uint32_t (&e)[IT], uint32_t& pc) {
    const uint64_t c0 = c * kChunk;
    if (rescan) {  // the source is the row itself: the position is the index
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const uint64_t j = c0 + (uint64_t)it * NT + threadIdx.x;
        v[it] = vsrc[j < n ? j : last];
        e[it] = (uint32_t)j;
      }
      pc = (uint32_t)c0 - 1u;
    } else {
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const uint64_t j = c0 + (uint64_t)it * NT + threadIdx.x;
        const uint64_t jj = j < n ? j : last;
        v[it] = vsrc[jj];
        e[it] = isrc[jj];
      }
      if constexpr (RUNS) pc = isrc[std::min(c0 ? c0 - 1 : 0, last)];  // the same word for every lane
    }
  };
  float v[IT];
  uint32_t e[IT], pc = 0u;
  load(bx, v, e, pc);
  for (uint64_t c = bx; c < nchunks; c += nbx) {
    const uint32_t eq_base = D.ceqoff[R.chunk0 + c];
    const uint32_t out_base = D.cout[R.chunk0 + c];
    const uint32_t teq = D.ceq[R.chunk0 + c];
    float nv[IT];
    uint32_t ne[IT], npc = 0u;
    load(c + nbx, nv, ne, npc);  // the block's next chunk, in flight during this one
    // per (it, wave): ranks of equal keys, needed only where some key of the
    // chunk equals T* with tie quota left (usually one chunk of the row)
    uint32_t eq_pre[IT];
    uint32_t eq_bits = 0;
    if (teq != 0u && eq_base < m) {
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const uint64_t j = c * kChunk + (uint64_t)it * NT + threadIdx.x;
        const bool is_eq = j < n && mag_key(v[it]) == T;
        const uint64_t em = ballot(is_eq);
        eq_bits |= (is_eq ? 1u : 0u) << it;
        eq_pre[it] = lanes_below(em);
        if (lane == 0) s_eq[it * NW + wid] = popc64(em);
      }
      __syncthreads();
      static_assert(IT * NW == kWave, "one wave scans the per-(it, wave) counts");
      if (threadIdx.x < kWave) {
        const uint32_t x = s_eq[threadIdx.x];
        s_eq[threadIdx.x] = wave_inclusive_scan(x) - x;
      }
      __syncthreads();
    }
    // then ranks of the selected elements
    uint32_t sel_bits = 0;
    uint32_t sel_pre[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * NT + threadIdx.x;
      const uint32_t key = mag_key(v[it]);
      const bool is_eq = (eq_bits >> it) & 1u;  // set only on the tie path above
      const bool sel = j < n && (key > T || (is_eq && eq_base + s_eq[it * NW + wid] + eq_pre[it] < m));
      sel_bits |= (sel ? 1u : 0u) << it;
      const uint64_t sm = ballot(sel);
      sel_pre[it] = lanes_below(sm);
      if (lane == 0) s_sel[it * NW + wid] = popc64(sm);
      if (RUNS && lane == kWave - 1) s_last[it * NW + wid] = e[it];
    }
    __syncthreads();
    static_assert(IT * NW == kWave, "one wave scans the per-(it, wave) counts");
    if (threadIdx.x < kWave) {
      const uint32_t x = s_sel[threadIdx.x];
      s_sel[threadIdx.x] = wave_inclusive_scan(x) - x;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint64_t j = c * kChunk + (uint64_t)it * NT + threadIdx.x;
      if (j >= n) continue;
      const bool high = mag_key(v[it]) >= mid;  // written as +0 by the stream kernel
      if ((sel_bits >> it) & 1u) {
        const uint32_t pos = out_base + s_sel[it * NW + wid] + sel_pre[it];
        if (pos < K) {  // non-temporal: the reduce reads them from HBM anyway, and dirty lines
                        // left in the memory-side cache would be written back during its first pass
          __builtin_nontemporal_store(e[it] + R.idx_off, &oi[pos]);
          __builtin_nontemporal_store(v[it], &ov[pos]);
        }
        if (rescan || !high) __builtin_nontemporal_store(0.0f, &r[pN + e[it]]);
      } else if (!rescan && high) {
        __builtin_nontemporal_store(v[it], &r[pN + e[it]]);  // zeroed on the guess but not selected: restore
      }
    }
    if constexpr (RUNS) {
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const uint64_t j = c * kChunk + (uint64_t)it * NT + threadIdx.x;
        // the predecessor's index: the lane below, or for lane 0 the last
        // candidate of the (it, wave) before, or the one before the chunk
        const uint32_t flat = it * NW + wid;
        const uint32_t below = flat ? s_last[flat - 1] : pc;
        const uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp((int)below, (int)e[it], 0x138, 0xF, 0xF, false);
        if (j >= n) continue;  // lanes past the end come after every active lane of the wave
        const uint32_t s_hi = e[it] >> kSegmentBits;
        const uint32_t s_lo = j ? (prev >> kSegmentBits) + 1u : 0u;
        if (s_lo <= s_hi || j == n - 1) {
          // selected candidates before this one (its output position if selected)
          const uint32_t at = (uint32_t)R.out0 + std::min(out_base + s_sel[flat] + sel_pre[it], K);
          for (uint32_t s = s_lo; s <= s_hi; ++s) tab[s] = at;
          if (j == n - 1)
            for (uint32_t s = s_hi + 1u; s <= D.S; ++s) tab[s] = (uint32_t)R.out0 + K;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      v[it] = nv[it];
      e[it] = ne[it];
    }
    pc = npc;
    __syncthreads();  // s_eq / s_sel are reused by the next chunk
  }
}

// ---------------------------------------------------------------------------
// per-layer call: layer offsets and k's in, row table and tile-to-row out.
// ---------------------------------------------------------------------------
constexpr int kLayersPerSetup = 120;

struct LayerChunk {
  uint64_t off[kLayersPerSetup + 1];
  uint64_t k[kLayersPerSetup];
  uint64_t koff[kLayersPerSetup];  // output offset of the layer within a node's row
};

__global__ void k_layers_in(uint64_t* loff, uint64_t* lk, uint64_t* lkoff, uint32_t first, uint32_t count,
                            LayerChunk in) {
  for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) {
    lk[first + i] = in.k[i];
    lkoff[first + i] = in.koff[i];
    loff[first + i] = in.off[i];
  }
  if (threadIdx.x == 0) loff[first + count] = in.off[count];
}

// One workgroup: every row's sizes (row_size, as the host computed them),
// exclusive scans of their slices, the sample ranks of its thresholds, and
// the lists of sampled rows for the two prediction block sizes.
__global__ __launch_bounds__(1024) void k_rows_plan(Row* rows, uint32_t* big_rows, uint32_t* mid_rows,
                                                    const uint64_t* loff, const uint64_t* lk, const uint64_t* lkoff,
                                                    uint32_t P, uint64_t N, uint32_t nl, uint64_t K) {
  __shared__ uint64_t scr[1024 / kWave + 1];
  uint64_t c_cand = 0, c_tiles = 0, c_groups = 0, c_chunks = 0, c_pass = 0, c_big = 0, c_mid = 0;  // carried
  const uint64_t nrows = (uint64_t)P * nl;
  for (uint64_t r0 = 0; r0 < nrows; r0 += 1024) {
    const uint64_t ri = r0 + threadIdx.x;
    const bool in = ri < nrows;
    uint64_t base = 0, n = 0, k = 0, koff = 0, xoff = 0;
    uint32_t p = 0;
    if (in) {
      p = (uint32_t)(ri / nl);
      const uint32_t l = (uint32_t)(ri % nl);
      xoff = loff[l];
      n = loff[l + 1] - xoff;
      k = lk[l];
      koff = lkoff[l];
      base = (uint64_t)p * N + xoff;
    }
    const RowSize z = row_size(base, n, k, true);
    uint64_t t;
    const uint64_t cand = c_cand + block_exclusive_scan_u64<1024>(in ? (uint64_t)z.nsub * z.capS : 0, scr, t);
    c_cand += t;
    const uint64_t tile0 = c_tiles + block_exclusive_scan_u64<1024>(in ? z.nt : 0, scr, t);
    c_tiles += t;
    const uint64_t group0 = c_groups + block_exclusive_scan_u64<1024>(in ? z.groups : 0, scr, t);
    c_groups += t;
    const uint64_t chunk0 = c_chunks + block_exclusive_scan_u64<1024>(in ? z.chunks : 0, scr, t);
    c_chunks += t;
    const uint64_t pass0 = c_pass + block_exclusive_scan_u64<1024>(in ? z.npass : 0, scr, t);
    c_pass += t;
    const bool big = in && big_predict(n, k, z.schunks);
    const uint64_t big0 = c_big + block_exclusive_scan_u64<1024>(big ? 1 : 0, scr, t);
    c_big += t;
    if (big) big_rows[big0] = (uint32_t)ri;
    const bool sampled = in && layer_sampled(n, k) && !big;
    const uint64_t mid0 = c_mid + block_exclusive_scan_u64<1024>(sampled ? 1 : 0, scr, t);
    c_mid += t;
    if (sampled) mid_rows[mid0] = (uint32_t)ri;
    if (in) {
      Row R{};
      R.base = base;
      R.cand = cand;
      R.tile0 = tile0;
      R.group0 = group0;
      R.chunk0 = chunk0;
      R.out0 = (uint64_t)p * K + koff;
      R.n = (uint32_t)n;
      R.k = (uint32_t)k;
      R.capS = (uint32_t)z.capS;
      R.nsub = z.nsub;
      R.tps_log = z.tps_log;
      const uint64_t S = (uint64_t)z.schunks * kSampleChunk;
      if (n <= S) {
        R.rs_lo = R.rs_mid = (uint32_t)k;
      } else {
        const double qs = (double)k / (double)n * (double)S;
        R.rs_lo = (uint32_t)fmin(ceil(qs + 4.0 * sqrt(qs) + 16.0), (double)S);
        R.rs_mid = (uint32_t)fmin(fmax(1.0, ceil(qs)), (double)S);
      }
      R.idx_off = (uint32_t)xoff;
      R.schunks = z.schunks;
      R.pass0 = (uint32_t)pass0;
      R.npass = z.npass;
      rows[ri] = R;
    }
  }
}

// The same table where every node's layer l starts at the same tile phase
// (N a multiple of kTileAlign) and there are at most 1024 layers: all nodes'
// rows then have one node's sizes, so a single scan over the layers gives
// each layer's offsets inside a node and the node's totals, and row
// p * nl + l is p times the totals plus layer l's offsets (k_rows_plan's
// scans over every row took 102 us for 64 nodes of 160 layers).
__global__ __launch_bounds__(1024) void k_rows_plan_nodes(Row* rows, uint32_t* big_rows, uint32_t* mid_rows,
                                                          const uint64_t* loff, const uint64_t* lk,
                                                          const uint64_t* lkoff, uint32_t P, uint64_t N, uint32_t nl,
                                                          uint64_t K) {
  __shared__ uint64_t scr[1024 / kWave + 1];
  __shared__ uint64_t s_cand[1024];
  __shared__ uint32_t s_tile[1024], s_group[1024], s_chunk[1024], s_pass[1024], s_big[1024], s_mid[1024];
  __shared__ uint32_t s_capS[1024], s_rslo[1024], s_rsmid[1024], s_misc[1024];
  __shared__ uint64_t s_tot[7];
  const uint32_t l = threadIdx.x;
  const bool in = l < nl;
  uint64_t n = 0, k = 0, xoff = 0;
  if (in) {
    xoff = loff[l];
    n = loff[l + 1] - xoff;
    k = lk[l];
  }
  const RowSize z = row_size(xoff, n, k, true);  // node p's layer: base p * N + xoff, the same phase
  const bool big = in && big_predict(n, k, z.schunks);
  const bool sampled = in && layer_sampled(n, k) && !big;
  uint64_t t;
  const uint64_t cand = block_exclusive_scan_u64<1024>(in ? (uint64_t)z.nsub * z.capS : 0, scr, t);
  if (l == 0) s_tot[0] = t;
  const uint64_t tile = block_exclusive_scan_u64<1024>(in ? z.nt : 0, scr, t);
  if (l == 0) s_tot[1] = t;
  const uint64_t group = block_exclusive_scan_u64<1024>(in ? z.groups : 0, scr, t);
  if (l == 0) s_tot[2] = t;
  const uint64_t chunk = block_exclusive_scan_u64<1024>(in ? z.chunks : 0, scr, t);
  if (l == 0) s_tot[3] = t;
  const uint64_t pass = block_exclusive_scan_u64<1024>(in ? z.npass : 0, scr, t);
  if (l == 0) s_tot[4] = t;
  const uint64_t nbig = block_exclusive_scan_u64<1024>(big ? 1 : 0, scr, t);
  if (l == 0) s_tot[5] = t;
  const uint64_t nmid = block_exclusive_scan_u64<1024>(sampled ? 1 : 0, scr, t);
  if (l == 0) s_tot[6] = t;
  s_cand[l] = cand;
  // within a node these fit 32 bits: tiles, groups, chunks and blocks are
  // at most a node's elements over 1024, 262144, 4096 and 8192
  s_tile[l] = (uint32_t)tile;
  s_group[l] = (uint32_t)group;
  s_chunk[l] = (uint32_t)chunk;
  s_pass[l] = (uint32_t)pass;
  s_big[l] = (uint32_t)nbig;
  s_mid[l] = (uint32_t)nmid;
  const uint64_t S = (uint64_t)z.schunks * kSampleChunk;
  if (n <= S) {
    s_rslo[l] = s_rsmid[l] = (uint32_t)k;
  } else {
    const double qs = (double)k / (double)n * (double)S;
    s_rslo[l] = (uint32_t)fmin(ceil(qs + 4.0 * sqrt(qs) + 16.0), (double)S);
    s_rsmid[l] = (uint32_t)fmin(fmax(1.0, ceil(qs)), (double)S);
  }
  s_capS[l] = (uint32_t)z.capS;
  // counter regions (<= 256), log2 of tiles per counter (<= 4), the two row
  // lists, sample chunks (<= 512) and blocks per pass (<= 64)
  s_misc[l] = z.nsub | z.tps_log << 9 | (big ? 1u : 0u) << 12 | (sampled ? 1u : 0u) << 13 | z.schunks << 14 |
              z.npass << 24;
  __syncthreads();
  const uint64_t nrows = (uint64_t)P * nl;
  for (uint64_t ri = threadIdx.x; ri < nrows; ri += 1024) {
    const uint64_t p = ri / nl;
    const uint32_t ll = (uint32_t)(ri % nl);
    const uint32_t misc = s_misc[ll];
    const uint64_t xo = loff[ll];
    Row R{};
    R.base = p * N + xo;
    R.cand = p * s_tot[0] + s_cand[ll];
    R.tile0 = p * s_tot[1] + s_tile[ll];
    R.group0 = p * s_tot[2] + s_group[ll];
    R.chunk0 = p * s_tot[3] + s_chunk[ll];
    R.out0 = p * K + lkoff[ll];
    R.n = (uint32_t)(loff[ll + 1] - xo);
    R.k = (uint32_t)lk[ll];
    R.capS = s_capS[ll];
    R.nsub = misc & 511u;
    R.tps_log = (misc >> 9) & 7u;
    R.rs_lo = s_rslo[ll];
    R.rs_mid = s_rsmid[ll];
    R.idx_off = (uint32_t)xo;
    R.schunks = (misc >> 14) & 1023u;
    R.pass0 = (uint32_t)(p * s_tot[4] + s_pass[ll]);
    R.npass = misc >> 24;
    rows[ri] = R;
    if ((misc >> 12) & 1u) big_rows[p * s_tot[5] + s_big[ll]] = (uint32_t)ri;
    if ((misc >> 13) & 1u) mid_rows[p * s_tot[6] + s_mid[ll]] = (uint32_t)ri;
  }
}

// block-to-row tables of the per-layer grids; each row reset for the call
__global__ __launch_bounds__(256) void k_tile_rows(const Row* rows, uint32_t* tile_row, uint32_t* group_row,
                                                   uint32_t* pass_row, Dev D) {
  const uint32_t p = blockIdx.x;
  const Row R = rows[p];
  // every row reset here; the rows that need no sample get their thresholds
  reset_row<256, true>(D, p, R);
  uint32_t lo, mid;
  if (threadIdx.x == 0 && fixed_thresholds(R, true, lo, mid)) set_state(D, p, lo, mid);
  const uint32_t nt = row_tiles(R);
  for (uint32_t t = threadIdx.x; t < nt; t += 256) tile_row[R.tile0 + t] = p;
  const uint32_t ng = (nt + kGroup - 1) / kGroup;
  for (uint32_t t = threadIdx.x; t < ng; t += 256) group_row[R.group0 + t] = p;
  for (uint32_t t = threadIdx.x; t < R.npass; t += 256) pass_row[R.pass0 + t] = p;
}

// The launch sequence shared by both calls. nrows rows; the stream grid has
// one workgroup per tile slot; `tile_slots`, `groups`, `max_cap` size the
// other grids.
template <bool ROWS>
hipError_t run(const Dev& D, uint64_t nrows, uint64_t stream_blocks, uint64_t groups, uint64_t max_tiles,
               uint64_t max_cap, uint64_t passes, uint64_t big_rows, uint64_t mid_rows, bool any_k, const float* grad,
               float* residual,
               uint32_t* out_idx, float* out_val, hipStream_t stream, const OpEvents* ev) {
  const uint32_t R = (uint32_t)nrows;
  // measurement events (whole-vector call only): the op's span runs from the
  // predictor's dispatch to the last kernel's, the stream kernel's own pair
  // times it alone
  const OpEvents none{};
  const OpEvents& E = ev ? *ev : none;
  hipError_t e = hipSuccess;
  if constexpr (ROWS) {
    if (mid_rows > 0)
      hipLaunchKernelGGL((k_predict<true, kSmallPredictThreads, 1>), dim3((uint32_t)mid_rows),
                         dim3(kSmallPredictThreads), 0, stream, grad, residual, D);
    if (big_rows > 0)
      hipLaunchKernelGGL((k_predict<true, kLayerPredictThreads, 2>), dim3((uint32_t)big_rows),
                         dim3(kLayerPredictThreads), 0, stream, grad, residual, D);
  } else {
    const bool predict_last = stream_blocks == 0 && !any_k;
    e = launch_ev(k_predict<false, kPredictThreads, 0>, dim3(R), dim3(kPredictThreads), stream, E.op_start,
                  predict_last ? E.op_stop : nullptr, grad, residual, D);
  }
  if (e == hipSuccess && stream_blocks > 0) {
    if (E.k_start || E.k_stop || (!any_k && E.op_stop)) {
      // the stream kernel carries one start and one stop event: its own pair,
      // or the op's stop when it is the op's last kernel and its pair is unused
      const hipEvent_t s0 = E.k_start;
      const hipEvent_t s1 = E.k_stop ? E.k_stop : (!any_k ? E.op_stop : nullptr);
      e = launch_ev(k_stream<ROWS>, dim3((uint32_t)stream_blocks), dim3(kStreamThreads), stream, s0, s1, grad,
                    residual, D);
      if (e == hipSuccess && !any_k && E.k_stop && E.op_stop) e = hipEventRecord(E.op_stop, stream);
    } else {
      hipLaunchKernelGGL(k_stream<ROWS>, dim3((uint32_t)stream_blocks), dim3(kStreamThreads), 0, stream, grad,
                         residual, D);
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess || !any_k) return e;

  // select / count / emit passes: enough blocks to fill the chip once, each
  // looping over several chunks, so the per-block digit decisions are
  // amortised; the rescan path loops over more work with the same grids
  const uint64_t pass_row = std::max<uint64_t>(1, 2048 / nrows);
  const uint32_t hist_blocks =
      (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((max_cap + 16383) / 16384, pass_row));
  const uint32_t chunk_blocks =
      (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>((max_cap + kChunk - 1) / kChunk, pass_row));
  // per-layer call: 1D grids over all groups / all pass blocks of all rows
  const dim3 gG = ROWS ? dim3((uint32_t)groups) : dim3((uint32_t)std::max<uint64_t>(1, groups), R);
  const dim3 gH = ROWS ? dim3((uint32_t)passes) : dim3(hist_blocks, R);
  const dim3 gC = ROWS ? dim3((uint32_t)passes) : dim3(chunk_blocks, R);
  if (ROWS && groups > 0) hipLaunchKernelGGL(k_tsum<ROWS>, gG, dim3(256), 0, stream, D);
  if (!ROWS) hipLaunchKernelGGL(k_tsum<ROWS>, gG, dim3(256), 0, stream, D);
  hipLaunchKernelGGL(k_gscan<ROWS>, dim3(R), dim3(1024), 0, stream, D);
  if (!ROWS || groups > 0) hipLaunchKernelGGL(k_gather<ROWS>, gG, dim3(kGroup), 0, stream, residual, D);
  hipLaunchKernelGGL((k_hist<0, ROWS>), gH, dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL((k_hist<1, ROWS>), gH, dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL((k_hist<2, ROWS>), gH, dim3(256), 0, stream, residual, D);
  hipLaunchKernelGGL(k_count<ROWS>, gC, dim3(kChunkThreads), 0, stream, residual, D);
  hipLaunchKernelGGL(k_scan<ROWS>, dim3(R), dim3(1024), 0, stream, D);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!ROWS && D.runs != nullptr)
    return launch_ev(k_emit<false, true, kEmitIt>, gC, dim3(kChunk / kEmitIt), stream, nullptr, E.op_stop, residual,
                     out_idx, out_val, D);
  return launch_ev(k_emit<ROWS, false, kEmitIt>, gC, dim3(kChunk / kEmitIt), stream, nullptr, E.op_stop, residual,
                   out_idx, out_val, D);
}

// Run table of a finished [P][k] output, by the emit pass's rule applied to
// the output pairs themselves (pair j writes the entries s with
// idx[j-1] < s * 4096 <= idx[j]): for calls where no emit pass runs (rows
// selected by one workgroup each, and k == 0, where every run is empty).
__global__ __launch_bounds__(256) void k_runs_of_output(const uint32_t* __restrict__ out_idx, uint32_t* runs,
                                                        uint32_t k, uint32_t S) {
  const uint32_t p = blockIdx.y;
  uint32_t* tab = runs + (uint64_t)p * (S + 1);
  const uint32_t base = p * k;  // the host checks P * k < 2^32
  const uint32_t stride = gridDim.x * 256;
  if (k == 0) {
    for (uint32_t s = blockIdx.x * 256 + threadIdx.x; s <= S; s += stride) tab[s] = base;
    return;
  }
  for (uint32_t j = blockIdx.x * 256 + threadIdx.x; j < k; j += stride) {
    const uint32_t s_hi = out_idx[base + j] >> kSegmentBits;
    for (uint32_t s = j ? (out_idx[base + j - 1] >> kSegmentBits) + 1u : 0u; s <= s_hi; ++s) tab[s] = base + j;
    if (j == k - 1)
      for (uint32_t s = s_hi + 1u; s <= S; ++s) tab[s] = base + k;
  }
}

Dev make_dev(const Layout& L, char* w, uint32_t P) {
  Dev D{};
  D.P = P;
  D.capS = L.capS;
  D.cap = L.cap;
  D.tps_log = L.tps_log;
  D.MT = L.MT;
  D.MG = L.MG;
  D.MC = L.MC;
  D.info = reinterpret_cast<uint32_t*>(w + L.info);
  D.err = reinterpret_cast<uint32_t*>(w + L.err);
  D.state = reinterpret_cast<NodeState*>(w + L.state);
  D.h0 = reinterpret_cast<uint32_t*>(w + L.h0);
  D.h1 = reinterpret_cast<uint32_t*>(w + L.h1);
  D.h2 = reinterpret_cast<uint32_t*>(w + L.h2);
  D.h1s = reinterpret_cast<uint32_t*>(w + L.h1s);
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
  D.cdig = reinterpret_cast<uint16_t*>(w + L.cdig);
  D.rows = nullptr;
  D.tile_row = nullptr;
  return D;
}

}  // namespace

size_t topk_workspace_bytes(uint32_t P, uint64_t N, uint64_t k) { return make_node_layout(P, N, k).total; }

hipError_t topk_runs_of_output_launch(uint32_t P, uint64_t N, uint64_t k, const uint32_t* out_idx, uint32_t* runs,
                                      hipStream_t stream) {
  const uint32_t S = (uint32_t)((N + SPARCML_SEGMENT - 1) / SPARCML_SEGMENT);
  const uint64_t work = std::max<uint64_t>(k, (uint64_t)S + 1);
  const uint32_t bx = (uint32_t)std::min<uint64_t>((work + 255) / 256, 64);
  hipLaunchKernelGGL(k_runs_of_output, dim3(bx, P), dim3(256), 0, stream, out_idx, runs, (uint32_t)k, S);
  return hipGetLastError();
}

hipError_t topk_ef_launch(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                          uint32_t* out_idx, float* out_val, uint32_t* runs, void* ws, hipStream_t stream,
                          const OpEvents* ev) {
  const Layout L = make_node_layout(P, N, k);
  Dev D = make_dev(L, static_cast<char*>(ws), P);
  D.N = (uint32_t)N;
  D.k = (uint32_t)k;
  D.runs = k > 0 ? runs : nullptr;
  D.S = (uint32_t)((N + SPARCML_SEGMENT - 1) / SPARCML_SEGMENT);
  if (N <= (uint64_t)kSample) {
    D.rs_lo = D.rs_mid = (uint32_t)k;
  } else {
    const double qs = (double)k / (double)N * kSample;
    D.rs_lo = (uint32_t)std::min<double>(std::ceil(qs + 4.0 * std::sqrt(qs) + 16.0), (double)kSample);
    D.rs_mid = (uint32_t)std::min<double>(std::max<double>(1.0, std::ceil(qs)), (double)kSample);
  }
  const hipError_t e =
      run<false>(D, P, L.MT * P, L.MG, L.MT, L.cap, 0, 0, 0, k > 0, grad, residual, out_idx, out_val, stream, ev);
  // with k == 0 no emit pass runs: every run is empty
  if (e == hipSuccess && runs != nullptr && k == 0) return topk_runs_of_output_launch(P, N, 0, out_idx, runs, stream);
  return e;
}

size_t topk_layers_workspace_bytes(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k) {
  const LayerPlan lp = plan_layers(P, N, nl, off, k);
  return make_layout(lp.Q, nl).total;
}

uint64_t topk_layers_stream_blocks(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k) {
  return plan_layers(P, N, nl, off, k).Q.tiles;
}

hipError_t topk_layers_launch(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k,
                              const float* grad, float* residual, uint32_t* out_idx, float* out_val, void* ws,
                              hipStream_t stream) {
  const LayerPlan lp = plan_layers(P, N, nl, off, k);
  const Layout L = make_layout(lp.Q, nl);
  char* w = static_cast<char*>(ws);
  Dev D = make_dev(L, w, (uint32_t)lp.Q.rows);
  Row* rows = reinterpret_cast<Row*>(w + L.rows);
  uint32_t* tile_row = reinterpret_cast<uint32_t*>(w + L.tile_row);
  uint64_t* loff = reinterpret_cast<uint64_t*>(w + L.loff);
  uint64_t* lk = reinterpret_cast<uint64_t*>(w + L.lk);
  uint32_t* group_row = reinterpret_cast<uint32_t*>(w + L.group_row);
  uint32_t* pass_row = reinterpret_cast<uint32_t*>(w + L.pass_row);
  uint64_t* lkoff = reinterpret_cast<uint64_t*>(w + L.lkoff);
  uint32_t* big_rows = reinterpret_cast<uint32_t*>(w + L.big_rows);
  uint32_t* mid_rows = reinterpret_cast<uint32_t*>(w + L.mid_rows);
  D.big_rows = big_rows;
  D.mid_rows = mid_rows;
  D.rows = rows;
  D.tile_row = tile_row;
  D.group_row = group_row;
  D.pass_row = pass_row;
  uint64_t koff = 0;
  for (uint32_t first = 0; first < nl; first += kLayersPerSetup) {
    LayerChunk in{};
    const uint32_t count = std::min<uint32_t>(kLayersPerSetup, nl - first);
    for (uint32_t i = 0; i < count; ++i) {
      in.off[i] = off[first + i];
      in.k[i] = k[first + i];
      in.koff[i] = koff;
      koff += k[first + i];
    }
    in.off[count] = off[first + count];
    hipLaunchKernelGGL(k_layers_in, dim3(1), dim3(128), 0, stream, loff, lk, lkoff, first, count, in);
  }
  if (N % kTileAlign == 0 && nl <= 1024)
    hipLaunchKernelGGL(k_rows_plan_nodes, dim3(1), dim3(1024), 0, stream, rows, big_rows, mid_rows, loff, lk, lkoff,
                       P, N, nl, lp.K);
  else
    hipLaunchKernelGGL(k_rows_plan, dim3(1), dim3(1024), 0, stream, rows, big_rows, mid_rows, loff, lk, lkoff, P, N,
                       nl, lp.K);
  hipLaunchKernelGGL(k_tile_rows, dim3((uint32_t)lp.Q.rows), dim3(256), 0, stream, rows, tile_row, group_row,
                     pass_row, D);
  return run<true>(D, lp.Q.rows, lp.Q.tiles, lp.Q.groups, lp.max_tiles, lp.max_cap, lp.Q.passes, lp.Q.big, lp.Q.mid,
                   lp.K > 0,
                   grad, residual, out_idx, out_val, stream, nullptr);
}

}  // namespace sparcml
