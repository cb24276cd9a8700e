// Plain CPU oracle for the SparCML data-parallel hot path.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
// calls this file; only the test suite, the smoke check and the bench's CPU
// baseline do. It shares no code, header, table or constant with the HIP
// kernels under sparse_gradient_reduction_amd/csrc.
//
// Sources (cited by page title and section):
//   [SparCML] "SparCML: High-Performance Sparse Communication for Machine
//             Learning", paperlayer.ai digest of arXiv 1802.08021v3.
//   [Philox]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
//             as 1, 2, 3", SC'11, Philox-4x32 round and key schedule.
//
// Every function below computes the plain definition of its step, not a fast
// algorithm: a full ordering for Top-k, a dense fp64 accumulator for the
// reduction, one Philox block per group of four positions for the quantizer.
// Parity status of each function is stated in its header comment.
//
// Build: g++ -O2 -std=c++17 -fopenmp -ffp-contract=off -fPIC -shared
// (no -ffast-math, no FMA contraction, gradual underflow kept).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include <omp.h>

extern "C" {

// Threads an OpenMP region of the oracle may use (reported with CPU timings).
int oracle_max_threads(void) { return omp_get_max_threads(); }

// ---------------------------------------------------------------------------
// Error-feedback Top-k  ([SparCML] §2.2 "Communication-Reduction Techniques":
// each node sends its k largest-magnitude components and keeps the rest for
// the next iteration; §4 "Sparse Quantized Reduction": the unapplied part is
// carried forward as residual error).
//
// Per node p (node-major [P][N] arrays):
//   a_i   = fl32(g_i + r_i)                    (one IEEE single add)
//   key_i = bits(a_i) & 0x7FFFFFFF             (orders |a_i|, -0 ties +0)
//   S     = the first k positions under the total order
//           (key descending, index ascending)  (ties go to the lower index)
//   out_idx = S ascending, out_val = a[S]
//   r_new   = a, then r_new[S] = +0.0
// Pinned by: brute force with numpy lexsort, the pairwise characterisation
// of S, the all-equal / k=0 / k=N special cases and the exact identity
// r_new + scatter(out_val) == fl32(g + r_old).
// ---------------------------------------------------------------------------
static inline uint32_t mag_key(float a) {
  uint32_t b;
  std::memcpy(&b, &a, 4);
  return b & 0x7FFFFFFFu;
}

void oracle_topk_ef(uint32_t P, uint64_t N, uint64_t k, const float* grad,
                    float* residual, uint32_t* out_idx, float* out_val) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < (int64_t)P; ++p) {
    const float* g = grad + (uint64_t)p * N;
    float* r = residual + (uint64_t)p * N;
    std::vector<float> a(N);
    for (uint64_t i = 0; i < N; ++i) a[i] = g[i] + r[i];

    std::vector<uint32_t> order(N);
    for (uint64_t i = 0; i < N; ++i) order[i] = (uint32_t)i;
    auto before = [&](uint32_t x, uint32_t y) {
      uint32_t kx = mag_key(a[x]), ky = mag_key(a[y]);
      if (kx != ky) return kx > ky;
      return x < y;
    };
    if (k > 0 && k < N) std::nth_element(order.begin(), order.begin() + k, order.end(), before);
    std::vector<uint32_t> sel(order.begin(), order.begin() + k);
    std::sort(sel.begin(), sel.end());

    for (uint64_t i = 0; i < N; ++i) r[i] = a[i];
    for (uint64_t j = 0; j < k; ++j) {
      out_idx[(uint64_t)p * k + j] = sel[j];
      out_val[(uint64_t)p * k + j] = a[sel[j]];
      r[sel[j]] = +0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Per-layer error-feedback Top-k ([SparCML] §8.4: the ResNet50 runs sparsify
// each layer; §2.2 and §4 as above).
//
// Every node's vector is cut into layers [off[l], off[l+1]); oracle_topk_ef's
// selection runs on each layer of each node by itself, keeping k[l]
// positions. Node p's output row is the concatenation over layers of each
// layer's selection (node-relative indices, ascending), so it is ascending;
// layer l starts at sum_{l'<l} k[l']. The residual is a with +0 at every
// kept position.
// Pinned by: brute force with numpy lexsort per layer, the one-layer case
// that is oracle_topk_ef itself, and the exact EF identity.
// ---------------------------------------------------------------------------
void oracle_topk_ef_layers(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k,
                           const float* grad, float* residual, uint32_t* out_idx, float* out_val) {
  uint64_t K = 0;
  for (uint32_t l = 0; l < nl; ++l) K += k[l];
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < (int64_t)P; ++p) {
    const float* g = grad + (uint64_t)p * N;
    float* r = residual + (uint64_t)p * N;
    std::vector<float> a(N);
    for (uint64_t i = 0; i < N; ++i) a[i] = g[i] + r[i];
    for (uint64_t i = 0; i < N; ++i) r[i] = a[i];
    auto before = [&](uint32_t x, uint32_t y) {
      uint32_t kx = mag_key(a[x]), ky = mag_key(a[y]);
      if (kx != ky) return kx > ky;
      return x < y;
    };
    uint64_t o = (uint64_t)p * K;
    for (uint32_t l = 0; l < nl; ++l) {
      std::vector<uint32_t> order;
      for (uint64_t i = off[l]; i < off[l + 1]; ++i) order.push_back((uint32_t)i);
      const uint64_t kl = k[l];
      if (kl > 0 && kl < order.size()) std::nth_element(order.begin(), order.begin() + kl, order.end(), before);
      std::vector<uint32_t> sel(order.begin(), order.begin() + kl);
      std::sort(sel.begin(), sel.end());
      for (uint64_t t = 0; t < kl; ++t, ++o) {
        out_idx[o] = sel[t];
        out_val[o] = a[sel[t]];
        r[sel[t]] = +0.0f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Bucketed error-feedback Top-k ([SparCML] §8.3: the CIFAR-10 runs keep k
// entries out of every 512, e.g. 16/512; §2.2 and §4 as above for the
// selection rule and the residual).
//
// Reading used here: per node, the N positions form buckets of `bucket`
// consecutive positions (the last one partial, restarting per node, as the
// quantizer's buckets do). Bucket j with len_j positions keeps
// k_j = min(k_per_bucket, len_j) of them, chosen exactly as oracle_topk_ef
// chooses within the bucket (key descending, index ascending). The node's
// output is the concatenation over buckets of each bucket's selection in
// ascending index order, so it is ascending overall; bucket j's pairs start
// at j * min(k_per_bucket, bucket), and a node has K = sum_j k_j pairs (rows
// of K).
// The residual is a with +0 at every selected position.
// Pinned by: brute force per bucket with numpy lexsort, the bucket >= N case
// that is oracle_topk_ef itself, and the exact EF identity.
// ---------------------------------------------------------------------------
uint64_t oracle_bucketed_count(uint64_t N, uint32_t bucket, uint32_t kb) {
  if (N == 0) return 0;
  const uint64_t nb = (N + bucket - 1) / bucket;
  const uint64_t last = N - (nb - 1) * bucket;
  return (nb - 1) * (uint64_t)std::min<uint64_t>(kb, bucket) + std::min<uint64_t>(kb, last);
}

void oracle_topk_ef_bucketed(uint32_t P, uint64_t N, uint32_t bucket, uint32_t kb, const float* grad,
                             float* residual, uint32_t* out_idx, float* out_val) {
  const uint64_t K = oracle_bucketed_count(N, bucket, kb);
  const uint64_t nb = (N + bucket - 1) / bucket;
  const uint64_t kfull = std::min<uint64_t>(kb, bucket);  // pairs of a whole bucket
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < (int64_t)P; ++p) {
    const float* g = grad + (uint64_t)p * N;
    float* r = residual + (uint64_t)p * N;
    std::vector<float> a(N);
    for (uint64_t i = 0; i < N; ++i) a[i] = g[i] + r[i];
    for (uint64_t i = 0; i < N; ++i) r[i] = a[i];
    auto before = [&](uint32_t x, uint32_t y) {
      uint32_t kx = mag_key(a[x]), ky = mag_key(a[y]);
      if (kx != ky) return kx > ky;
      return x < y;
    };
    for (uint64_t j = 0; j < nb; ++j) {
      const uint64_t lo = j * bucket, hi = std::min<uint64_t>(lo + bucket, N);
      const uint64_t kj = std::min<uint64_t>(kb, hi - lo);
      std::vector<uint32_t> order;
      for (uint64_t i = lo; i < hi; ++i) order.push_back((uint32_t)i);
      if (kj > 0 && kj < order.size())
        std::nth_element(order.begin(), order.begin() + kj, order.end(), before);
      std::vector<uint32_t> sel(order.begin(), order.begin() + kj);
      std::sort(sel.begin(), sel.end());
      for (uint64_t t = 0; t < kj; ++t) {
        const uint64_t o = (uint64_t)p * K + j * kfull + t;
        out_idx[o] = sel[t];
        out_val[o] = a[sel[t]];
        r[sel[t]] = +0.0f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Philox-4x32-10 block function, written from [Philox] (SC'11): four 32-bit
// counter words, two 32-bit key words; each round multiplies counter words 0
// and 2 by the two Philox-4x32 multipliers into 64-bit products, and builds
// the next counter from the high halves xor-ed with the other counter words
// and the round key, and the low halves; the key is bumped by the two Weyl
// constants (golden ratio and sqrt(3)-1, scaled to 32 bits) between rounds.
// Pinned by: comparison with rocRAND's host-callable Philox-4x32-10 engine.
// ---------------------------------------------------------------------------
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  const uint32_t MUL_A = 0xD2511F53u, MUL_B = 0xCD9E8D57u;
  const uint32_t WEYL_A = 0x9E3779B9u, WEYL_B = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += WEYL_A;
      k1 += WEYL_B;
    }
    uint64_t prod_a = (uint64_t)MUL_A * c0;
    uint64_t prod_b = (uint64_t)MUL_B * c2;
    uint32_t hi_a = (uint32_t)(prod_a >> 32), lo_a = (uint32_t)prod_a;
    uint32_t hi_b = (uint32_t)(prod_b >> 32), lo_b = (uint32_t)prod_b;
    uint32_t n0 = hi_b ^ c1 ^ k0;
    uint32_t n1 = lo_b;
    uint32_t n2 = hi_a ^ c3 ^ k1;
    uint32_t n3 = lo_a;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// ---------------------------------------------------------------------------
// b-bit stochastic quantization, b in {2, 4, 8} ([SparCML] §6 "Supporting
// Low-Precision Communication": QSGD quantizes buckets independently and
// stochastically, each with one full-precision scale, with 2-, 4- and 8-bit
// outputs; §2.2: the quantization noise is zero-mean; §4: the reduced dense
// vector may itself be quantized).
//
// Reading used here (the digest gives no formula): a code is a sign bit over
// b-1 magnitude bits, so there are s = 2^(b-1) - 1 nonzero levels (1, 7,
// 127). Per row r (node node0 + r), the n values in their given order form
// buckets of `bucket` consecutive positions, the last one partial. For
// bucket j:
//   scale = max |v| over the bucket (exact), st = fl32(scale / s)
// For position e with value v:
//   scale == 0 -> level 0
//   else x = fl32(fl32(|v| / scale) * s), l = floor(x), f = x - l (exact),
//        w = word (e & 3) of Philox4x32-10(counter {e>>2, node0 + r, step, 0},
//                                          key {lo32(seed), hi32(seed)}),
//        u = (w >> 8) * 2^-24, level = l + (u < f)
//   code = ((v < 0) << (b-1)) | level
// Codes are packed 8/b to a byte, position e at bit (e mod 8/b) * b of byte
// e*b/8 (lowest position in the lowest bits); rows are ceil(n*b/8) bytes and
// unused bits are zero. The 4-bit case is the format used on the sent values.
// Parity: codes pinned by the level/sign invariants, the unbiasedness of the
// dequantized values over many seeds and a recomputation from rocRAND's
// Philox stream; beyond those the code stream is fixed by this reading, not
// by the pages.
// ---------------------------------------------------------------------------
static uint32_t qsgd_levels(uint32_t bits) { return (1u << (bits - 1)) - 1u; }

void oracle_qsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
                 uint32_t node0, const float* val, uint8_t* codes, float* scales) {
  const uint32_t s = qsgd_levels(bits);
  const float sf = (float)s;
  const uint64_t per_byte = 8 / bits;
  const uint64_t row_bytes = (n * bits + 7) / 8;
  const uint64_t nbuckets = (n + bucket - 1) / bucket;
  const uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < (int64_t)P; ++r) {
    const uint32_t node = node0 + (uint32_t)r;
    const float* v = val + (uint64_t)r * n;
    uint8_t* row = codes + (uint64_t)r * row_bytes;
    std::memset(row, 0, row_bytes);
    for (uint64_t j = 0; j < nbuckets; ++j) {
      uint64_t lo = j * bucket, hi = std::min<uint64_t>(lo + bucket, n);
      float scale = 0.0f;
      for (uint64_t e = lo; e < hi; ++e) scale = std::max(scale, std::fabs(v[e]));
      scales[(uint64_t)r * nbuckets + j] = scale;
      for (uint64_t e = lo; e < hi; ++e) {
        uint32_t level = 0;
        if (scale != 0.0f) {
          float ratio = std::fabs(v[e]) / scale;
          float x = ratio * sf;
          float l = std::floor(x);
          float f = x - l;
          uint32_t ctr[4] = {(uint32_t)(e >> 2), node, step, 0u};
          uint32_t w[4];
          oracle_philox4x32_10(ctr, key, w);
          float u = (float)(w[e & 3] >> 8) * (1.0f / 16777216.0f);
          level = (uint32_t)l + (u < f ? 1u : 0u);
        }
        uint32_t code = ((v[e] < 0.0f) ? (1u << (bits - 1)) : 0u) | level;
        row[e / per_byte] |= (uint8_t)(code << ((e % per_byte) * bits));
      }
    }
  }
}

// Inverse of oracle_qsgd: val = (sign ? -1 : +1) * fl32(level * fl32(scale / s)).
void oracle_dqsgd(uint32_t bits, uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                  const float* scales, float* val) {
  const uint32_t s = qsgd_levels(bits);
  const uint64_t per_byte = 8 / bits;
  const uint64_t row_bytes = (n * bits + 7) / 8;
  const uint64_t nbuckets = (n + bucket - 1) / bucket;
  const uint32_t mask = (1u << bits) - 1u;
  for (uint64_t p = 0; p < P; ++p) {
    for (uint64_t e = 0; e < n; ++e) {
      uint8_t byte = codes[p * row_bytes + e / per_byte];
      uint32_t code = (byte >> ((e % per_byte) * bits)) & mask;
      float st = scales[p * nbuckets + e / bucket] / (float)s;
      float mag = (float)(code & s) * st;
      val[p * n + e] = (code >> (bits - 1)) ? -mag : mag;
    }
  }
}

// The 4-bit format on node rows 0..P-1.
void oracle_q4(uint32_t P, uint64_t n, uint32_t bucket, uint64_t seed, uint32_t step,
               const float* val, uint8_t* codes, float* scales) {
  oracle_qsgd(4, P, n, bucket, seed, step, 0u, val, codes, scales);
}

void oracle_dq4(uint32_t P, uint64_t n, uint32_t bucket, const uint8_t* codes,
                const float* scales, float* val) {
  oracle_dqsgd(4, P, n, bucket, codes, scales, val);
}

// ---------------------------------------------------------------------------
// Sparse reduction with the dense switch ([SparCML] §5.1 "Sparse Streams":
// index-value pairs that turn dense once fill-in makes them wasteful, at a
// threshold delta; §5.2: sum with neutral element 0; §5.3: dense when the
// result size K reaches delta; App. B: the result's nonzero count is the
// number of indices in the union of the contributed index sets).
//
//   acc[N] (fp64) = 0, occ[N] = 0
//   for every pair (i, v) of every node: acc[i] += v, occ[i] = 1
//   K = sum occ  (structural: an index counts even if its sum is 0)
//   T = ceil(delta * N) in double
//   K >= T -> dense:  out_val[i] = fl32(acc[i]) for all i < N
//   else   -> sparse: (i, fl32(acc[i])) for occ[i] = 1, ascending i
// Any index >= N is reported through the return value (-1) and nothing is
// written; duplicates within a node are simply summed.
// Pinned by: np.bincount / np.unique on random inputs, full-overlap and
// disjoint cases (App. B's tight union bound), and unions of T-1, T, T+1.
// ---------------------------------------------------------------------------
int oracle_reduce(uint32_t P, uint64_t N, double delta, const uint64_t* offsets,
                  const uint32_t* idx, const float* val, uint64_t* nnz_out,
                  uint32_t* is_dense_out, uint32_t* out_idx, float* out_val) {
  std::vector<double> acc(N, 0.0);
  std::vector<uint8_t> occ(N, 0);
  for (uint64_t p = 0; p < P; ++p) {
    for (uint64_t e = offsets[p]; e < offsets[p + 1]; ++e) {
      if ((uint64_t)idx[e] >= N) return -1;
      acc[idx[e]] += (double)val[e];
      occ[idx[e]] = 1;
    }
  }
  uint64_t K = 0;
  for (uint64_t i = 0; i < N; ++i) K += occ[i];
  double T = std::ceil(delta * (double)N);
  bool dense = (double)K >= T;
  *nnz_out = K;
  *is_dense_out = dense ? 1u : 0u;
  if (dense) {
    for (uint64_t i = 0; i < N; ++i) out_val[i] = (float)acc[i];
  } else {
    uint64_t j = 0;
    for (uint64_t i = 0; i < N; ++i) {
      if (occ[i]) {
        out_idx[j] = (uint32_t)i;
        out_val[j] = (float)acc[i];
        ++j;
      }
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Run table of sorted sparse contributions ([SparCML] §5.3.2: the split phase
// gives each owner one range of indices, and each node hands it the part of
// its sorted pairs that falls in that range).
//
// The index space is cut into S = ceil(N / seg) ranges of seg indices. For
// node p (pairs [offsets[p], offsets[p+1])) and s = 0..S:
//   runs[p][s] = offsets[p] + #{ pairs of node p with index < s * seg }
// written out as a count per range and a running sum over the ranges, so
// that for ascending indices it is the position of the node's first pair
// with index >= s * seg (the node's end for s = S). Returns -1 for an index
// >= N.
// Pinned by: a brute-force count over every (node, s) on small inputs,
// runs[p][0] = offsets[p], runs[p][S] = offsets[p+1], and every pair between
// runs[p][s] and runs[p][s+1] lying in range s.
// ---------------------------------------------------------------------------
int oracle_run_table(uint32_t P, uint64_t N, uint32_t seg, const uint64_t* offsets, const uint32_t* idx,
                     uint32_t* runs) {
  const uint64_t S = (N + seg - 1) / seg;
  std::vector<uint64_t> cnt(S + 1);
  for (uint64_t p = 0; p < P; ++p) {
    std::fill(cnt.begin(), cnt.end(), 0);
    for (uint64_t e = offsets[p]; e < offsets[p + 1]; ++e) {
      if ((uint64_t)idx[e] >= N) return -1;
      cnt[idx[e] / seg] += 1;  // pairs in range idx / seg
    }
    uint64_t below = offsets[p];  // offsets[p] + pairs in ranges before s
    for (uint64_t s = 0; s <= S; ++s) {
      runs[p * (S + 1) + s] = (uint32_t)below;
      below += cnt[s];
    }
  }
  return 0;
}

}  // extern "C"
