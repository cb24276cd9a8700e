// Error-feedback Top-k of short rows for gfx950: one workgroup per node.
//
// SparCML (paperlayer.ai digest of arXiv 1802.08021v3), section 2.2: a node
// sends the k entries of largest magnitude of its accumulated gradient
// a = g + r and, section 4, keeps the others as the residual for the next
// step. Selection order: magnitude key (the IEEE bits with the sign cleared)
// descending, index ascending; the sent entries are emitted in index order
// and zeroed in the residual. The result is the one the candidate pipeline of
// topk_ef.hip computes.
//
// That pipeline is a chain of about a dozen dependent kernels, each lasting a
// few microseconds whatever the row length, which is the whole cost for short
// rows. Here a 1024-thread workgroup owns one node:
//   accumulate  a = g + r over the row, written over r, with the histogram of
//               the keys' top 11 bits in LDS;
//   refine      two passes over a (in r, now cache-resident) histogram the
//               next two 10-bit digits among the keys that share the chosen
//               prefix, which gives T, the k-th largest key, and m, how many
//               keys equal to T are taken (the lowest indices);
//   count       each wave counts the keys > T and == T over its own contiguous
//               stretch of the row; the sixteen totals give each stretch its
//               output offset and the tie rank it starts from;
//   emit        each wave walks its stretch again in index order, placing the
//               selected pairs by ballots and zeroing their residual entries.
// A row is read as its whole 16-byte groups of four (absolute positions
// 4q .. 4q+3 inside the row), each thread's positions clamped into the row
// and the surplus masked, so that the loads of a pass issue together with no
// branch between them; the at most three elements before the first whole
// group (the head) and after the last (the tail) are handled one per lane,
// the head by the first wave before its stretch, the tail by the last wave
// after its stretch.
//
// Rows of at most kRowRegMax elements (sixteen waves x sixteen steps of 64
// groups) are also held in registers: every pass uses the waves' stretches,
// each lane keeping a of its groups in VGPRs from the accumulate pass on, so
// that the refine, count and emit passes read no memory but the edges. Such a
// row moves 12 bytes per element (g and r read, a written) instead of 28.
#include "device_common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>

namespace sparcml {
namespace {

constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / kWave;    // 16
constexpr int kD0 = 2048, kD1 = 1024, kD2 = 1024;  // key digits: 11 + 10 + 10 bits
constexpr int kUnroll = 4;                         // groups per thread in flight
constexpr int kRegSteps = 16;                      // register-resident steps of 64 groups per wave
constexpr int kRegChunk = 4;                       // steps loaded together into the registers
constexpr uint64_t kRowRegMax = (uint64_t)kRowWaves * kRegSteps * kWave * 4;  // 65536 elements

// Group j (of nq) of the row starting at group q0, as four values; `own` is
// 0xF for a group of the row and 0 for a position past its end (which reads
// the row's last group again instead).
__device__ __forceinline__ void load_group(const float* __restrict__ x, uint64_t q0, uint64_t nq, uint64_t j,
                                           float (&v)[4], uint32_t& own) {
  const f32x4 t = reinterpret_cast<const f32x4*>(x)[q0 + (j < nq ? j : nq - 1)];
  v[0] = t.x;
  v[1] = t.y;
  v[2] = t.z;
  v[3] = t.w;
  own = j < nq ? 0xFu : 0u;
}

// Histogram over the row's keys in r of the digit (key >> shift) & (NB - 1),
// for keys whose bits above shift + 10 equal prefix.
template <int NB>
__device__ __forceinline__ void refine_pass(const float* __restrict__ r, uint64_t q0, uint64_t nq, uint32_t* h,
                                            uint32_t prefix, int shift) {
  constexpr int NT = kRowThreads;
  for (uint64_t j0 = 0; j0 < nq; j0 += (uint64_t)NT * kUnroll) {
    float v[kUnroll][4];
    uint32_t own[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load_group(r, q0, nq, j0 + (uint64_t)u * NT + threadIdx.x, v[u], own[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t key = mag_key(v[u][c]);
        if (own[u] && (key >> (shift + 10)) == prefix) atomicAdd(&h[(key >> shift) & (NB - 1)], 1u);
      }
  }
}

// The whole selection of one row by the calling 1024-thread workgroup: the
// row's N elements start at base in g and r; its k pairs go to oi / ov with
// idx_off added to the row-local indices; *path = 2 (this path) and *err =
// nonzero if the selection did not come to k, as the workspace reports for
// the candidate pipeline.
template <bool kReg>
__device__ __forceinline__ void select_row(const float* __restrict__ g, float* __restrict__ r, uint64_t base,
                                           uint64_t N, uint32_t k, uint32_t* __restrict__ oi, float* __restrict__ ov,
                                           uint32_t idx_off, uint32_t* path, uint32_t* err) {
  constexpr int NT = kRowThreads;
  __shared__ uint32_t h[kD0];
  __shared__ uint32_t scr[NT / kWave + 3];
  __shared__ uint32_t s_gt[kRowWaves], s_eq[kRowWaves];
  const uint64_t end = base + N;
  const uint64_t q0 = (base + 3) >> 2;                                    // first whole group
  const uint64_t nq = (end >> 2) > q0 ? (end >> 2) - q0 : 0;              // whole groups
  const uint64_t head_end = std::min<uint64_t>(4 * q0, end);              // head: [base, head_end)
  const uint64_t tail0 = std::min(std::max<uint64_t>(4 * (q0 + nq), head_end), end);  // tail: [tail0, end)
  const uint32_t nh = (uint32_t)(head_end - base), ntl = (uint32_t)(end - tail0);  // each at most 3
  // element of the head (lanes 0..2) or tail (lanes 4..6) this thread takes, if any
  const uint32_t tid = threadIdx.x;
  const bool edge = (tid < 4 && tid < nh) || (tid >= 4 && tid < 4 + ntl);
  const uint64_t e_edge = tid < 4 ? base + tid : tail0 + (tid - 4);
  for (uint32_t i = tid; i < kD0; i += NT) h[i] = 0u;
  // each wave's stretch of whole steps of 64 groups (count and emit, and every
  // pass of a register-resident row)
  const uint32_t wid = tid / kWave, lane = lane_id();
  const uint64_t steps = (nq + kWave - 1) / kWave;
  const uint64_t per_wave = (steps + kRowWaves - 1) / kRowWaves;
  const uint64_t s_lo = std::min<uint64_t>((uint64_t)wid * per_wave, steps) * kWave;
  const uint64_t s_hi = std::min<uint64_t>((uint64_t)(wid + 1) * per_wave, steps) * kWave;
  const int w_steps = (int)((s_hi - s_lo) / kWave);  // steps of this wave's stretch
  float a_reg[kReg ? kRegSteps : 1][4];              // register-resident a, step i of the stretch
  uint32_t own_reg = 0u;                             // bit i: lane's group of step i is in the row
  if (kReg && per_wave > (uint64_t)kRegSteps) {      // longer than the launch allows: report, select nothing
    if (tid == 0) {
      *path = 2u;
      *err = 1u;
    }
    return;
  }
  __syncthreads();

  // accumulate: a = g + r written over r; histogram of the top 11 key bits
  if constexpr (kReg) {
#pragma unroll
    for (int i0 = 0; i0 < kRegSteps; i0 += kRegChunk) {
      if (i0 >= w_steps) continue;  // wave-uniform; the trip count stays constant so a_reg stays in VGPRs
      float gv[kRegChunk][4];
#pragma unroll
      for (int u = 0; u < kRegChunk; ++u) {
        const uint64_t j = s_lo + (uint64_t)(i0 + u) * kWave + lane;
        uint32_t own;
        load_group(g, q0, nq, j < s_hi ? j : nq, gv[u], own);
        load_group(r, q0, nq, j < s_hi ? j : nq, a_reg[i0 + u], own);
        own_reg |= (own ? 1u : 0u) << (i0 + u);
      }
#pragma unroll
      for (int u = 0; u < kRegChunk; ++u) {
#pragma unroll
        for (int c = 0; c < 4; ++c) a_reg[i0 + u][c] = gv[u][c] + a_reg[i0 + u][c];
        if ((own_reg >> (i0 + u)) & 1u) {
          f32x4 t;
          t.x = a_reg[i0 + u][0];
          t.y = a_reg[i0 + u][1];
          t.z = a_reg[i0 + u][2];
          t.w = a_reg[i0 + u][3];
          reinterpret_cast<f32x4*>(r)[q0 + s_lo + (uint64_t)(i0 + u) * kWave + lane] = t;
          if (k != 0u) {
#pragma unroll
            for (int c = 0; c < 4; ++c) atomicAdd(&h[mag_key(a_reg[i0 + u][c]) >> 20], 1u);
          }
        }
      }
    }
  }
  for (uint64_t j0 = 0; !kReg && j0 < nq; j0 += (uint64_t)NT * kUnroll) {
    float gv[kUnroll][4], rv[kUnroll][4];
    uint32_t own[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t j = j0 + (uint64_t)u * NT + tid;
      load_group(g, q0, nq, j, gv[u], own[u]);
      load_group(r, q0, nq, j, rv[u], own[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float a[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = gv[u][c] + rv[u][c];
      if (own[u]) {
        f32x4 t;
        t.x = a[0];
        t.y = a[1];
        t.z = a[2];
        t.w = a[3];
        reinterpret_cast<f32x4*>(r)[q0 + j0 + (uint64_t)u * NT + tid] = t;
        if (k != 0u) {
#pragma unroll
          for (int c = 0; c < 4; ++c) atomicAdd(&h[mag_key(a[c]) >> 20], 1u);
        }
      }
    }
  }
  if (edge) {
    const float a = g[e_edge] + r[e_edge];
    r[e_edge] = a;
    if (k != 0u) atomicAdd(&h[mag_key(a) >> 20], 1u);
  }
  if (k == 0u) {  // nothing is sent: the residual is a
    if (tid == 0) {
      *path = 2u;
      *err = 0u;
    }
    return;
  }
  __syncthreads();

  // histogram pass over the register-resident a: digit (key >> shift) & (NB - 1)
  // of the keys whose bits above shift + 10 equal prefix
  auto refine_regs = [&](uint32_t prefix, int shift, uint32_t mask) {
#pragma unroll
    for (int i = 0; i < kRegSteps; ++i) {
      if (kReg && i < w_steps && ((own_reg >> i) & 1u)) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t key = mag_key(a_reg[i][c]);
          if ((key >> (shift + 10)) == prefix) atomicAdd(&h[(key >> shift) & mask], 1u);
        }
      }
    }
  };

  // refine: T = the k-th largest key, m = keys equal to T that are taken
  uint32_t d0, d1, d2, above;
  block_find_suffix<NT, kD0>(h, k, scr, d0, above);
  uint32_t rank = k - above;
  for (uint32_t i = tid; i < kD1; i += NT) h[i] = 0u;
  __syncthreads();
  if constexpr (kReg)
    refine_regs(d0, 10, kD1 - 1);
  else
    refine_pass<kD1>(r, q0, nq, h, d0, 10);
  if (edge) {
    const uint32_t key = mag_key(r[e_edge]);
    if ((key >> 20) == d0) atomicAdd(&h[(key >> 10) & (kD1 - 1)], 1u);
  }
  __syncthreads();
  block_find_suffix<NT, kD1>(h, rank, scr, d1, above);
  rank -= above;
  const uint32_t prefix = (d0 << 10) | d1;  // key >> 10
  for (uint32_t i = tid; i < kD2; i += NT) h[i] = 0u;
  __syncthreads();
  if constexpr (kReg)
    refine_regs(prefix, 0, kD2 - 1);
  else
    refine_pass<kD2>(r, q0, nq, h, prefix, 0);
  if (edge) {
    const uint32_t key = mag_key(r[e_edge]);
    if ((key >> 10) == prefix) atomicAdd(&h[key & (kD2 - 1)], 1u);
  }
  __syncthreads();
  block_find_suffix<NT, kD2>(h, rank, scr, d2, above);
  const uint32_t T = (prefix << 10) | d2;
  const uint32_t m = rank - above;

  // Keys equal to T in the row: bin d2 of the last histogram, whose bins are
  // whole keys. When all of them are taken (the usual case of a unique T) the
  // selection is simply key >= T and no tie rank is needed.
  const bool all_ties = h[d2] == m;

  auto load_steps = [&](uint64_t s0, float (&v)[kUnroll][4], uint32_t (&own)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t j = s0 + (uint64_t)u * kWave + lane;
      load_group(r, q0, nq, j < s_hi ? j : nq, v[u], own[u]);
    }
  };
  // the head (first wave) or the tail (last wave) as one step, one element per lane
  auto edge_step = [&](bool head, float (&v)[4], uint32_t& own, uint64_t& e_first) {
    const uint32_t n = head ? nh : ntl;
    e_first = (head ? base : tail0) + lane;
    v[0] = v[1] = v[2] = v[3] = 0.0f;
    own = 0u;
    if (lane < n) {
      v[0] = r[e_first];
      own = 1u;
    }
  };
  const bool first_wave = wid == 0, last_wave = wid == (uint32_t)kRowWaves - 1;

  // count, then emit; kAll: every key equal to T is taken
  auto finish = [&](auto take_all) {
    constexpr bool kAll = decltype(take_all)::value;
    // count: over each wave's stretch, the keys >= T (kAll), else the keys > T and == T
    uint32_t gt = 0, eq = 0;  // wave-uniform
    auto count_step = [&](const float (&v)[4], uint32_t own) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool in = (own >> c) & 1u;
        const uint32_t key = mag_key(v[c]);
        if constexpr (kAll) {
          gt += popc64(ballot(in && key >= T));
        } else {
          gt += popc64(ballot(in && key > T));
          eq += popc64(ballot(in && key == T));
        }
      }
    };
    if (first_wave && nh != 0u) {
      float v[4];
      uint32_t own;
      uint64_t e;
      edge_step(true, v, own, e);
      count_step(v, own);
    }
    if constexpr (kReg) {
#pragma unroll
      for (int i = 0; i < kRegSteps; ++i) {
        if (i >= w_steps) continue;
        count_step(a_reg[i], ((own_reg >> i) & 1u) ? 0xFu : 0u);
      }
    }
    for (uint64_t s0 = s_lo; !kReg && s0 < s_hi; s0 += (uint64_t)kWave * kUnroll) {
      float v[kUnroll][4];
      uint32_t own[kUnroll];
      load_steps(s0, v, own);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) count_step(v[u], own[u]);
    }
    if (last_wave && ntl != 0u) {
      float v[4];
      uint32_t own;
      uint64_t e;
      edge_step(false, v, own, e);
      count_step(v, own);
    }
    if (lane == 0) {
      s_gt[wid] = gt;
      s_eq[wid] = eq;
    }
    __syncthreads();
    // lane w < 16 of every wave takes wave w's totals: ties before it, ties it
    // takes (the lowest indices first), and selected pairs before it
    const uint32_t e_w = lane < (uint32_t)kRowWaves ? s_eq[lane] : 0u;
    const uint32_t g_w = lane < (uint32_t)kRowWaves ? s_gt[lane] : 0u;
    const uint32_t eq_before = wave_inclusive_scan(e_w) - e_w;
    const uint32_t sel_w = g_w + (eq_before >= m ? 0u : std::min(m - eq_before, e_w));
    const uint32_t sel_incl = wave_inclusive_scan(sel_w);
    uint32_t eq_run = __builtin_amdgcn_readlane(eq_before, wid);  // ties and selected pairs before
    uint32_t pos = __builtin_amdgcn_readlane(sel_incl - sel_w, wid);  // this wave's stretch
    const uint32_t all_sel = __builtin_amdgcn_readlane(sel_incl, kRowWaves - 1);
    if (tid == 0) {
      *path = 2u;
      *err = all_sel != k ? 1u : 0u;
    }

    // emit: the stretch in index order (lane, then element within the group);
    // element c of lane l is at e_first + c (own bit c set)
    auto emit_step = [&](const float (&v)[4], uint32_t own, uint64_t e_first) {
      uint32_t sel = 0u;
      if constexpr (kAll) {
        uint64_t sm[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool s = ((own >> c) & 1u) && mag_key(v[c]) >= T;
          sel |= s ? 1u << c : 0u;
          sm[c] = ballot(s);
        }
        if ((sm[0] | sm[1] | sm[2] | sm[3]) == 0u) return;  // nothing selected in this step
        uint32_t p = pos + lanes_below(sm[0]) + lanes_below(sm[1]) + lanes_below(sm[2]) + lanes_below(sm[3]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if ((sel >> c) & 1u) {
            const uint64_t e = e_first + c;
            if (p < k) {
              oi[p] = (uint32_t)(e - base) + idx_off;
              ov[p] = v[c];
            }
            r[e] = 0.0f;
            ++p;
          }
        pos += popc64(sm[0]) + popc64(sm[1]) + popc64(sm[2]) + popc64(sm[3]);
        return;
      }
      uint32_t is_eq = 0u, is_gt = 0u;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool in = (own >> c) & 1u;
        const uint32_t key = mag_key(v[c]);
        if (in && key == T) is_eq |= 1u << c;
        if (in && key > T) is_gt |= 1u << c;
      }
      // tie ranks in index order: ties before this step, in lower lanes, and
      // earlier in this lane
      uint32_t eq_below = 0, step_eq = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint64_t em = ballot((is_eq >> c) & 1u);
        eq_below += lanes_below(em);
        step_eq += popc64(em);
      }
      uint32_t rank_t = eq_run + eq_below;
      sel = is_gt;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((is_eq >> c) & 1u) {
          if (rank_t < m) sel |= 1u << c;
          ++rank_t;
        }
      eq_run += step_eq;
      uint32_t sel_below = 0, step_sel = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint64_t sm = ballot((sel >> c) & 1u);
        sel_below += lanes_below(sm);
        step_sel += popc64(sm);
      }
      uint32_t p = pos + sel_below;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((sel >> c) & 1u) {
          const uint64_t e = e_first + c;
          if (p < k) {
            oi[p] = (uint32_t)(e - base) + idx_off;
            ov[p] = v[c];
          }
          r[e] = 0.0f;
          ++p;
        }
      pos += step_sel;
    };
    if (first_wave && nh != 0u) {
      float v[4];
      uint32_t own;
      uint64_t e;
      edge_step(true, v, own, e);
      emit_step(v, own, e);
    }
    if constexpr (kReg) {
#pragma unroll
      for (int i = 0; i < kRegSteps; ++i) {
        if (i >= w_steps) continue;
        emit_step(a_reg[i], ((own_reg >> i) & 1u) ? 0xFu : 0u, 4 * (q0 + s_lo + (uint64_t)i * kWave + lane));
      }
    }
    for (uint64_t s0 = s_lo; !kReg && s0 < s_hi; s0 += (uint64_t)kWave * kUnroll) {
      float v[kUnroll][4];
      uint32_t own[kUnroll];
      load_steps(s0, v, own);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) emit_step(v[u], own[u], 4 * (q0 + s0 + (uint64_t)u * kWave + lane));
    }
    if (last_wave && ntl != 0u) {
      float v[4];
      uint32_t own;
      uint64_t e;
      edge_step(false, v, own, e);
      emit_step(v, own, e);
    }
  };
  if (all_ties)
    finish(std::true_type{});
  else
    finish(std::false_type{});
}
// whole-node call: row p of [P][N]; info holds the [P] path and [P]
// consistency words
template <bool kReg>
__global__ __launch_bounds__(kRowThreads) void k_topk_row(const float* __restrict__ g, float* __restrict__ r,
                                                          uint64_t N, uint32_t k, uint32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_val, uint32_t* __restrict__ info) {
  const uint32_t p = blockIdx.x;
  select_row<kReg>(g, r, (uint64_t)p * N, N, k, out_idx + (uint64_t)p * k, out_val + (uint64_t)p * k, 0u, info + p,
             info + gridDim.x + p);
}

// per-layer call: row p * nl + l is layer l ([loff[l], loff[l+1])) of node p,
// whose lk[l] pairs go at p * K + lkoff[l]; info holds the [P * nl] path and
// [P * nl] consistency words
template <bool kReg>
__global__ __launch_bounds__(kRowThreads) void k_topk_layer_rows(const float* __restrict__ g, float* __restrict__ r,
                                                                 uint64_t N, uint32_t nl, const uint64_t* loff,
                                                                 const uint64_t* lk, const uint64_t* lkoff, uint64_t K,
                                                                 uint32_t* __restrict__ out_idx,
                                                                 float* __restrict__ out_val,
                                                                 uint32_t* __restrict__ info) {
  const uint32_t row = blockIdx.x, p = row / nl, l = row % nl;
  const uint64_t o = loff[l];
  const uint64_t out = (uint64_t)p * K + lkoff[l];
  select_row<kReg>(g, r, (uint64_t)p * N + o, loff[l + 1] - o, (uint32_t)lk[l], out_idx + out, out_val + out, (uint32_t)o,
             info + row, info + gridDim.x + row);
}

// layer tables copied to the device, kRowLayersPerCopy layers per launch
// (kernel arguments): loff[first .. first+count], lk and lkoff[first ..)
constexpr uint32_t kRowLayersPerCopy = 64;
struct RowLayerChunk {
  uint64_t off[kRowLayersPerCopy + 1];
  uint64_t k[kRowLayersPerCopy];
  uint64_t koff[kRowLayersPerCopy];
};

__global__ void k_row_layers_in(uint64_t* loff, uint64_t* lk, uint64_t* lkoff, uint32_t first, uint32_t count,
                                RowLayerChunk in) {
  for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) {
    loff[first + i] = in.off[i];
    lk[first + i] = in.k[i];
    lkoff[first + i] = in.koff[i];
  }
  if (threadIdx.x == 0) loff[first + count] = in.off[count];
}

}  // namespace

size_t topk_layer_rows_workspace_bytes(uint32_t P, uint32_t nl) {
  return (8ull * P * nl + 255) / 256 * 256 + 24ull * (nl + 1);
}

hipError_t topk_layer_rows_launch(uint32_t P, uint64_t N, uint32_t nl, const uint64_t* off, const uint64_t* k,
                                  const float* grad, float* residual, uint32_t* out_idx, float* out_val, void* ws,
                                  hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  uint32_t* info = reinterpret_cast<uint32_t*>(w);  // [P * nl] path words, then [P * nl] consistency words
  uint64_t* loff = reinterpret_cast<uint64_t*>(w + (8ull * P * nl + 255) / 256 * 256);
  uint64_t* lk = loff + nl + 1;
  uint64_t* lkoff = lk + nl;
  uint64_t koff = 0;
  for (uint32_t first = 0; first < nl; first += kRowLayersPerCopy) {
    RowLayerChunk in{};
    const uint32_t count = std::min<uint32_t>(kRowLayersPerCopy, nl - first);
    for (uint32_t i = 0; i < count; ++i) {
      in.off[i] = off[first + i];
      in.k[i] = k[first + i];
      in.koff[i] = koff;
      koff += k[first + i];
    }
    in.off[count] = off[first + count];
    hipLaunchKernelGGL(k_row_layers_in, dim3(1), dim3(64), 0, stream, loff, lk, lkoff, first, count, in);
  }
  uint64_t longest = 0;
  for (uint32_t l = 0; l < nl; ++l) longest = std::max(longest, off[l + 1] - off[l]);
  if (longest <= kRowRegMax)
    hipLaunchKernelGGL(k_topk_layer_rows<true>, dim3(P * nl), dim3(kRowThreads), 0, stream, grad, residual, N, nl,
                       loff, lk, lkoff, koff, out_idx, out_val, info);
  else
    hipLaunchKernelGGL(k_topk_layer_rows<false>, dim3(P * nl), dim3(kRowThreads), 0, stream, grad, residual, N, nl,
                       loff, lk, lkoff, koff, out_idx, out_val, info);
  return hipGetLastError();
}

hipError_t topk_row_launch(uint32_t P, uint64_t N, uint64_t k, const float* grad, float* residual,
                           uint32_t* out_idx, float* out_val, uint32_t* info, hipStream_t stream,
                           const OpEvents* ev) {
  // one kernel, the op's first, last and dominant at once: it carries the
  // op's pair when one is given, else the kernel pair
  const hipEvent_t e0 = ev ? (ev->op_start ? ev->op_start : ev->k_start) : nullptr;
  const hipEvent_t e1 = ev ? (ev->op_stop ? ev->op_stop : ev->k_stop) : nullptr;
  if (N <= kRowRegMax)
    return launch_ev(k_topk_row<true>, dim3(P), dim3(kRowThreads), stream, e0, e1, grad, residual, N, (uint32_t)k,
                     out_idx, out_val, info);
  return launch_ev(k_topk_row<false>, dim3(P), dim3(kRowThreads), stream, e0, e1, grad, residual, N, (uint32_t)k,
                   out_idx, out_val, info);
}

}  // namespace sparcml
