// Lightning-indexer scores (QbitAI article on DeepSeek-V4, hybrid attention
// section: the indexer is inherited from V3.2's DSA; "DeepSeek V4 Architecture
// Tricks", section "CSA": 64 indexer heads of dim 128; section "FP4 / FP8
// Quantization-Aware Training": the indexer QK path runs in FP4):
//   I[b,t,s] = sum_h w[b,t,h] * relu(qI[b,t,h] . kI[b,s])   for s < vis(b,t).
//
// The QK product is the one dense contraction of the path.  For H_I = 64 and
// d_I = 128 in fp8 or MXFP4 it runs on gfx950's 32x32x64 f8f6f4 MFMA: the 64
// heads are two 32-row A tiles held in registers for the whole kernel, each
// group of 32 keys is the B tile, and two K=64 steps cover d_I.  The ReLU,
// head weighting and head sum happen on the accumulators: a lane holds 16 head
// rows of one key column per tile, so it reduces them locally and one lane swap
// (lane l <-> l^32) completes the 64-head sum.
//
// Operand layout: a lane (column j = l%32, k-group g = l/32) of both A and B
// holds the same 32 k-positions of its row; which d_I positions those are is a
// free choice as long as A and B agree.  Lane group g loads bytes
// [64g + 32ks, 64g + 32ks + 32) of a row for K-step ks (fp8), i.e. 64
// contiguous bytes per lane and key.  For MXFP4 each lane's 32 values must be
// exactly one 32-element scale block, so lane group g takes block 2g + ks
// together with that block's E8M0 scale.
#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>

#include "common.h"

namespace lca {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kIdxWaves = 4;
constexpr int kKeysPerGroup = 32;
constexpr int kBlockKeys = kIdxWaves * kKeysPerGroup;  // 128 keys per workgroup step
// Workgroups per query row: the row's 128-key blocks are dealt round-robin to
// the row's workgroups, so the workgroups of a row sweep its keys together
// (a few MiB apart at most) instead of each streaming a separate chunk; this
// keeps HBM row-buffer locality.  Chosen so that a decode batch has about
// 1536 workgroups (6 per CU).
constexpr int kTargetBlocks = 1536;

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

__device__ __forceinline__ v8i load16(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// fmt 0 = fp8 e4m3 operands (unit scales), 4 = fp4 e2m1 operands (per-lane E8M0 scales)
template <int FMT>
__device__ __forceinline__ v16f mfma(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, sa, 0, sb);
}

__device__ __forceinline__ int lanes_below64(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

template <bool MX>
struct KeyGroup {
  v8i b[2];
  int sb[2];
};

// B operand (32 keys) of one key group for this lane: key row `key`.
template <bool MX>
__device__ __forceinline__ void load_group(const uint8_t* kb_base, const uint8_t* ks_base, int key,
                                           int g, KeyGroup<MX>& G) {
  constexpr int kRowBytes = MX ? 64 : 128;
  const uint8_t* kp = kb_base + static_cast<size_t>(key) * kRowBytes;
  if (MX) {
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(ks_base + static_cast<size_t>(key) * 4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int blk = 2 * g + ks;
      G.b[ks] = load16(kp + 16 * blk);
      G.sb[ks] = (sc >> (8 * blk)) & 0xff;
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      G.b[ks] = load32(kp + 64 * g + 32 * ks);
      G.sb[ks] = 127;
    }
  }
}

// A operand of one query row: heads 32*ht + j, K-steps ks = 0, 1.
template <bool MX>
__device__ __forceinline__ void load_query(const uint8_t* qI, const uint8_t* qI_scale, long long row,
                                           int j, int g, v8i (&A)[2][2], int (&sA)[2][2]) {
  constexpr int kRowBytes = MX ? 64 : 128;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const size_t hrow = static_cast<size_t>(row) * 64 + 32 * ht + j;
    const uint8_t* qp = qI + hrow * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (MX) {
        const int blk = 2 * g + ks;
        A[ht][ks] = load16(qp + 16 * blk);
        sA[ht][ks] = qI_scale[hrow * 4 + blk];
      } else {
        A[ht][ks] = load32(qp + 64 * g + 32 * ks);
        sA[ht][ks] = 127;
      }
    }
  }
}

// x of lane l plus x of lane l ^ 32, with gfx950's lane-half swap (a VALU op:
// lanes 32..63 of the first operand trade places with lanes 0..31 of the
// second, so the two results hold the pair's values in either order).
__device__ __forceinline__ float lane_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(static_cast<uint32_t>(r[0])) + __uint_as_float(static_cast<uint32_t>(r[1]));
}

// A 32-key group against the query's 64 heads: accumulator tile ht holds heads
// 32*ht + 8*(r/4) + 4*g + (r%4) in register r, key column j.
struct GroupAcc {
  v16f a[2];
};

template <bool MX>
__device__ __forceinline__ GroupAcc group_mma(const v8i (&A)[2][2], const int (&sA)[2][2],
                                              const KeyGroup<MX>& cur) {
  constexpr int kFmt = MX ? 4 : 0;
  GroupAcc r;
  r.a[0] = v16f{0};
  r.a[1] = v16f{0};
  r.a[0] = mfma<kFmt>(A[0][0], cur.b[0], r.a[0], sA[0][0], cur.sb[0]);
  r.a[1] = mfma<kFmt>(A[1][0], cur.b[0], r.a[1], sA[1][0], cur.sb[0]);
  r.a[0] = mfma<kFmt>(A[0][1], cur.b[1], r.a[0], sA[0][1], cur.sb[1]);
  r.a[1] = mfma<kFmt>(A[1][1], cur.b[1], r.a[1], sA[1][1], cur.sb[1]);
  return r;
}

// Score of key column j (valid in every lane; lanes j and j+32 agree): the 64
// heads' ReLU'd dot products weighted by w_s and summed, in four independent
// partial sums; four consecutive registers read one float4 of the weights.
// group_reduce_reg: the same with the lane's 32 weights in registers
// (wr[4 ht + a] = w_s[32 ht + 8 a + 4 g .. + 4]).
__device__ __forceinline__ float group_reduce_reg(const GroupAcc& acc, const float4 (&wr)[8]) {
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 w4 = wr[4 * ht + a];
      p[0] = fmaf(w4.x, fmaxf(acc.a[ht][4 * a], 0.f), p[0]);
      p[1] = fmaf(w4.y, fmaxf(acc.a[ht][4 * a + 1], 0.f), p[1]);
      p[2] = fmaf(w4.z, fmaxf(acc.a[ht][4 * a + 2], 0.f), p[2]);
      p[3] = fmaf(w4.w, fmaxf(acc.a[ht][4 * a + 3], 0.f), p[3]);
    }
  }
  return lane_pair_sum((p[0] + p[1]) + (p[2] + p[3]));
}
__device__ __forceinline__ float group_reduce(const GroupAcc& acc, const float* w_s, int g) {
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 w4 = *reinterpret_cast<const float4*>(&w_s[32 * ht + 8 * a + 4 * g]);
      p[0] = fmaf(w4.x, fmaxf(acc.a[ht][4 * a], 0.f), p[0]);
      p[1] = fmaf(w4.y, fmaxf(acc.a[ht][4 * a + 1], 0.f), p[1]);
      p[2] = fmaf(w4.z, fmaxf(acc.a[ht][4 * a + 2], 0.f), p[2]);
      p[3] = fmaf(w4.w, fmaxf(acc.a[ht][4 * a + 3], 0.f), p[3]);
    }
  }
  return lane_pair_sum((p[0] + p[1]) + (p[2] + p[3]));
}

template <bool MX>
__device__ __forceinline__ float group_score(const v8i (&A)[2][2], const int (&sA)[2][2],
                                             const KeyGroup<MX>& cur, const float* w_s, int g) {
  return group_reduce(group_mma<MX>(A, sA, cur), w_s, g);
}

// Scores of every visible key, written to scores[row]; HIST: also add their
// score_bin histogram into hist[row] (global, zeroed by the caller) through a
// per-workgroup LDS histogram.  Workgroup wi of a row takes the row's 128-key
// blocks wi, wi + wpr, ...; wave w the 32 keys at offset 32w of each.
template <bool MX, bool HIST, typename ST>
__global__ __launch_bounds__(kWave * kIdxWaves, 3) void indexer_mfma_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale,
    const uint8_t* __restrict__ kI, const uint8_t* __restrict__ kI_scale, int n_q, int N_cap,
    int wpr, const float* __restrict__ w, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, ST* __restrict__ scores,
    uint32_t* __restrict__ hist) {
  constexpr int kRowBytes = MX ? 64 : 128;  // bytes of one 128-dim vector
  __shared__ uint32_t lh[HIST ? kScoreHistBins : 1];
  __shared__ __attribute__((aligned(16))) float w_s[64];
  const long long row = blockIdx.x / wpr;
  const int wi = blockIdx.x % wpr;
  const int b = static_cast<int>(row / n_q);
  const int vis = visible_entries(q_pos[row], m, n_entries[b], N_cap);
  if (wi * kBlockKeys >= vis) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 31;
  const int g = lane >> 5;
  if (HIST) {
    for (int i = threadIdx.x; i < kScoreHistBins; i += kWave * kIdxWaves) lh[i] = 0;
  }
  v8i A[2][2];
  int sA[2][2];
  load_query<MX>(qI, qI_scale, row, j, g, A, sA);
  if (threadIdx.x < 64) w_s[threadIdx.x] = w[static_cast<size_t>(row) * 64 + threadIdx.x];
  const uint8_t* kb_base = kI + static_cast<size_t>(b) * N_cap * kRowBytes;
  const uint8_t* ks_base = MX ? kI_scale + static_cast<size_t>(b) * N_cap * 4 : nullptr;
  ST* out = scores + static_cast<size_t>(row) * N_cap;
  __syncthreads();

  // Every wave runs all n_t steps (a group past the end loads a clamped key and
  // stores nothing).
  const int stride = kBlockKeys * wpr;
  const int n_t = (vis - wi * kBlockKeys + stride - 1) / stride;
  auto key0 = [&](int t) {
    return (wi + min(t, n_t - 1) * wpr) * kBlockKeys + wave * kKeysPerGroup;
  };
  auto load = [&](KeyGroup<MX>& G, int t) {
    load_group<MX>(kb_base, ks_base, min(key0(t) + j, vis - 1), g, G);
  };
  auto step = [&](const KeyGroup<MX>& cur, int t) {
    const float s = group_score<MX>(A, sA, cur, w_s, g);
    const int kb = key0(t);
    if (g == 0 && kb + j < vis) {
      store_score(&out[kb + j], s);
      if (HIST) atomicAdd(&lh[score_bin(key_as_stored<ST>(s))], 1u);
    }
  };
  // Three named buffers, unrolled by three: a load always fills the buffer whose
  // group was consumed one step earlier, so nothing is copied between registers
  // (a copy of a buffer still in flight would make the wave wait for it) and two
  // groups stay in flight while one is computed.  The loads are unconditional:
  // a load under a branch leaves the count of newer loads unknown, and the wave
  // would then wait for all of them.  The query operands arrive first.
  __builtin_amdgcn_s_waitcnt(0);
  KeyGroup<MX> g0, g1, g2;
  load(g0, 0);
  __builtin_amdgcn_sched_barrier(0);  // g0's loads go out before g1's, as in the loop
  load(g1, 1);
  for (int t = 0; t < n_t; t += 3) {
    load(g2, t + 2);
    step(g0, t);
    if (t + 1 >= n_t) break;
    load(g0, t + 3);
    step(g1, t + 1);
    if (t + 2 >= n_t) break;
    load(g1, t + 4);
    step(g2, t + 2);
  }
  if (HIST) {
    __syncthreads();
    uint32_t* gh = hist + row * kScoreHistBins;
    for (int i = threadIdx.x; i < kScoreHistBins; i += kWave * kIdxWaves)
      if (lh[i]) atomicAdd(&gh[hist_slot(i)], lh[i]);
  }
}

// ---------------------------------------------------------------------------
// Fused selection (SelectWs): the scores stay in LDS and only the entries that
// can still be among the row's k largest leave the chip.

constexpr int kSelWaves = 12;                      // one workgroup per CU
constexpr int kSelThreads = kWave * kSelWaves;
// LDS scores per workgroup: at most 280 blocks (140 KiB; the workgroup is alone on its CU)
constexpr int kSelMaxBlocks = 280;

// After a workgroup's scores are final: bound the row's threshold bin from
// below, write every entry at or above the bound into the workgroup's region
// of the row's emit array, then add the rest of the workgroup's histogram (lh
// holds the counts not flushed yet) to the row's.  Histogram counts only grow,
// and the counts in lh are added only after the row histogram has been read,
// so (count read) + (count in lh) never exceeds the final count of a bin: if
// bins >= b hold >= k entries by that sum, the final k-th largest key lies in
// bin >= b.  Every entry of the final top-k is therefore emitted, whatever the
// order in which workgroups run, and no workgroup waits for another.  The bound
// looks at the blockDim bins ending 32 bins above the workgroup's highest bin;
// entries elsewhere only make it weaker.
template <int NW>
__device__ void select_emit(uint32_t* lh, const float* sc, int n_t, int wi, int wpr, int vis,
                            long long row, const SelectWs& o, int k, uint32_t kmax) {
  constexpr int NT = NW * kWave;
  __shared__ int sh_bin, scan_sh[NW];
  __shared__ uint32_t top_sh[NW];
  __shared__ int emit_n;  // pairs written to the region so far
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  uint32_t* gh = o.hist + row * kScoreHistBins;
  for (int off = 32; off >= 1; off >>= 1)
    kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(kmax, off, kWave)));
  if (lane == 0) top_sh[wave] = kmax;
  if (tid == 0) {
    sh_bin = -1;
    emit_n = 0;
  }
  __syncthreads();
  uint32_t tk = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) tk = max(tk, top_sh[x]);
  const int top = static_cast<int>(score_bin(tk));
  const int hi = min(top + 32, kScoreHistBins - 1);
  const int bin = hi - tid;
  int v = 0;
  if (bin >= 0)
    v = static_cast<int>(__hip_atomic_load(&gh[hist_slot(bin)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
                         lh[bin]);
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int u = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += u;
  }
  if (lane == kWave - 1) scan_sh[wave] = incl;
  __syncthreads();
  for (int x = 0; x < wave; ++x) incl += scan_sh[x];
  // the highest bin whose cumulative count from hi reaches k (a unique thread)
  if (incl >= k && incl - v < k) sh_bin = bin;
  const int b_lb = __syncthreads_or(incl >= k) ? sh_bin : -1;
  // emission: wave w takes blocks w, w + NW, ...; lane l holds keys l and l + 64
  // of a block.  The scores of kEmitBatch blocks are read (unconditionally: the
  // LDS array holds n_t whole blocks) before any is used, so the LDS reads
  // overlap, and one LDS atomic per batch places the batch's pairs in the region.
  uint2* reg = o.emit + static_cast<size_t>(row) * o.n_blk * kSelBlock + select_region(o.n_blk, wpr, wi);
  constexpr int kEmitBatch = 4;
  for (int t0 = wave; t0 < n_t; t0 += kEmitBatch * NW) {
    float s0[kEmitBatch], s1[kEmitBatch];
#pragma unroll
    for (int u = 0; u < kEmitBatch; ++u) {
      const int t = min(t0 + u * NW, n_t - 1);
      s0[u] = sc[t * kSelBlock + lane];
      s1[u] = sc[t * kSelBlock + kWave + lane];
    }
    uint32_t k0[kEmitBatch], k1[kEmitBatch];
    uint64_t m0[kEmitBatch], m1[kEmitBatch];
    int n_tot = 0;
#pragma unroll
    for (int u = 0; u < kEmitBatch; ++u) {
      const int t = t0 + u * NW;  // t < n_t is the same for the whole wave
      const int i0 = (wi + t * wpr) * kSelBlock + lane, i1 = i0 + kWave;
      k0[u] = score_key(s0[u]);
      k1[u] = score_key(s1[u]);
      const bool e0 = t < n_t && i0 < vis && static_cast<int>(score_bin(k0[u])) >= b_lb;
      const bool e1 = t < n_t && i1 < vis && static_cast<int>(score_bin(k1[u])) >= b_lb;
      m0[u] = __ballot(e0);
      m1[u] = __ballot(e1);
      n_tot += __popcll(m0[u]) + __popcll(m1[u]);
    }
    if (n_tot == 0) continue;  // the same for the whole wave
    int base = 0;
    if (lane == 0) base = atomicAdd(&emit_n, n_tot);
    base = __shfl(base, 0, kWave);
#pragma unroll
    for (int u = 0; u < kEmitBatch; ++u) {
      const int i0 = (wi + (t0 + u * NW) * wpr) * kSelBlock + lane;
      if ((m0[u] >> lane) & 1)
        reg[base + lanes_below64(m0[u])] = make_uint2(k0[u], static_cast<uint32_t>(i0));
      base += __popcll(m0[u]);
      if ((m1[u] >> lane) & 1)
        reg[base + lanes_below64(m1[u])] = make_uint2(k1[u], static_cast<uint32_t>(i0 + kWave));
      base += __popcll(m1[u]);
    }
  }
  for (int bb = tid; bb < kScoreHistBins; bb += NT)
    if (lh[bb]) atomicAdd(&gh[hist_slot(bb)], lh[bb]);
  __syncthreads();  // emit_n is final
  if (tid == 0) o.emit_cnt[row * o.n_blk + wi] = emit_n;
}

// One 12-wave workgroup per CU.  Rows are interleaved over the grid (row =
// blockIdx % rows), workgroup wi of a row owns the row's blocks wi, wi + wpr,
// ... (n_t of them, 4 groups of 32 keys each), and the workgroup's waves take
// its groups from an LDS counter, so a wave that the CU serves faster simply
// takes more of them and all waves end together.  Group q's scores go to
// sc[32 q ...] (block q/4, offset 32 (q%4)).  The wave that takes the middle
// group also flushes the histogram so far (atomic exchange on the LDS bins, no
// barrier), which lets the row's other workgroups bound the threshold tightly.
template <bool MX>
__global__ __launch_bounds__(kSelThreads, 1) void indexer_select_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale,
    const uint8_t* __restrict__ kI, const uint8_t* __restrict__ kI_scale, int n_q, int N_cap,
    int wpr, const float* __restrict__ w, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, SelectWs sel, int k, int32_t* __restrict__ sel_idx) {
  constexpr int kRowBytes = MX ? 64 : 128;
  constexpr int kFirst = 3;  // groups per wave assigned before the counter
  __shared__ uint32_t lh[kScoreHistBins];
  __shared__ __attribute__((aligned(16))) float w_s[64];
  __shared__ int next_grp;
  extern __shared__ float sc[];
  const long long rows = gridDim.x / wpr;
  const long long row = blockIdx.x % rows;
  const int wi = static_cast<int>(blockIdx.x / rows);
  const int b = static_cast<int>(row / n_q);
  int qp, ne;
  if (sel.n_tokens) {  // a decode step's position, straight from the token count
    const int p = sel.n_tokens[b];
    if (p >= 0) {
      qp = p;
      ne = min((p + 1) / m, N_cap);
      if (wi == 0 && threadIdx.x == 0) {
        sel.q_pos_out[row] = qp;
        sel.n_entries_out[b] = ne;
      }
    } else {
      qp = q_pos[row];
      ne = n_entries[b];
    }
  } else {
    qp = q_pos[row];
    ne = n_entries[b];
  }
  const int vis = visible_entries(qp, m, ne, N_cap);
  int32_t* out = sel_idx + row * k;
  if (vis <= k) {  // every visible entry is selected: no scores needed
    if (wi == 0)
      for (int i = threadIdx.x; i < k; i += kSelThreads) out[i] = i < vis ? i : -1;
    return;
  }
  if (wi * kBlockKeys >= vis) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int j = lane & 31;
  const int g = lane >> 5;
  for (int i = tid; i < kScoreHistBins; i += kSelThreads) lh[i] = 0;
  if (tid == 0) next_grp = kSelWaves * kFirst;
  v8i A[2][2];
  int sA[2][2];
  load_query<MX>(qI, qI_scale, row, j, g, A, sA);
  if (tid < 64) w_s[tid] = w[static_cast<size_t>(row) * 64 + tid];
  const uint8_t* kb_base = kI + static_cast<size_t>(b) * N_cap * kRowBytes;
  const uint8_t* ks_base = MX ? kI_scale + static_cast<size_t>(b) * N_cap * 4 : nullptr;
  const int stride = kBlockKeys * wpr;
  const int n_t = (vis - wi * kBlockKeys + stride - 1) / stride;
  const int n_grp = 4 * n_t;
  const int mid = n_grp / 2;
  __syncthreads();

  auto key0 = [&](int q) {  // first key of group q (q past the end: the last group)
    q = min(q, n_grp - 1);
    return (wi + (q >> 2) * wpr) * kBlockKeys + (q & 3) * kKeysPerGroup;
  };
  auto load = [&](KeyGroup<MX>& G, int q) {
    load_group<MX>(kb_base, ks_base, min(key0(q) + j, vis - 1), g, G);
  };
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_grp, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  uint32_t kmax = 0;  // largest score key this lane wrote
  auto step = [&](const KeyGroup<MX>& cur, int q) {
    const float s = group_score<MX>(A, sA, cur, w_s, g);
    const int kb = key0(q);
    if (g == 0 && kb + j < vis) {
      const uint32_t key = score_key(s);
      sc[q * kKeysPerGroup + j] = s;
      kmax = max(kmax, key);
      atomicAdd(&lh[score_bin(key)], 1u);
    }
  };
  // Group numbers only grow along a wave (the first kFirst are static, the rest
  // come from the counter), so the first one past the end ends the wave.  The
  // wave holding group `mid` stops there, flushes the histogram so far and
  // restarts: the pipelined loop itself holds no global write, which keeps the
  // compiler's waits for the key loads exact.
  int qa = wave, qb = wave + kSelWaves, qc = wave + 2 * kSelWaves;
  int stop = (qa == mid || qb == mid || qc == mid) ? mid : n_grp;
  while (true) {
    __builtin_amdgcn_s_waitcnt(0);  // (re)start with nothing in flight
    KeyGroup<MX> g0, g1, g2;
    load(g0, qa);
    __builtin_amdgcn_sched_barrier(0);  // g0's loads go out before g1's, as in the loop
    load(g1, qb);
    // three named buffers, unrolled by three (see indexer_mfma_kernel)
    while (true) {
      if (qa >= stop) break;
      load(g2, qc);
      const int qd = grab();
      if (qd == mid) stop = mid;
      step(g0, qa);
      if (qb >= stop) {
        qa = qb; qb = qc; qc = qd;
        break;
      }
      load(g0, qd);
      const int qe = grab();
      if (qe == mid) stop = mid;
      step(g1, qb);
      if (qc >= stop) {
        qa = qc; qb = qd; qc = qe;
        break;
      }
      load(g1, qe);
      const int qf = grab();
      if (qf == mid) stop = mid;
      step(g2, qc);
      qa = qd; qb = qe; qc = qf;
    }
    if (qa >= n_grp) break;
    // qa == mid: about half of the workgroup's groups are done
    uint32_t* gh = sel.hist + row * kScoreHistBins;
    for (int i = lane; i < kScoreHistBins; i += kWave) {
      const uint32_t c = atomicExch(&lh[i], 0u);
      if (c) atomicAdd(&gh[hist_slot(i)], c);
    }
    stop = n_grp;
  }
  __syncthreads();
  select_emit<kSelWaves>(lh, sc, n_t, wi, wpr, vis, row, sel, k, kmax);
}

// ---------------------------------------------------------------------------
// Many query rows (prefill): kRowsPerWG consecutive query rows of one sequence
// per workgroup, one per wave.  The rows' keys stream through LDS in 128-key
// tiles (double-buffered, staged through registers), so a key leaves L2 once
// per kRowsPerWG rows instead of once per row; each wave keeps its row's query
// tiles in registers and runs every key group of a tile against them.  Several
// waves per SIMD hide the MFMA -> ReLU/weights -> store chain of each wave.
// LDS key rows are padded to 144 (fp8) / 80 (MXFP4) bytes so that the B-operand
// reads of 8 consecutive keys hit distinct banks.
constexpr int kRowsPerWG = 8;
constexpr int kRowsThreads = kWave * kRowsPerWG;
constexpr int kTileKeys = 64;

template <bool MX, typename ST>
__global__ __launch_bounds__(kRowsThreads, 2) void indexer_rows_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale,
    const uint8_t* __restrict__ kI, const uint8_t* __restrict__ kI_scale, int n_q, int N_cap,
    int groups_per_seq, const float* __restrict__ w, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, ST* __restrict__ scores) {
  constexpr int kRowBytes = MX ? 64 : 128;
  constexpr int kLdsRow = kRowBytes + 16;
  constexpr int kChunks = kTileKeys * kRowBytes / 16;  // 16-byte chunks per tile
  constexpr int kChunksPerThread = (kChunks + kRowsThreads - 1) / kRowsThreads;
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][kTileKeys * kLdsRow];
  __shared__ uint32_t kts[2][MX ? kTileKeys : 1];
  __shared__ __attribute__((aligned(16))) float w_s[kRowsPerWG][64];
  __shared__ int vis_s[kRowsPerWG];
  const int b = blockIdx.x / groups_per_seq;
  const int r0 = (blockIdx.x % groups_per_seq) * kRowsPerWG;  // first row within the sequence
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, g = lane >> 5;
  const long long row_base = static_cast<long long>(b) * n_q;
  if (tid < kRowsPerWG) {
    const int r = r0 + tid;
    vis_s[tid] = r < n_q ? visible_entries(q_pos[row_base + r], m, n_entries[b], N_cap) : 0;
  }
  for (int i = tid; i < kRowsPerWG * 64; i += kRowsThreads) {
    const int r = r0 + i / 64;
    w_s[i / 64][i % 64] = r < n_q ? w[(row_base + r) * 64 + i % 64] : 0.f;
  }
  // the wave's row (a row past n_q computes on the last row and stores nothing)
  v8i A[2][2];
  int sA[2][2];
  load_query<MX>(qI, qI_scale, row_base + min(r0 + wave, n_q - 1), j, g, A, sA);
  __syncthreads();
  int vis_max = 0;
#pragma unroll
  for (int u = 0; u < kRowsPerWG; ++u) vis_max = max(vis_max, vis_s[u]);
  // the 32 head weights this lane applies, kept in registers for every key group
  float4 wr[8];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int a = 0; a < 4; ++a) wr[4 * ht + a] = *reinterpret_cast<const float4*>(&w_s[wave][32 * ht + 8 * a + 4 * g]);
  const int vis = vis_s[wave];
  const int n_tiles = (vis_max + kTileKeys - 1) / kTileKeys;
  if (n_tiles == 0) return;
  const uint8_t* kb_base = kI + static_cast<size_t>(b) * N_cap * kRowBytes;
  const uint8_t* ks_base = MX ? kI_scale + static_cast<size_t>(b) * N_cap * 4 : nullptr;
  ST* out = scores + static_cast<size_t>(row_base + r0 + wave) * N_cap;

  // tile staging: chunk c = tid + 512 i is bytes 16 (c % (kRowBytes/16)) of key
  // c / (kRowBytes/16); keys past vis_max load the last visible key
  uint4 st[kChunksPerThread];
  uint32_t sts = 0;
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int c = min(tid + kRowsThreads * i, kChunks - 1);
      const int key = min(t * kTileKeys + c / (kRowBytes / 16), vis_max - 1);
      st[i] = *reinterpret_cast<const uint4*>(kb_base + static_cast<size_t>(key) * kRowBytes +
                                              16 * (c % (kRowBytes / 16)));
    }
    if (MX) {
      const int key = min(t * kTileKeys + (tid & (kTileKeys - 1)), vis_max - 1);
      sts = *reinterpret_cast<const uint32_t*>(ks_base + static_cast<size_t>(key) * 4);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int c = tid + kRowsThreads * i;
      if (c < kChunks)
        *reinterpret_cast<uint4*>(&kt[buf][(c / (kRowBytes / 16)) * kLdsRow + 16 * (c % (kRowBytes / 16))]) = st[i];
    }
    if (MX && tid < kTileKeys) kts[buf][tid] = sts;
  };
  load_tile(0);
  store_tile(0);
  __syncthreads();
  // Tile t+1 goes into the other buffer while tile t is computed: that buffer
  // held tile t-1, which every wave finished before the barrier ending step t-1.
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);  // in flight during this tile
    auto lds_group = [&](int grp) {
      const int kl = kKeysPerGroup * grp + j;  // key within the tile
      const uint8_t* kp = &kt[buf][kl * kLdsRow];
      KeyGroup<MX> G;
      if (MX) {
        const uint32_t sc = kts[buf][kl];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int blk = 2 * g + ks;
          G.b[ks] = load16(kp + 16 * blk);
          G.sb[ks] = (sc >> (8 * blk)) & 0xff;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          G.b[ks] = load32(kp + 64 * g + 32 * ks);
          G.sb[ks] = 127;
        }
      }
      return G;
    };
    // the next group's MFMAs are issued before this group's reduction
    constexpr int kGroups = kTileKeys / kKeysPerGroup;
    GroupAcc acc[kGroups];
    acc[0] = group_mma<MX>(A, sA, lds_group(0));
#pragma unroll
    for (int grp = 0; grp < kGroups; ++grp) {
      if (grp + 1 < kGroups) acc[grp + 1] = group_mma<MX>(A, sA, lds_group(grp + 1));
      const float sv = group_reduce_reg(acc[grp], wr);
      const int key = t * kTileKeys + kKeysPerGroup * grp + j;
      if (g == 0 && key < vis) store_score(&out[key], sv);
      if (grp + 1 < kGroups) {
        // the next group's four MFMAs spread over this group's epilogue (one per
        // 16 VALU operations) instead of issued back to back ahead of it
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // sixteen VALU
        }
      }
    }
    if (t + 1 < n_tiles) {
      store_tile(buf ^ 1);
      __syncthreads();
    }
  }
}

// Scalar fp32 path for small shapes: one thread per (query, entry).
constexpr int kF32Threads = 256;

template <typename ST>
__global__ __launch_bounds__(kF32Threads) void indexer_f32_kernel(
    const float* __restrict__ qI, const float* __restrict__ kI, int n_q, int H_I, int d_I,
    int N_cap, int n_chunks, const float* __restrict__ w, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, ST* __restrict__ scores) {
  extern __shared__ float sm[];  // [H_I * d_I] query, then [H_I] weights
  const long long row = blockIdx.x / n_chunks;
  const int chunk = blockIdx.x % n_chunks;
  const int b = static_cast<int>(row / n_q);
  const int vis = visible_entries(q_pos[row], m, n_entries[b], N_cap);
  const int s0 = chunk * kF32Threads;
  if (s0 >= vis) return;
  const int HD = H_I * d_I;
  for (int i = threadIdx.x; i < HD; i += kF32Threads) sm[i] = qI[static_cast<size_t>(row) * HD + i];
  for (int i = threadIdx.x; i < H_I; i += kF32Threads) sm[HD + i] = w[static_cast<size_t>(row) * H_I + i];
  __syncthreads();
  const int s = s0 + threadIdx.x;
  if (s >= vis) return;
  const float* kp = kI + (static_cast<size_t>(b) * N_cap + s) * d_I;
  float acc = 0.f;
  for (int h = 0; h < H_I; ++h) {
    const float* qp = sm + h * d_I;
    float d = 0.f;
    for (int i = 0; i < d_I; ++i) d = fmaf(qp[i], kp[i], d);
    acc = fmaf(sm[HD + h], fmaxf(d, 0.f), acc);
  }
  store_score(&scores[static_cast<size_t>(row) * N_cap + s], acc);
}

}  // namespace

// Compute units of the current device, asked on every call (a host-side
// attribute lookup): the library keeps no per-process cache of it.
static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    return cus;
  return 256;
}

// The fused selection keeps up to kSelMaxBlocks blocks of scores in dynamic
// LDS, above the default limit: the kernel's limit is raised once per device
// and kernel instance (std::call_once, so concurrent first calls from several
// host threads are safe), and the result of that call is kept with it.
constexpr int kMaxDevices = 64;

template <bool MX>
static hipError_t select_lds_limit() {
  static std::once_flag once[kMaxDevices];
  static hipError_t result[kMaxDevices];
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    result[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(indexer_select_kernel<MX>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                      static_cast<int>(sizeof(float) * kBlockKeys * kSelMaxBlocks));
  });
  return result[dev];
}

hipError_t launch_indexer(int B, int n_q, int H_I, int d_I, int idx_fmt, const void* qI,
                          const uint8_t* qI_scale, const void* kI, const uint8_t* kI_scale,
                          int N_cap, const float* w, const int32_t* q_pos, int m,
                          const int32_t* n_entries, void* scores, hipStream_t s,
                          uint32_t* hist, hipEvent_t ev_start, hipEvent_t ev_stop,
                          const SelectWs* sel, int k, int score_fmt, int32_t* sel_idx,
                          const StateAppend* app) {
  const long long rows = static_cast<long long>(B) * n_q;
  if (rows == 0 || N_cap == 0) return hipSuccess;
  if (score_fmt != LCA_F32 && score_fmt != LCA_BF16) return hipErrorInvalidValue;
  const bool sbf = score_fmt == LCA_BF16;
  float* sf = static_cast<float*>(scores);
  uint16_t* sb = static_cast<uint16_t*>(scores);
  if (idx_fmt == LCA_F32) {
    if (sel) return hipErrorInvalidValue;  // the selecting kernel is MFMA-only
    const int n_chunks = (N_cap + kF32Threads - 1) / kF32Threads;
    const size_t lds = sizeof(float) * (static_cast<size_t>(H_I) * d_I + H_I);
    const dim3 g(static_cast<unsigned>(rows * n_chunks));
    auto go = [&](auto kern, auto* out) {
      if (ev_start || ev_stop)
        hipExtLaunchKernelGGL(kern, g, dim3(kF32Threads), lds, s, ev_start, ev_stop, 0,
                              static_cast<const float*>(qI), static_cast<const float*>(kI), n_q, H_I,
                              d_I, N_cap, n_chunks, w, q_pos, m, n_entries, out);
      else
        hipLaunchKernelGGL(kern, g, dim3(kF32Threads), lds, s, static_cast<const float*>(qI),
                           static_cast<const float*>(kI), n_q, H_I, d_I, N_cap, n_chunks, w, q_pos,
                           m, n_entries, out);
    };
    if (sbf) go(indexer_f32_kernel<uint16_t>, sb);
    else go(indexer_f32_kernel<float>, sf);
    return hipGetLastError();
  }
  const long long max_blocks = (N_cap + kBlockKeys - 1) / kBlockKeys;
  const uint8_t* q8 = static_cast<const uint8_t*>(qI);
  const uint8_t* k8 = static_cast<const uint8_t*>(kI);
  const bool mx = idx_fmt == LCA_MXFP4;
  if (sel) {
    // one workgroup per CU in a single round when the row's blocks fit in
    // floor(CUs / rows) workgroups' LDS, else more workgroups (and rounds)
    long long wpr = std::max<long long>(device_cus() / rows,
                                        (max_blocks + kSelMaxBlocks - 1) / kSelMaxBlocks);
    wpr = std::min(wpr, max_blocks);
    if (wpr > kSelMaxWpr || !select_supported(N_cap, k) || sel_idx == nullptr) return hipErrorInvalidValue;
    const size_t lds = sizeof(float) * kBlockKeys * static_cast<size_t>((max_blocks + wpr - 1) / wpr);
    const dim3 grid(static_cast<unsigned>(rows * wpr)), block(kSelThreads);
    const int iw = static_cast<int>(wpr);
    const SelectWs so = *sel;
    hipError_t e = mx ? select_lds_limit<true>() : select_lds_limit<false>();
    if (e != hipSuccess) return e;
    auto go = [&](auto kern) {
      if (ev_start || ev_stop)
        hipExtLaunchKernelGGL(kern, grid, block, lds, s, ev_start, ev_stop, 0, q8, qI_scale, k8,
                              kI_scale, n_q, N_cap, iw, w, q_pos, m, n_entries, so, k, sel_idx);
      else
        hipLaunchKernelGGL(kern, grid, block, lds, s, q8, qI_scale, k8, kI_scale, n_q, N_cap, iw, w,
                           q_pos, m, n_entries, so, k, sel_idx);
    };
    if (mx) go(indexer_select_kernel<true>);
    else go(indexer_select_kernel<false>);
    if (e != hipSuccess || (e = hipGetLastError()) != hipSuccess) return e;
    return launch_select_finish(rows, n_q, N_cap, iw, q_pos, m, n_entries, k, so, sel_idx, s, app);
  }
  if (app) return hipErrorInvalidValue;  // the append rides on the finish pass only
  if (!hist && n_q >= kRowsPerWG * 8) {
    // many rows per sequence: row groups share each key tile through LDS
    const int gps = (n_q + kRowsPerWG - 1) / kRowsPerWG;
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(B) * gps)), block(kRowsThreads);
    auto go = [&](auto kern, auto* out) {
      if (ev_start || ev_stop)
        hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev_start, ev_stop, 0, q8, qI_scale, k8,
                              kI_scale, n_q, N_cap, gps, w, q_pos, m, n_entries, out);
      else
        hipLaunchKernelGGL(kern, grid, block, 0, s, q8, qI_scale, k8, kI_scale, n_q, N_cap, gps, w,
                           q_pos, m, n_entries, out);
    };
    if (mx) sbf ? go(indexer_rows_kernel<true, uint16_t>, sb) : go(indexer_rows_kernel<true, float>, sf);
    else sbf ? go(indexer_rows_kernel<false, uint16_t>, sb) : go(indexer_rows_kernel<false, float>, sf);
    return hipGetLastError();
  }
  long long wpr = (kTargetBlocks + rows - 1) / rows;
  wpr = wpr < 1 ? 1 : (wpr > max_blocks ? max_blocks : wpr);
  const dim3 grid(static_cast<unsigned>(rows * wpr));
  const int n_chunks = static_cast<int>(wpr);
  const dim3 block(kWave * kIdxWaves);
  // start/stop events, when given, are stamped by the dispatch itself
  auto go = [&](auto kern, auto* out) {
    if (ev_start || ev_stop)
      hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev_start, ev_stop, 0, q8, qI_scale, k8,
                            kI_scale, n_q, N_cap, n_chunks, w, q_pos, m, n_entries, out, hist);
    else
      hipLaunchKernelGGL(kern, grid, block, 0, s, q8, qI_scale, k8, kI_scale, n_q, N_cap, n_chunks,
                         w, q_pos, m, n_entries, out, hist);
  };
  if (sbf) {
    if (!mx) {
      if (hist) go(indexer_mfma_kernel<false, true, uint16_t>, sb);
      else go(indexer_mfma_kernel<false, false, uint16_t>, sb);
    } else {
      if (hist) go(indexer_mfma_kernel<true, true, uint16_t>, sb);
      else go(indexer_mfma_kernel<true, false, uint16_t>, sb);
    }
  } else {
    if (!mx) {
      if (hist) go(indexer_mfma_kernel<false, true, float>, sf);
      else go(indexer_mfma_kernel<false, false, float>, sf);
    } else {
      if (hist) go(indexer_mfma_kernel<true, true, float>, sf);
      else go(indexer_mfma_kernel<true, false, float>, sf);
    }
  }
  return hipGetLastError();
}

}  // namespace lca
