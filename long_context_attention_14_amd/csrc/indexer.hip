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
constexpr int kPrefetch = 2;

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

// HIST: also accumulate the score_bin histogram of the written scores into
// hist[row] (global, zeroed by the caller) through a per-workgroup LDS histogram.
template <bool MX, bool HIST>
__global__ __launch_bounds__(kWave * kIdxWaves, 3) void indexer_mfma_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qI_scale,
    const uint8_t* __restrict__ kI, const uint8_t* __restrict__ kI_scale, int n_q, int N_cap,
    int wpr, const float* __restrict__ w, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, float* __restrict__ scores,
    uint32_t* __restrict__ hist) {
  constexpr int kFmt = MX ? 4 : 0;
  constexpr int kRowBytes = MX ? 64 : 128;  // bytes of one 128-dim vector
  __shared__ uint32_t lh[HIST ? kScoreHistBins : 1];
  const long long row = blockIdx.x / wpr;
  const int wi = blockIdx.x % wpr;
  const int b = static_cast<int>(row / n_q);
  const int vis = visible_entries(q_pos[row], m, n_entries[b], N_cap);
  if (wi * kBlockKeys >= vis) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int j = lane & 31;
  const int g = lane >> 5;
  if (HIST) {
    for (int i = threadIdx.x; i < kScoreHistBins; i += kWave * kIdxWaves) lh[i] = 0;
  }

  // A operand: query heads 32*ht + j, K-steps ks = 0, 1
  v8i A[2][2];
  int sA[2][2];
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
  // head weights in LDS: register r of accumulator tile ht is head
  // 32*ht + 8*(r/4) + 4*g + (r%4), so four consecutive registers read one float4
  __shared__ __attribute__((aligned(16))) float w_s[64];
  if (threadIdx.x < 64) w_s[threadIdx.x] = w[static_cast<size_t>(row) * 64 + threadIdx.x];

  const uint8_t* kb_base = kI + static_cast<size_t>(b) * N_cap * kRowBytes;
  const uint8_t* ks_base = MX ? kI_scale + static_cast<size_t>(b) * N_cap * 4 : nullptr;
  float* out = scores + static_cast<size_t>(row) * N_cap;
  __syncthreads();

  // this wave's groups: keys [kb, kb + 32) for kb = wi*128 + 32*wave + t*stride
  const int stride = kBlockKeys * wpr;
  int kb = wi * kBlockKeys + wave * kKeysPerGroup;
  KeyGroup<MX> buf[kPrefetch];
#pragma unroll
  for (int p = 0; p < kPrefetch; ++p) {
    const int kk = kb + p * stride;
    if (kk < vis) load_group<MX>(kb_base, ks_base, min(kk + j, vis - 1), g, buf[p]);
  }
  for (; kb < vis; kb += stride) {
    KeyGroup<MX> nxt;
    const int kn = kb + kPrefetch * stride;
    if (kn < vis) load_group<MX>(kb_base, ks_base, min(kn + j, vis - 1), g, nxt);
    const KeyGroup<MX>& cur = buf[0];
    v16f acc0 = {0}, acc1 = {0};
    acc0 = mfma<kFmt>(A[0][0], cur.b[0], acc0, sA[0][0], cur.sb[0]);
    acc0 = mfma<kFmt>(A[0][1], cur.b[1], acc0, sA[0][1], cur.sb[1]);
    acc1 = mfma<kFmt>(A[1][0], cur.b[0], acc1, sA[1][0], cur.sb[0]);
    acc1 = mfma<kFmt>(A[1][1], cur.b[1], acc1, sA[1][1], cur.sb[1]);
    float s = 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 w4 = *reinterpret_cast<const float4*>(&w_s[8 * a + 4 * g]);
      s += w4.x * fmaxf(acc0[4 * a], 0.f);
      s += w4.y * fmaxf(acc0[4 * a + 1], 0.f);
      s += w4.z * fmaxf(acc0[4 * a + 2], 0.f);
      s += w4.w * fmaxf(acc0[4 * a + 3], 0.f);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 w4 = *reinterpret_cast<const float4*>(&w_s[32 + 8 * a + 4 * g]);
      s += w4.x * fmaxf(acc1[4 * a], 0.f);
      s += w4.y * fmaxf(acc1[4 * a + 1], 0.f);
      s += w4.z * fmaxf(acc1[4 * a + 2], 0.f);
      s += w4.w * fmaxf(acc1[4 * a + 3], 0.f);
    }
    s += __shfl_xor(s, 32, kWave);
    if (g == 0 && kb + j < vis) {
      out[kb + j] = s;
      if (HIST) atomicAdd(&lh[score_bin(score_key(s))], 1u);
    }
#pragma unroll
    for (int p = 0; p < kPrefetch - 1; ++p) buf[p] = buf[p + 1];
    buf[kPrefetch - 1] = nxt;
  }
  if (HIST) {
    __syncthreads();
    uint32_t* gh = hist + row * kScoreHistBins;
    for (int i = threadIdx.x; i < kScoreHistBins; i += kWave * kIdxWaves)
      if (lh[i]) atomicAdd(&gh[i], lh[i]);
  }
}

// Scalar fp32 path for small shapes: one thread per (query, entry).
constexpr int kF32Threads = 256;

__global__ __launch_bounds__(kF32Threads) void indexer_f32_kernel(
    const float* __restrict__ qI, const float* __restrict__ kI, int n_q, int H_I, int d_I,
    int N_cap, int n_chunks, const float* __restrict__ w, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, float* __restrict__ scores) {
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
  scores[static_cast<size_t>(row) * N_cap + s] = acc;
}

}  // namespace

hipError_t launch_indexer(int B, int n_q, int H_I, int d_I, int idx_fmt, const void* qI,
                          const uint8_t* qI_scale, const void* kI, const uint8_t* kI_scale,
                          int N_cap, const float* w, const int32_t* q_pos, int m,
                          const int32_t* n_entries, float* scores, hipStream_t s,
                          uint32_t* hist, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const long long rows = static_cast<long long>(B) * n_q;
  if (rows == 0 || N_cap == 0) return hipSuccess;
  if (idx_fmt == LCA_F32) {
    const int n_chunks = (N_cap + kF32Threads - 1) / kF32Threads;
    const size_t lds = sizeof(float) * (static_cast<size_t>(H_I) * d_I + H_I);
    const dim3 g(static_cast<unsigned>(rows * n_chunks));
    if (ev_start || ev_stop)
      hipExtLaunchKernelGGL(indexer_f32_kernel, g, dim3(kF32Threads), lds, s, ev_start, ev_stop, 0,
                            static_cast<const float*>(qI), static_cast<const float*>(kI), n_q, H_I,
                            d_I, N_cap, n_chunks, w, q_pos, m, n_entries, scores);
    else
      hipLaunchKernelGGL(indexer_f32_kernel, g, dim3(kF32Threads), lds, s,
                         static_cast<const float*>(qI), static_cast<const float*>(kI), n_q, H_I, d_I,
                         N_cap, n_chunks, w, q_pos, m, n_entries, scores);
    return hipGetLastError();
  }
  const long long max_blocks = (N_cap + kBlockKeys - 1) / kBlockKeys;
  long long wpr = (kTargetBlocks + rows - 1) / rows;
  wpr = wpr < 1 ? 1 : (wpr > max_blocks ? max_blocks : wpr);
  const dim3 grid(static_cast<unsigned>(rows * wpr));
  const int n_chunks = static_cast<int>(wpr);
  const dim3 block(kWave * kIdxWaves);
  const uint8_t* q8 = static_cast<const uint8_t*>(qI);
  const uint8_t* k8 = static_cast<const uint8_t*>(kI);
  const bool mx = idx_fmt == LCA_MXFP4;
  // start/stop events, when given, are stamped by the dispatch itself
  auto go = [&](auto kern) {
    if (ev_start || ev_stop)
      hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev_start, ev_stop, 0, q8, qI_scale, k8, kI_scale,
                            n_q, N_cap, n_chunks, w, q_pos, m, n_entries, scores, hist);
    else
      hipLaunchKernelGGL(kern, grid, block, 0, s, q8, qI_scale, k8, kI_scale, n_q, N_cap, n_chunks, w,
                         q_pos, m, n_entries, scores, hist);
  };
  if (!mx && !hist)
    go(indexer_mfma_kernel<false, false>);
  else if (!mx)
    go(indexer_mfma_kernel<false, true>);
  else if (!hist)
    go(indexer_mfma_kernel<true, false>);
  else
    go(indexer_mfma_kernel<true, true>);
  return hipGetLastError();
}

}  // namespace lca
