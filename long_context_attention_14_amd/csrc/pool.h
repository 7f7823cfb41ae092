// Softmax-gated pooling of candidate rows into one compressed entry, shared by
// the compressor, the decode-time state append and the decode attention kernel
// that appends HCA tokens itself ("DeepSeek V4 Architecture Tricks", section
// "压缩 KV 的具体 trick": a per-channel softmax over the gate logits plus a
// learned positional bias of the candidates, applied to their KV values, then
// RMSNorm).  Every caller pools the same slots in the same waves and combines
// the waves' states in the same order, so every path gives an entry the same
// bits.
#pragma once
#include "common.h"

namespace lca {

struct Pool {
  float mx, sum, acc;
};

template <int CPL>
__device__ __forceinline__ void pool_init(Pool* p) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) p[i] = {-INFINITY, 0.f, 0.f};
}

// Online softmax update of one candidate (KV values c, logits z).
template <int CPL>
__device__ __forceinline__ void pool_add(Pool* p, const float* cv, const float* zv) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const float nm = fmaxf(p[i].mx, zv[i]);
    const float sc = __expf(p[i].mx - nm);
    const float e = __expf(zv[i] - nm);
    p[i].sum = p[i].sum * sc + e;
    p[i].acc = p[i].acc * sc + e * cv[i];
    p[i].mx = nm;
  }
}

// E / sqrt(mean(E^2) + eps) across the wave's c channels.
template <int CPL>
__device__ __forceinline__ void pool_finish_norm(const Pool* p, int c, float eps, float* out) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    out[i] = p[i].acc * __builtin_amdgcn_rcpf(p[i].sum);
    ss += out[i] * out[i];
  }
  ss = wave_sum(ss);
  const float r = rsqrt_hw(ss / static_cast<float>(c) + eps);
#pragma unroll
  for (int i = 0; i < CPL; ++i) out[i] *= r;
}

constexpr int kPoolWaves = 8;

// The entry from the waves' partial pooling states: every wave stores its
// state, then wave 0 combines them in slot order -- order[x] is the wave that
// pooled the x-th slot group (a fixed order, so the result does not depend on
// timing) -- and RMS-normalises.  Returns true in wave 0, whose `out` then
// holds the entry.  Every wave of the workgroup must call it.
template <int CPL>
__device__ __forceinline__ bool pool_combine_norm(float (*part)[3][CPL][kWave], const Pool* pool,
                                                  const int (&order)[kPoolWaves], int wv, int lane,
                                                  int c, float eps, float* out) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    part[wv][0][j][lane] = pool[j].mx;
    part[wv][1][j][lane] = pool[j].sum;
    part[wv][2][j][lane] = pool[j].acc;
  }
  __syncthreads();
  if (wv != 0) return false;
  Pool tot[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < kPoolWaves; ++x) M = fmaxf(M, part[order[x]][0][j][lane]);
    float sum = 0.f, acc = 0.f;
#pragma unroll
    for (int x = 0; x < kPoolWaves; ++x) {
      const float mx = part[order[x]][0][j][lane];
      const float f = mx == -INFINITY ? 0.f : __expf(mx - M);
      sum += part[order[x]][1][j][lane] * f;
      acc += part[order[x]][2][j][lane] * f;
    }
    tot[j] = {M, sum, acc};
  }
  pool_finish_norm<CPL>(tot, c, eps, out);
  return true;
}

template <int CPL>
__device__ __forceinline__ void load_bias(const float* P, int slot, int c, int lane, float* pv) {
  load_row<CPL>(P + static_cast<size_t>(slot) * c, LCA_F32, c, lane, pv);
}

// The window row of a new token: its KV candidate RMS-normalised (unit gain).
template <int CPL>
__device__ __forceinline__ void window_row(const float* tc, int c, float eps, float* u) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    u[j] = tc[j];
    ss += u[j] * u[j];
  }
  ss = wave_sum(ss);
  const float rs = rsqrt_hw(ss / static_cast<float>(c) + eps);
#pragma unroll
  for (int j = 0; j < CPL; ++j) u[j] *= rs;
}

// The tail block that a decode token completes, pooled by the kAppendWaves waves
// of a workgroup: wave wv takes slots wv, wv + kPoolWaves, ... in increasing
// order, kBatch slots' rows loaded before any is pooled (a long HCA tail pays
// one memory latency per batch).  CSA slot j < m is the previous block's token
// j (tail row (1-half)*m + j, absent for the first entry s == 0), slot m + j
// the own block's token j (row half*m + j); HCA slot j is tail row j.  The new
// token's row (`row`) is taken from registers (tc, tz): it may not have reached
// memory.  The waves' states are then combined in slot-group order 0, 1, ...
template <int CPL, int IOF>
__device__ __forceinline__ void pool_tail(int csa, int m, int T_cap, int half, int s, int row,
                                          const uint8_t* tCb, const uint8_t* tZb, const float* P,
                                          int c, int lane, int wv, const float* tc, const float* tz,
                                          Pool* pool) {
  constexpr int kBatch = CPL > 8 ? 1 : 4;
  const size_t io_row = row_bytes(IOF, c);
  auto add_row = [&](const float* rc, const float* rz, const float* bias) {
    float zv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) zv[j] = rz[j] + bias[j];
    pool_add<CPL>(pool, rc, zv);
  };
  for (int j0 = wv; j0 < T_cap; j0 += kPoolWaves * kBatch) {
    float bc[kBatch][CPL], bz[kBatch][CPL], bb[kBatch][CPL];
    bool use[kBatch], mine[kBatch];
    // unconditional loads (slots past the tail read slot j0's rows and are not
    // used): a load under a branch would be waited for at the branch's end
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + kPoolWaves * u;
      const int jl = j < T_cap ? j : j0;
      const bool prev = csa && jl < m;
      const int r = csa ? (prev ? (1 - half) * m + jl : half * m + (jl - m)) : jl;
      use[u] = j < T_cap && (!prev || s > 0);
      mine[u] = r == row;
      load_row<CPL>(tCb + r * io_row, IOF, c, lane, bc[u]);
      load_row<CPL>(tZb + r * io_row, IOF, c, lane, bz[u]);
      load_bias<CPL>(P, jl, c, lane, bb[u]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (!use[u]) continue;  // the same for the whole wave
      if (mine[u]) add_row(tc, tz, bb[u]);
      else add_row(bc[u], bz[u], bb[u]);
    }
  }
}

}  // namespace lca
