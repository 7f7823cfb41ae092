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
    p[i].sum = fmaf(p[i].sum, sc, e);
    p[i].acc = fmaf(p[i].acc, sc, e * cv[i]);  // written out: two products, one sum
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
  if (wv < kPoolWaves) {  // a larger workgroup's other waves only meet the barrier
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      part[wv][0][j][lane] = pool[j].mx;
      part[wv][1][j][lane] = pool[j].sum;
      part[wv][2][j][lane] = pool[j].acc;
    }
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
template <int CPL, int IOF, int kBatch = (CPL > 8 ? 1 : 4)>
__device__ __forceinline__ void pool_tail(int csa, int m, int T_cap, int half, int s, int row,
                                          const uint8_t* tCb, const uint8_t* tZb, const float* P,
                                          int c, int lane, int wv, const float* tc, const float* tz,
                                          Pool* pool) {
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

// One workgroup of kAppendWaves waves per sequence: append the token, and
// compress its block when the token completes it.  The block's candidate slots
// are pooled as in compress_kernel (slot j by one wave, each wave an online
// per-channel softmax over its slots in increasing order, the partial states
// combined in slot order through LDS), so the entry has the bits the prefill
// compressor gives it and does not depend on timing.  Tail rows other than the
// new token were written by earlier steps; the new token's row is used from
// registers.  As a side job the workgroups clear zero_buf.
constexpr int kAppendWaves = kPoolWaves;

// Sequence b's append, by the workgroup's first kAppendWaves waves (a larger
// workgroup's other waves only take part in its barriers); b is also this
// workgroup's index among the n_wg that share the side job.  part: LDS scratch
// of kAppendWaves x 3 x CPL x kWave floats.  LEAN: no speculative tail loads and
// one candidate row per load batch (fewer registers, one more memory round
// trip; the same slots per wave and the same combination order, so the same
// bits).
template <int CPL, int IOF, bool LEAN = false>
__device__ __forceinline__ void state_append_body(
    int b, int n_wg, float (*part)[3][CPL][kWave], int csa, int m, int c, int n_win,
    const uint8_t* tokC, const uint8_t* tokZ, uint8_t* tailC, uint8_t* tailZ, uint8_t* ring,
    int kv_fmt, const float* P, uint8_t* cache, int N_cap, int32_t* n_tokens, int32_t* q_pos,
    int32_t* n_entries, float eps, double rope_step, const KvPages& pg, uint32_t* zero_buf,
    long long zero_words) {
  constexpr int io_fmt = IOF;  // compile-time: no format branches around the row loads
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  for (long long i = static_cast<long long>(b) * blockDim.x + threadIdx.x; i < zero_words;
       i += static_cast<long long>(n_wg) * blockDim.x)
    zero_buf[i] = 0u;
  const size_t io_row = row_bytes(io_fmt, c);
  const size_t kv_row = row_bytes(kv_fmt, c);
  const int T_cap = csa ? 2 * m : m;
  uint8_t* tCb = tailC + static_cast<size_t>(b) * T_cap * io_row;
  uint8_t* tZb = tailZ + static_cast<size_t>(b) * T_cap * io_row;
  // A CSA tail of at most kAppendWaves rows is read speculatively (one row per
  // wave, with the bias rows of both slots that row can take) before the token
  // count arrives, so that the step pays one memory latency.
  const bool spec = !LEAN && CPL <= 8 && csa && T_cap <= kAppendWaves;
  float sc[CPL], sz[CPL], sp0[CPL], sp1[CPL];
  if (spec && wv < T_cap) {
    load_row<CPL>(tCb + wv * io_row, io_fmt, c, lane, sc);
    load_row<CPL>(tZb + wv * io_row, io_fmt, c, lane, sz);
    load_bias<CPL>(P, wv % m, c, lane, sp0);
    load_bias<CPL>(P, m + wv % m, c, lane, sp1);
  }
  float tc[CPL], tz[CPL];
  load_row<CPL>(tokC + static_cast<size_t>(b) * io_row, io_fmt, c, lane, tc);
  load_row<CPL>(tokZ + static_cast<size_t>(b) * io_row, io_fmt, c, lane, tz);
  const int p = n_tokens[b];
  if (p < 0) return;  // the same for every wave
  // every wave has read the count before wave 0 advances it below
  __syncthreads();
  const int blk = p / m;
  const int half = csa ? (blk & 1) : 0;
  const int row = half * m + p % m;
  float2 rope_p = make_float2(1.f, 0.f);
  if (wv == 0) {
    store_row<CPL>(tCb + row * io_row, io_fmt, c, lane, tc);
    store_row<CPL>(tZb + row * io_row, io_fmt, c, lane, tz);
    // window KV of the new token
    float u[CPL];
    window_row<CPL>(tc, c, eps, u);
    if (rope_step != 0.0) {
      rope_p = rope_cs_lane(p, rope_step);  // also the angles of an entry this token completes
      rope_lane<CPL>(u, lane, c, rope_p);
    }
    store_row<CPL>(ring + (static_cast<size_t>(b) * n_win + p % n_win) * kv_row, kv_fmt, c, lane, u);
    if (lane == 0) {
      n_tokens[b] = p + 1;
      if (q_pos) {
        q_pos[b] = p;
        const int ne = (p + 1) / m;
        n_entries[b] = ne < N_cap ? ne : N_cap;
      }
    }
  }
  if ((p + 1) % m != 0) return;

  // candidate slots: CSA slot j < m is the previous block's token j (tail row
  // (1-half)*m + j, absent for the first entry), slot m + j the own block's
  // token j (row half*m + j); HCA slot j is row j.  The new token's row is
  // taken from registers.
  const int s = (p + 1) / m - 1;
  // the new entry's row in the cache (through the block table when paged),
  // looked up before the candidate loads; -1: beyond N_cap or an absent page
  const long long out_row = (wv == 0 && s < N_cap) ? kv_row_of(pg, b, N_cap, s) : -1;
  if (LCA_DEVICE_CHECKS && wv == 0 && lane == 0 && s < N_cap) dbg_check(out_row >= 0);
  Pool pool[CPL];
  pool_init<CPL>(pool);
  auto add_row = [&](const float* rc, const float* rz, const float* bias) {
    float zv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) zv[j] = rz[j] + bias[j];
    pool_add<CPL>(pool, rc, zv);
  };
  int order[kPoolWaves];  // order[x]: the wave that pooled slot group x
  if (spec) {
    // wave wv holds tail row wv (loaded before the count was known): its slot
    // is m + wv % m in the own half, wv % m in the other
    if (wv < T_cap) {
      const bool own = (wv / m) == half;
      if (own || s > 0) add_row(wv == row ? tc : sc, wv == row ? tz : sz, own ? sp1 : sp0);
    }
#pragma unroll
    for (int x = 0; x < kPoolWaves; ++x)
      order[x] = x < T_cap ? (x < m ? (1 - half) * m + x : half * m + (x - m)) : x;
  } else {
    if (wv < kAppendWaves)
      pool_tail<CPL, IOF, LEAN ? 1 : (CPL > 8 ? 1 : 4)>(csa, m, T_cap, half, s, row, tCb, tZb, P, c,
                                                       lane, wv, tc, tz, pool);
#pragma unroll
    for (int x = 0; x < kPoolWaves; ++x) order[x] = x;
  }
  float out[CPL];
  if (!pool_combine_norm<CPL>(part, pool, order, wv, lane, c, eps, out)) return;
  if (rope_step != 0.0) rope_lane<CPL>(out, lane, c, rope_p);  // the entry's last token is p
  if (out_row >= 0) store_row<CPL>(cache + static_cast<size_t>(out_row) * kv_row, kv_fmt, c, lane, out);
}

}  // namespace lca
