// KV compressor, window-KV normalisation and decode-time state append.
//
// Compressor ("DeepSeek V4 Architecture Tricks", section "压缩 KV 的具体 trick";
// QbitAI article on DeepSeek-V4, hybrid attention section): each compressed
// entry is a per-channel softmax over the gate logits plus a learned
// positional bias of its candidate tokens, applied to their KV candidates;
// CSA's candidates are the previous block and the own block (2m tokens), HCA's
// the own block (m' tokens).  The entry is RMS-normalised (unit gain) and cast
// to the cache format.
//
// Mapping: one 64-lane wavefront per entry; lane l owns channels
// [l*CPL, (l+1)*CPL) with CPL = c/64, so every candidate row is one coalesced
// c-wide load per wave; the softmax is computed online per channel in
// registers and the RMSNorm sum of squares is a wavefront reduction.
#include "common.h"

namespace lca {
namespace {

constexpr int kWavesPerBlock = 4;

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

template <int CPL>
__device__ __forceinline__ void load_bias(const float* P, int slot, int c, int lane, float* pv) {
  load_row<CPL>(P + static_cast<size_t>(slot) * c, LCA_F32, c, lane, pv);
}

// IOF: the candidates' format (F32 or BF16) as a compile-time constant, so that
// row loads carry no format branches (a load under a branch makes the compiler
// wait for it at the branch's end, which serialises the candidate loads).
template <int CPL, int IOF>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void compress_kernel(
    int csa, int m, int B, int n_new, int c, const uint8_t* C, const uint8_t* Z,
    const uint8_t* prevC, const uint8_t* prevZ, const float* P, uint8_t* cache, int kv_fmt,
    int N_cap, int first_entry, float eps, double rope_step, KvPages pg) {
  constexpr int io_fmt = IOF;
  const int lane = threadIdx.x & (kWave - 1);
  const int n_ent = n_new / m;
  const long long e = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (e >= static_cast<long long>(B) * n_ent) return;
  const int b = static_cast<int>(e / n_ent);
  const int s = static_cast<int>(e % n_ent);
  // the entry's row in the cache (through the block table when paged), looked
  // up before the candidate loads
  const long long out_row = kv_row_of(pg, b, N_cap, first_entry + s);
  const size_t io_row = row_bytes(io_fmt, c);
  const uint8_t* Cb = C + static_cast<size_t>(b) * n_new * io_row;
  const uint8_t* Zb = Z + static_cast<size_t>(b) * n_new * io_row;

  Pool pool[CPL];
  pool_init<CPL>(pool);
  float cv[CPL], zv[CPL], pv[CPL];
  if (csa) {
    // slots 0..m-1: previous block (absent for the first entry without prevC)
    const bool have_prev = s > 0 || prevC != nullptr;
    if (have_prev) {
      for (int i = 0; i < m; ++i) {
        const uint8_t* rc = s > 0 ? Cb + (static_cast<size_t>(s - 1) * m + i) * io_row
                                  : prevC + (static_cast<size_t>(b) * m + i) * io_row;
        const uint8_t* rz = s > 0 ? Zb + (static_cast<size_t>(s - 1) * m + i) * io_row
                                  : prevZ + (static_cast<size_t>(b) * m + i) * io_row;
        load_row<CPL>(rc, io_fmt, c, lane, cv);
        load_row<CPL>(rz, io_fmt, c, lane, zv);
        load_bias<CPL>(P, i, c, lane, pv);
#pragma unroll
        for (int j = 0; j < CPL; ++j) zv[j] += pv[j];
        pool_add<CPL>(pool, cv, zv);
      }
    }
  }
  const int slot0 = csa ? m : 0;
  for (int i = 0; i < m; ++i) {
    const size_t r = static_cast<size_t>(s) * m + i;
    load_row<CPL>(Cb + r * io_row, io_fmt, c, lane, cv);
    load_row<CPL>(Zb + r * io_row, io_fmt, c, lane, zv);
    load_bias<CPL>(P, slot0 + i, c, lane, pv);
#pragma unroll
    for (int j = 0; j < CPL; ++j) zv[j] += pv[j];
    pool_add<CPL>(pool, cv, zv);
  }
  float out[CPL];
  pool_finish_norm<CPL>(pool, c, eps, out);
  // RoPE position of an entry: the last token it covers
  if (rope_step != 0.0)
    rope_lane<CPL>(out, lane, c,
                   rope_cs_lane((static_cast<long long>(first_entry) + s + 1) * m - 1, rope_step));
  const size_t kv_row = row_bytes(kv_fmt, c);
  if (out_row >= 0) store_row<CPL>(cache + static_cast<size_t>(out_row) * kv_row, kv_fmt, c, lane, out);
}

template <int CPL>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void rmsnorm_rows_kernel(
    int B, int n, int c, const uint8_t* x, int x_fmt, uint8_t* y, int y_fmt, int y_seq_rows,
    float eps, long long pos0, double rope_step) {
  const int lane = threadIdx.x & (kWave - 1);
  const long long r = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (r >= static_cast<long long>(B) * n) return;
  const int b = static_cast<int>(r / n);
  const int i = static_cast<int>(r % n);
  float v[CPL];
  load_row<CPL>(x + static_cast<size_t>(r) * row_bytes(x_fmt, c), x_fmt, c, lane, v);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) ss += v[j] * v[j];
  ss = wave_sum(ss);
  const float rs = rsqrt_hw(ss / static_cast<float>(c) + eps);
#pragma unroll
  for (int j = 0; j < CPL; ++j) v[j] *= rs;
  if (rope_step != 0.0) rope_lane<CPL>(v, lane, c, rope_cs_lane(pos0 + i, rope_step));
  store_row<CPL>(y + (static_cast<size_t>(b) * y_seq_rows + i) * row_bytes(y_fmt, c), y_fmt, c, lane,
                 v);
}

// One workgroup of kAppendWaves waves per sequence: append the token, and
// compress its block when the token completes it.  The block's candidates are
// spread over the waves (candidate j goes to wave j % kAppendWaves), each wave
// keeping an online per-channel softmax; the partial states are combined in
// wave order through LDS, so the result does not depend on timing.  Tail rows
// other than the new token were written by earlier steps; the new token's row is
// used from registers.  As a side job the workgroups clear zero_buf.
constexpr int kAppendWaves = 8;

template <int CPL, int IOF>
__global__ __launch_bounds__(kWave * kAppendWaves) void state_append_kernel(
    int csa, int m, int B, int c, int n_win, const uint8_t* tokC, const uint8_t* tokZ,
    uint8_t* tailC, uint8_t* tailZ, uint8_t* ring, int kv_fmt, const float* P, uint8_t* cache,
    int N_cap, int32_t* n_tokens, int32_t* q_pos, int32_t* n_entries, float eps, double rope_step,
    KvPages pg, uint32_t* zero_buf, long long zero_words) {
  constexpr int io_fmt = IOF;  // compile-time: no format branches around the row loads
  __shared__ float part[kAppendWaves][3][CPL][kWave];  // lane-contiguous: no bank conflicts
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int b = blockIdx.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < zero_words;
       i += static_cast<long long>(gridDim.x) * blockDim.x)
    zero_buf[i] = 0u;
  const size_t io_row = row_bytes(io_fmt, c);
  const size_t kv_row = row_bytes(kv_fmt, c);
  const int T_cap = csa ? 2 * m : m;
  uint8_t* tCb = tailC + static_cast<size_t>(b) * T_cap * io_row;
  uint8_t* tZb = tailZ + static_cast<size_t>(b) * T_cap * io_row;
  // A CSA tail of at most kAppendWaves rows is read speculatively (one row per
  // wave, with the bias rows of both slots that row can take) before the token
  // count arrives, so that the step pays one memory latency.
  const bool spec = CPL <= 8 && csa && T_cap <= kAppendWaves;
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
    if (rope_step != 0.0) {
      rope_p = rope_cs_lane(p, rope_step);  // also the angles of an entry this token completes
      rope_lane<CPL>(u, lane, c, rope_p);
    }
    store_row<CPL>(ring + (static_cast<size_t>(b) * n_win + p % n_win) * kv_row, kv_fmt, c, lane, u);
    if (lane == 0) {
      n_tokens[b] = p + 1;
      q_pos[b] = p;
      const int ne = (p + 1) / m;
      n_entries[b] = ne < N_cap ? ne : N_cap;
    }
  }
  if ((p + 1) % m != 0) return;

  // candidates, by physical tail row r: CSA rows of the current half are slots
  // m..2m-1 (own block), the other half slots 0..m-1 (previous block, absent
  // for the first entry); HCA row r is slot r.  The new token's row is taken
  // from registers.
  const int s = (p + 1) / m - 1;
  // the new entry's row in the cache (through the block table when paged),
  // looked up before the candidate loads; -1: beyond N_cap or an absent page
  const long long out_row = (wv == 0 && s < N_cap) ? kv_row_of(pg, b, N_cap, s) : -1;
  Pool pool[CPL];
  pool_init<CPL>(pool);
  float cv[CPL], zv[CPL], pv[CPL];
  auto add_row = [&](int r, const float* rc, const float* rz, const float* bias) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) zv[j] = rz[j] + bias[j];
    pool_add<CPL>(pool, rc, zv);
  };
  if (spec) {
    if (wv < T_cap) {
      const bool own = (wv / m) == half;
      if (own || s > 0) {
        const float* rc = wv == row ? tc : sc;
        const float* rz = wv == row ? tz : sz;
        add_row(wv, rc, rz, own ? sp1 : sp0);
      }
    }
  } else if (CPL > 8) {
    for (int r = wv; r < T_cap; r += kAppendWaves) {
      const bool own = !csa || (r / m) == half;
      if (!own && s == 0) continue;
      const int slot = csa ? (own ? m + r % m : r % m) : r;
      if (r == row) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          cv[j] = tc[j];
          pv[j] = tz[j];
        }
      } else {
        load_row<CPL>(tCb + r * io_row, io_fmt, c, lane, cv);
        load_row<CPL>(tZb + r * io_row, io_fmt, c, lane, pv);
      }
      float bias[CPL];
      load_bias<CPL>(P, slot, c, lane, bias);
      add_row(r, cv, pv, bias);
    }
  } else {
    // rows r = wv + kAppendWaves * i, kAppendBatch of them loaded before any is
    // pooled, so a long HCA tail pays one memory latency per batch
    constexpr int kAppendBatch = 4;
    for (int r0 = wv; r0 < T_cap; r0 += kAppendWaves * kAppendBatch) {
      float bc[kAppendBatch][CPL], bz[kAppendBatch][CPL], bb[kAppendBatch][CPL];
      bool use[kAppendBatch];
      // unconditional loads (rows past the tail read row 0 and are not used): a
      // load under a branch would be waited for at the branch's end
#pragma unroll
      for (int u = 0; u < kAppendBatch; ++u) {
        const int r = r0 + kAppendWaves * u;
        const int rl = r < T_cap ? r : 0;
        const bool own = !csa || (rl / m) == half;
        use[u] = r < T_cap && (own || s > 0);
        const int slot = csa ? (own ? m + rl % m : rl % m) : rl;
        load_row<CPL>(tCb + rl * io_row, io_fmt, c, lane, bc[u]);
        load_row<CPL>(tZb + rl * io_row, io_fmt, c, lane, bz[u]);
        load_bias<CPL>(P, slot, c, lane, bb[u]);
      }
#pragma unroll
      for (int u = 0; u < kAppendBatch; ++u) {
        const int r = r0 + kAppendWaves * u;
        if (!use[u]) continue;  // the same for the whole wave
        // the new token's row may not have reached memory yet: take it from registers
        if (r == row) add_row(r, tc, tz, bb[u]);
        else add_row(r, bc[u], bz[u], bb[u]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    part[wv][0][j][lane] = pool[j].mx;
    part[wv][1][j][lane] = pool[j].sum;
    part[wv][2][j][lane] = pool[j].acc;
  }
  __syncthreads();
  if (wv != 0) return;
  Pool tot[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < kAppendWaves; ++x) M = fmaxf(M, part[x][0][j][lane]);
    float sum = 0.f, acc = 0.f;
#pragma unroll
    for (int x = 0; x < kAppendWaves; ++x) {
      const float mx = part[x][0][j][lane];
      const float f = mx == -INFINITY ? 0.f : __expf(mx - M);
      sum += part[x][1][j][lane] * f;
      acc += part[x][2][j][lane] * f;
    }
    tot[j] = {M, sum, acc};
  }
  float out[CPL];
  pool_finish_norm<CPL>(tot, c, eps, out);
  if (rope_step != 0.0) rope_lane<CPL>(out, lane, c, rope_p);  // the entry's last token is p
  if (out_row >= 0) store_row<CPL>(cache + static_cast<size_t>(out_row) * kv_row, kv_fmt, c, lane, out);
}

}  // namespace

#define LCA_DISPATCH_CPL(c, KERNEL, GRID, ...)                                              \
  do {                                                                                      \
    const int cpl_ = (c) / kWave;                                                           \
    if (cpl_ == 2)                                                                          \
      hipLaunchKernelGGL(KERNEL<2>, GRID, dim3(kWave * kWavesPerBlock), 0, s, __VA_ARGS__); \
    else if (cpl_ == 4)                                                                     \
      hipLaunchKernelGGL(KERNEL<4>, GRID, dim3(kWave * kWavesPerBlock), 0, s, __VA_ARGS__); \
    else if (cpl_ == 8)                                                                     \
      hipLaunchKernelGGL(KERNEL<8>, GRID, dim3(kWave * kWavesPerBlock), 0, s, __VA_ARGS__); \
    else if (cpl_ == 16)                                                                    \
      hipLaunchKernelGGL(KERNEL<16>, GRID, dim3(kWave * kWavesPerBlock), 0, s, __VA_ARGS__); \
    else                                                                                    \
      return hipErrorInvalidValue;                                                          \
  } while (0)

hipError_t launch_compress(int mode, int m, int B, int n_new, int c, const void* C, const void* Z,
                           int io_fmt, const void* prevC, const void* prevZ, const float* P,
                           void* cache, int kv_fmt, int N_cap, int first_entry, float eps,
                           double rope_step, const KvPages& pg, hipStream_t s) {
  const long long n = static_cast<long long>(B) * (n_new / m);
  if (n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n + kWavesPerBlock - 1) / kWavesPerBlock));
  const int csa = mode == LCA_CSA ? 1 : 0;
  const uint8_t* Cp = static_cast<const uint8_t*>(C);
  const uint8_t* Zp = static_cast<const uint8_t*>(Z);
  const uint8_t* pC = static_cast<const uint8_t*>(prevC);
  const uint8_t* pZ = static_cast<const uint8_t*>(prevZ);
  uint8_t* ch = static_cast<uint8_t*>(cache);
  const dim3 block(kWave * kWavesPerBlock);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, csa, m, B, n_new, c, Cp, Zp, pC, pZ, P, ch, kv_fmt,
                       N_cap, first_entry, eps, rope_step, pg);
  };
  const bool f32 = io_fmt == LCA_F32;
  switch (c / kWave) {
    case 2: f32 ? go(compress_kernel<2, LCA_F32>) : go(compress_kernel<2, LCA_BF16>); break;
    case 4: f32 ? go(compress_kernel<4, LCA_F32>) : go(compress_kernel<4, LCA_BF16>); break;
    case 8: f32 ? go(compress_kernel<8, LCA_F32>) : go(compress_kernel<8, LCA_BF16>); break;
    case 16: f32 ? go(compress_kernel<16, LCA_F32>) : go(compress_kernel<16, LCA_BF16>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(int B, int n, int c, const void* x, int x_fmt, void* y, int y_fmt,
                               int y_seq_rows, float eps, long long pos0, double rope_step,
                               hipStream_t s) {
  const long long rows = static_cast<long long>(B) * n;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + kWavesPerBlock - 1) / kWavesPerBlock));
  LCA_DISPATCH_CPL(c, rmsnorm_rows_kernel, grid, B, n, c, static_cast<const uint8_t*>(x), x_fmt,
                   static_cast<uint8_t*>(y), y_fmt, y_seq_rows, eps, pos0, rope_step);
  return hipGetLastError();
}

hipError_t launch_state_append(int mode, int m, int B, int c, int n_win, const void* tokC,
                               const void* tokZ, int io_fmt, void* tailC, void* tailZ, void* ring,
                               int kv_fmt, const float* P, void* cache, int N_cap,
                               int32_t* n_tokens, int32_t* q_pos, int32_t* n_entries, float eps,
                               double rope_step, const KvPages& pg, hipStream_t s,
                               uint32_t* zero_buf, long long zero_words) {
  if (B == 0) return hipSuccess;
  const dim3 grid(B), block(kWave * kAppendWaves);
  const int csa = mode == LCA_CSA ? 1 : 0;
  const uint8_t* tc = static_cast<const uint8_t*>(tokC);
  const uint8_t* tz = static_cast<const uint8_t*>(tokZ);
  uint8_t* tC = static_cast<uint8_t*>(tailC);
  uint8_t* tZ = static_cast<uint8_t*>(tailZ);
  uint8_t* rg = static_cast<uint8_t*>(ring);
  uint8_t* ch = static_cast<uint8_t*>(cache);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, csa, m, B, c, n_win, tc, tz, tC, tZ, rg, kv_fmt, P,
                       ch, N_cap, n_tokens, q_pos, n_entries, eps, rope_step, pg, zero_buf, zero_words);
  };
  const bool f32 = io_fmt == LCA_F32;
  switch (c / kWave) {
    case 2: f32 ? go(state_append_kernel<2, LCA_F32>) : go(state_append_kernel<2, LCA_BF16>); break;
    case 4: f32 ? go(state_append_kernel<4, LCA_F32>) : go(state_append_kernel<4, LCA_BF16>); break;
    case 8: f32 ? go(state_append_kernel<8, LCA_F32>) : go(state_append_kernel<8, LCA_BF16>); break;
    case 16: f32 ? go(state_append_kernel<16, LCA_F32>) : go(state_append_kernel<16, LCA_BF16>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lca
