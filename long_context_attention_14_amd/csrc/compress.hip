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
// Mapping: one workgroup of kPoolWaves waves per entry; lane l owns channels
// [l*CPL, (l+1)*CPL) with CPL = c/64, so every candidate row is one coalesced
// c-wide load per wave.  Candidate slot j (time order) is pooled by wave
// j % kPoolWaves with an online per-channel softmax in registers; the waves'
// partial states are combined in slot order, then RMS-normalised (a wavefront
// reduction).  The decode-time state append pools a completed block with the
// same slot-to-wave split and combination order, so an entry made by decode
// steps has the same bits as the entry the prefill compressor makes.
#include <algorithm>

#include "common.h"
#include "pool.h"

namespace lca {
namespace {

constexpr int kWavesPerBlock = 4;

// IOF: the candidates' format (F32 or BF16) as a compile-time constant, so that
// row loads carry no format branches (a load under a branch makes the compiler
// wait for it at the branch's end, which serialises the candidate loads).
// One workgroup per entry (grid = B * n_new / m); wave wv pools slots wv,
// wv + kPoolWaves, ... in increasing order, loading kBatch slots' rows before
// pooling any of them.
template <int CPL, int IOF>
__global__ __launch_bounds__(kWave * kPoolWaves) void compress_kernel(
    int csa, int m, int B, int n_new, int c, const uint8_t* C, const uint8_t* Z,
    const uint8_t* prevC, const uint8_t* prevZ, const float* P, uint8_t* cache, int kv_fmt,
    int N_cap, int first_entry, float eps, double rope_step, KvPages pg) {
  constexpr int io_fmt = IOF;
  constexpr int kBatch = CPL > 8 ? 1 : 4;
  __shared__ float part[kPoolWaves][3][CPL][kWave];  // lane-contiguous: no bank conflicts
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int n_ent = n_new / m;
  const int b = static_cast<int>(blockIdx.x / n_ent);
  const int s = static_cast<int>(blockIdx.x % n_ent);
  // the entry's row in the cache (through the block table when paged), looked
  // up before the candidate loads
  const long long out_row = wv == 0 ? kv_row_of(pg, b, N_cap, first_entry + s) : -1;
  if (LCA_DEVICE_CHECKS && wv == 0 && lane == 0) dbg_check(out_row >= 0);
  const size_t io_row = row_bytes(io_fmt, c);
  const uint8_t* Cb = C + static_cast<size_t>(b) * n_new * io_row;
  const uint8_t* Zb = Z + static_cast<size_t>(b) * n_new * io_row;
  const int W = csa ? 2 * m : m;
  // CSA slots 0..m-1: the previous block (chunk rows of block s-1, prevC/prevZ
  // for the chunk's first entry, absent without them); slots m..2m-1 and every
  // HCA slot: the entry's own block
  const bool have_prev = s > 0 || prevC != nullptr;
  Pool pool[CPL];
  pool_init<CPL>(pool);
  for (int j0 = wv; j0 < W; j0 += kPoolWaves * kBatch) {
    float bc[kBatch][CPL], bz[kBatch][CPL], bb[kBatch][CPL];
    bool use[kBatch];
    // unconditional loads (a slot past W reads slot j0's rows and is not used)
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + kPoolWaves * u;
      const int jl = j < W ? j : j0;
      const bool prev = csa && jl < m;
      const uint8_t* rc;
      const uint8_t* rz;
      if (prev && s == 0 && prevC != nullptr) {
        rc = prevC + (static_cast<size_t>(b) * m + jl) * io_row;
        rz = prevZ + (static_cast<size_t>(b) * m + jl) * io_row;
      } else {
        // previous block: row (s-1)*m + jl (row s*m when absent: loaded, unused)
        const size_t r = prev ? (s > 0 ? static_cast<size_t>(s - 1) * m + jl : static_cast<size_t>(s) * m)
                              : static_cast<size_t>(s) * m + (csa ? jl - m : jl);
        rc = Cb + r * io_row;
        rz = Zb + r * io_row;
      }
      use[u] = j < W && (!prev || have_prev);
      load_row<CPL>(rc, io_fmt, c, lane, bc[u]);
      load_row<CPL>(rz, io_fmt, c, lane, bz[u]);
      load_bias<CPL>(P, jl, c, lane, bb[u]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (!use[u]) continue;  // the same for the whole wave
      float zv[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) zv[i] = bz[u][i] + bb[u][i];
      pool_add<CPL>(pool, bc[u], zv);
    }
  }
  int order[kPoolWaves];
#pragma unroll
  for (int x = 0; x < kPoolWaves; ++x) order[x] = x;
  float out[CPL];
  if (!pool_combine_norm<CPL>(part, pool, order, wv, lane, c, eps, out)) return;
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

// One workgroup of kAppendWaves waves per sequence (state_append_body).
template <int CPL, int IOF>
__global__ __launch_bounds__(kWave * kAppendWaves) void state_append_kernel(
    int csa, int m, int B, int c, int n_win, const uint8_t* tokC, const uint8_t* tokZ,
    uint8_t* tailC, uint8_t* tailZ, uint8_t* ring, int kv_fmt, const float* P, uint8_t* cache,
    int N_cap, int32_t* n_tokens, int32_t* q_pos, int32_t* n_entries, float eps, double rope_step,
    KvPages pg, uint32_t* zero_buf, long long zero_words) {
  __shared__ float part[kAppendWaves][3][CPL][kWave];  // lane-contiguous: no bank conflicts
  state_append_body<CPL, IOF>(blockIdx.x, gridDim.x, part, csa, m, c, n_win, tokC, tokZ, tailC, tailZ,
                              ring, kv_fmt, P, cache, N_cap, n_tokens, q_pos, n_entries, eps, rope_step,
                              pg, zero_buf, zero_words);
}

// The part of a decode step's state append that the indexer needs first, for a
// step whose attention appends the token itself: the query position p =
// n_tokens[b] and the visible entry count, and the cleared zero_buf (the
// selection's row histogram).  n_tokens is advanced after the attention.
__global__ __launch_bounds__(256) void decode_prep_kernel(int m, int B, int N_cap,
                                                          const int32_t* n_tokens, int32_t* q_pos,
                                                          int32_t* n_entries, uint32_t* zero_buf,
                                                          long long zero_words) {
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < zero_words;
       i += static_cast<long long>(gridDim.x) * blockDim.x)
    zero_buf[i] = 0u;
  const int b = static_cast<int>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b < B) {
    const int p = n_tokens[b];
    if (p >= 0) {  // a negative count: the sequence is left as it is
      q_pos[b] = p;
      const int ne = (p + 1) / m;
      n_entries[b] = ne < N_cap ? ne : N_cap;
    }
  }
}

}  // namespace

hipError_t launch_decode_prep(int m, int B, int N_cap, const int32_t* n_tokens, int32_t* q_pos,
                              int32_t* n_entries, uint32_t* zero_buf, long long zero_words,
                              hipStream_t s) {
  if (B == 0) return hipSuccess;
  const long long want = std::max<long long>((B + 255) / 256, (zero_words + 1023) / 1024);
  const unsigned grid = static_cast<unsigned>(std::min<long long>(std::max<long long>(want, 1), 1024));
  hipLaunchKernelGGL(decode_prep_kernel, dim3(grid), dim3(256), 0, s, m, B, N_cap, n_tokens, q_pos,
                     n_entries, zero_buf, zero_words);
  return hipGetLastError();
}

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
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(n));  // one workgroup per entry
  const int csa = mode == LCA_CSA ? 1 : 0;
  const uint8_t* Cp = static_cast<const uint8_t*>(C);
  const uint8_t* Zp = static_cast<const uint8_t*>(Z);
  const uint8_t* pC = static_cast<const uint8_t*>(prevC);
  const uint8_t* pZ = static_cast<const uint8_t*>(prevZ);
  uint8_t* ch = static_cast<uint8_t*>(cache);
  const dim3 block(kWave * kPoolWaves);
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

LCA_DBG_ACCESSOR(dbg_violations_compress)

}  // namespace lca
