// Grouped output projection (QbitAI article on DeepSeek-V4, hybrid attention
// section, the fourth step of CSA): with head dim c = 512, projecting all n_h
// heads straight back to the hidden size d is expensive, so the heads are split
// into g groups, each group's concatenated outputs are projected to d_g, and the
// g results together are projected back to d:
//   z[t, j*d_g + r] = sum_i W_g[j, r, i] * o[t, j*(n_h/g)*c + i]      (bf16 z)
//   out[t, n]       = sum_q W_o[n, q] * z[t, q]
// Both products run on one bf16 MFMA GEMM kernel (fp32 accumulation):
// C[m, n] = sum_k A[m, k] * W[n, k] per batch, W stored output x input (row n
// holds the K inputs of output n).
//
// Mapping, many tokens (M > 32, MFMA-bound): a 256-thread workgroup computes a
// 128 x 128 tile of C in steps of 64 along K; A and W tiles are staged through
// registers into double-buffered LDS (rows padded to 144 B) and the four waves
// run 32x32x16 bf16 MFMAs on them; when the tiles are too few, K is split over
// workgroups (fp32 partials summed in split order by a second kernel, so results
// stay deterministic).
// Few tokens (M <= 32, a decode batch; HBM-bound: the V4-Pro shape streams
// 176 MiB of weights for 16 tokens): a workgroup owns 32 output columns, its
// waves take interleaved 64-wide K steps, the weight rows reach LDS in long
// contiguous segments a few chunks ahead, each workgroup starts at its own
// point of K (see gemm_skinny_kernel), and the waves' partial tiles are summed
// in wave order through LDS at the end.
#include "common.h"

namespace lca {
namespace {

typedef float gv16f __attribute__((ext_vector_type(16)));
typedef __bf16 gv8bf __attribute__((ext_vector_type(8)));

constexpr int kGBK = 64;             // K per step
constexpr int kGBN = 128;            // output columns per workgroup
constexpr int kGLds = kGBK + 8;      // LDS row stride in bf16 (144 B)
constexpr int kGThreads = 256;
constexpr int kGTargetWGs = 512;     // split K until about this many workgroups

struct GemmArgs {
  const uint16_t* A;  // A[m][k] at A + batch * a_bstride + m * lda + k
  long long lda, a_bstride;
  const uint16_t* W;  // W[n][k] at W + batch * w_bstride + n * K + k
  long long w_bstride;
  void* C;            // C[m][n] at C + batch * c_bstride + m * ldc + n (c_fmt)
  long long ldc, c_bstride;
  int c_fmt;
  float* part;        // split partials [split][batch][M][N] (n_split > 1)
  int M, N, K, batches, n_split, steps_per_split;
};

__device__ __forceinline__ gv8bf as8(uint4 u) { return __builtin_bit_cast(gv8bf, u); }
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ gv8bf as8v(u32x4 u) { return __builtin_bit_cast(gv8bf, u); }

template <int BM>
__global__ __launch_bounds__(kGThreads, 2) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WN = BM == 128 ? 2 : 4;        // waves along N
  constexpr int WM = 4 / WN;                   // waves along M
  constexpr int TM = BM / WM / 32;             // 32-row MFMA tiles per wave
  constexpr int TN = kGBN / WN / 32;           // 32-column MFMA tiles per wave
  constexpr int ACH = BM * kGBK / 8 / kGThreads;   // 16-byte A chunks per thread
  constexpr int WCH = kGBN * kGBK / 8 / kGThreads; // 16-byte W chunks per thread
  static_assert(ACH >= 1 && WCH >= 1, "tile too small for the workgroup");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kGLds];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][kGBN * kGLds];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j32 = lane & 31, g = lane >> 5;
  const int wm = w / WN, wn = w % WN;
  // Tile order (workgroup L runs on XCD L % 8, each XCD with its own L2): the
  // (row tile, split, batch) triples are dealt to the XCDs in eight contiguous
  // ranges, and an XCD takes each triple's column tiles one after another, so
  // an A tile is read from memory by one XCD and reused from its L2 (a batch's
  // W stays on the XCDs that own its rows).
  const int n_tiles = a.N / kGBN, m_tiles = (a.M + BM - 1) / BM;
  const long long n_trip = static_cast<long long>(m_tiles) * a.n_split * a.batches;
  const long long L = blockIdx.x;
  long long nt, trip;
  if (n_trip % 8 == 0) {
    const long long i = L / 8;
    nt = i % n_tiles;
    trip = (L % 8) * (n_trip / 8) + i / n_tiles;
  } else {
    nt = L % n_tiles;
    trip = L / n_tiles;
  }
  const int n0 = static_cast<int>(nt) * kGBN;
  const int m0 = static_cast<int>(trip % m_tiles) * BM;
  const int split = static_cast<int>((trip / m_tiles) % a.n_split);
  const int batch = static_cast<int>(trip / m_tiles / a.n_split);
  const uint16_t* Ab = a.A + batch * a.a_bstride;
  const uint16_t* Wb = a.W + batch * a.w_bstride + static_cast<long long>(n0) * a.K;
  const int k_begin = split * a.steps_per_split * kGBK;
  const int steps = a.steps_per_split;

  // a step's A and W chunks in registers; two named sets, so that a step's
  // loads go out two steps before they are stored to LDS
  struct Stage {
    uint4 a[ACH], w[WCH];
  };
  auto load = [&](Stage& R, int st) {  // steps past the end read the last one (not stored)
    const int k0 = k_begin + min(st, steps - 1) * kGBK;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int ch = tid + kGThreads * i, r = ch >> 3, kc = ch & 7;
      const int m = min(m0 + r, a.M - 1);  // rows past M read row M-1, staged as zeros
      R.a[i] = *reinterpret_cast<const uint4*>(Ab + m * a.lda + k0 + 8 * kc);
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int ch = tid + kGThreads * i, r = ch >> 3, kc = ch & 7;
      R.w[i] = *reinterpret_cast<const uint4*>(Wb + static_cast<long long>(r) * a.K + k0 + 8 * kc);
    }
  };
  auto store = [&](const Stage& R, int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int ch = tid + kGThreads * i, r = ch >> 3, kc = ch & 7;
      *reinterpret_cast<uint4*>(&As[buf][r * kGLds + 8 * kc]) =
          m0 + r < a.M ? R.a[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int ch = tid + kGThreads * i, r = ch >> 3, kc = ch & 7;
      *reinterpret_cast<uint4*>(&Ws[buf][r * kGLds + 8 * kc]) = R.w[i];
    }
  };

  gv16f acc[TM][TN];
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y) acc[x][y] = gv16f{0};

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kGBK / 16; ++ks) {
      uint4 av[TM], wv[TN];
#pragma unroll
      for (int x = 0; x < TM; ++x)
        av[x] = *reinterpret_cast<const uint4*>(
            &As[buf][(wm * TM * 32 + 32 * x + j32) * kGLds + 16 * ks + 8 * g]);
#pragma unroll
      for (int y = 0; y < TN; ++y)
        wv[y] = *reinterpret_cast<const uint4*>(
            &Ws[buf][(wn * TN * 32 + 32 * y + j32) * kGLds + 16 * ks + 8 * g]);
#pragma unroll
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as8(av[x]), as8(wv[y]), acc[x][y], 0, 0, 0);
    }
  };
  // step st is computed from LDS buffer st % 2; register set P carries even
  // steps and Q odd ones, each loaded two steps before it is stored
  Stage P, Q;
  load(P, 0);
  load(Q, 1);
  store(P, 0);
  __syncthreads();
  for (int st = 0; st < steps; st += 2) {
    load(P, st + 2);          // P was stored last step
    compute(0);
    if (st + 1 < steps) store(Q, 1);  // buffer 1 was last read two steps ago
    __syncthreads();
    if (st + 1 >= steps) break;
    load(Q, st + 3);
    compute(1);
    if (st + 2 < steps) store(P, 0);
    __syncthreads();
  }

  // accumulator register r of lane (j32, g): row 8 (r/4) + 4 g + r%4, column j32
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * TM * 32 + 32 * x + 8 * (r >> 2) + 4 * g + (r & 3);
        const int n = n0 + wn * TN * 32 + 32 * y + j32;
        if (m >= a.M) continue;
        const float v = acc[x][y][r];
        if (a.n_split > 1) {
          a.part[((static_cast<long long>(split) * a.batches + batch) * a.M + m) * a.N + n] = v;
        } else {
          const long long ci = batch * a.c_bstride + static_cast<long long>(m) * a.ldc + n;
          if (a.c_fmt == LCA_F32) static_cast<float*>(a.C)[ci] = v;
          else static_cast<uint16_t*>(a.C)[ci] = f32_to_bf16(v);
        }
      }
}

// C = the split partials summed in split order (deterministic), four columns a
// thread.
__global__ __launch_bounds__(256) void gemm_split_sum_kernel(GemmArgs a) {
  const long long n4 = a.N / 4;
  const long long gid = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= static_cast<long long>(a.batches) * a.M * n4) return;
  const int n = static_cast<int>(gid % n4) * 4;
  const long long bm = gid / n4;
  const int m = static_cast<int>(bm % a.M);
  const int batch = static_cast<int>(bm / a.M);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < a.n_split; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(
        &a.part[((static_cast<long long>(sp) * a.batches + batch) * a.M + m) * a.N + n]);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  const long long ci = batch * a.c_bstride + static_cast<long long>(m) * a.ldc + n;
  if (a.c_fmt == LCA_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.C) + ci) = s;
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.C) + ci) =
        make_uint2(pack_bf16(s.x, s.y), pack_bf16(s.z, s.w));
  }
}

// Few tokens: see the file comment.  NW waves per workgroup, 32 columns.  K
// goes in chunks of NW 64-wide steps, step c NW + w of chunk c belonging to
// wave w.  A chunk's 32 weight rows are loaded as whole row segments (8 NW
// consecutive 16-byte pieces per row: with four waves one load instruction of
// a wave covers 512 bytes of each of two rows), three chunks ahead in named
// register sets, stored to double-buffered LDS (rows padded by 16 bytes) and
// read from there as MFMA operands; the tokens' operands come straight from
// memory (they stay in L2).
template <int NW>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int CK = kGBK * NW;               // K of a chunk
  constexpr int kRowPieces = CK / 8;          // 16-byte pieces of a row in a chunk
  constexpr int PPT = 32 * kRowPieces / NT;   // pieces a thread loads per chunk
  constexpr int kSRow = CK + 8;               // LDS row stride (bf16)
  static_assert(PPT * NT == 32 * kRowPieces, "whole pieces per thread");
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][32 * kSRow];
  __shared__ float red[NW][32][33];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j32 = lane & 31, g = lane >> 5;
  const int n0 = blockIdx.x * 32;
  const int batch = blockIdx.y;
  const uint16_t* Wb = a.W + batch * a.w_bstride + static_cast<long long>(n0) * a.K;
  // lane (j32, g): A operand = A row j32 (rows past M read row M-1: they only
  // reach output rows past M, which are not stored), B operand = W row
  // n0 + j32; 8 K values at 16 ks + 8 g of a step
  const uint16_t* Ar = a.A + batch * a.a_bstride + static_cast<long long>(min(j32, a.M - 1)) * a.lda + 8 * g;
  const int steps = a.K / kGBK;
  const int nch = (steps + NW - 1) / NW;
  static_assert(PPT == 4, "four pieces a thread per chunk");
  // (plain vector types: copies of HIP's uint4 struct between address spaces
  // become memcpy calls that keep the sets in scratch memory)
  struct WSet {
    u32x4 v0, v1, v2, v3;
  };
  struct ASet {
    u32x4 x0, x1, x2, x3;
  };
  // Workgroup L takes the chunks in the order L, L + 1, ... (mod nch): the
  // rows of a weight matrix are a power-of-two number of bytes apart, and with
  // every workgroup at the same K offset the reads crowd onto a fraction of the
  // HBM channels (same work in the same order: 47 against 40 us for the
  // 16-token projection).  phys(c) is the chunk taken c-th; nch for the
  // clamped loads past the last one.
  const int rot = static_cast<int>((blockIdx.x + static_cast<long long>(blockIdx.y) * gridDim.x) % nch);
  auto phys = [&](int c) { return c < nch ? (c + rot) % nch : nch; };
  // piece p = tid + NT i of the c-th chunk: row p / kRowPieces, columns
  // phys(c) CK + 8 (p % kRowPieces) .. + 7 (past the last chunk: column K - 8,
  // never multiplied)
  auto wptr = [&](int c, int i) {
    const int p = tid + NT * i;
    const int col = min(phys(c) * CK + 8 * (p % kRowPieces), a.K - 8);
    return reinterpret_cast<const u32x4*>(Wb + static_cast<long long>(p / kRowPieces) * a.K + col);
  };
  auto load_w = [&](WSet& s, int c) {
    s.v0 = *wptr(c, 0);
    s.v1 = *wptr(c, 1);
    s.v2 = *wptr(c, 2);
    s.v3 = *wptr(c, 3);
  };
  auto wlds = [&](int buf, int i) {
    const int p = tid + NT * i;
    return reinterpret_cast<u32x4*>(&wt[buf][(p / kRowPieces) * kSRow + 8 * (p % kRowPieces)]);
  };
  auto store_w = [&](const WSet& s, int buf) {
    *wlds(buf, 0) = s.v0;
    *wlds(buf, 1) = s.v1;
    *wlds(buf, 2) = s.v2;
    *wlds(buf, 3) = s.v3;
  };
  auto load_a = [&](ASet& s, int c) {  // the wave's step of chunk c (clamped)
    const u32x4* ap = reinterpret_cast<const u32x4*>(Ar + min(phys(c) * NW + w, steps - 1) * kGBK);
    s.x0 = ap[0];
    s.x1 = ap[2];
    s.x2 = ap[4];
    s.x3 = ap[6];
  };
  gv16f acc = gv16f{0};
  auto mma = [&](const ASet& s, int c) {
    if (phys(c) * NW + w >= steps) return;  // (the same for the whole wave)
    const u32x4* wr = reinterpret_cast<const u32x4*>(&wt[c & 1][j32 * kSRow + kGBK * w + 8 * g]);
    const u32x4 b0 = wr[0], b1 = wr[2], b2 = wr[4], b3 = wr[6];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as8v(s.x0), as8v(b0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as8v(s.x1), as8v(b1), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as8v(s.x2), as8v(b2), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as8v(s.x3), as8v(b3), acc, 0, 0, 0);
  };
  // The j-th chunk taken lives in the sets (wj, aj), j mod 3: the weights of
  // chunk j + 1 are stored to LDS after chunk j's products, into the buffer
  // that chunk j - 1 used (every wave was done with it before the barrier that
  // ended step j - 1), and that set is refilled with chunk j + 4.  Loads and
  // stores past the last chunk are clamped and unused: with no branch around
  // them, each wait covers exactly its own set.
  WSet w0, w1, w2;
  ASet a0, a1, a2;
  load_a(a0, 0);
  load_w(w0, 0);
  load_a(a1, 1);
  load_w(w1, 1);
  load_a(a2, 2);
  load_w(w2, 2);
  store_w(w0, 0);
  load_w(w0, 3);
  __syncthreads();
  for (int c = 0; c < nch; c += 3) {
#define LCA_SKINNY_STEP(AC, WN, C) \
  mma(AC, C);                      \
  load_a(AC, (C) + 3);             \
  store_w(WN, ((C) + 1) & 1);      \
  load_w(WN, (C) + 4);             \
  __syncthreads();
    LCA_SKINNY_STEP(a0, w1, c)
    LCA_SKINNY_STEP(a1, w2, c + 1)
    LCA_SKINNY_STEP(a2, w0, c + 2)
#undef LCA_SKINNY_STEP
  }
  // register r of lane (j32, g): output row 8 (r/4) + 4 g + r%4, column n0 + j32
#pragma unroll
  for (int r = 0; r < 16; ++r) red[w][8 * (r >> 2) + 4 * g + (r & 3)][j32] = acc[r];
  __syncthreads();
  for (int i = tid; i < a.M * 32; i += NT) {
    const int m = i >> 5, nn = i & 31;
    float v = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) v += red[x][m][nn];
    const long long ci = batch * a.c_bstride + static_cast<long long>(m) * a.ldc + n0 + nn;
    if (a.c_fmt == LCA_F32) static_cast<float*>(a.C)[ci] = v;
    else static_cast<uint16_t*>(a.C)[ci] = f32_to_bf16(v);
  }
}

constexpr int kSkinnyM = 32;  // at most this many rows take the skinny kernel

int gemm_bm(int) { return 128; }

// K splits: double while the grid is below the target and every split keeps at
// least 4 steps.
int gemm_splits(int M, int N, int K, int batches) {
  const long long tiles = static_cast<long long>((M + gemm_bm(M) - 1) / gemm_bm(M)) * (N / kGBN) * batches;
  const int steps = K / kGBK;
  int sp = 1;
  while (tiles * sp < kGTargetWGs && steps % (2 * sp) == 0 && steps / (2 * sp) >= 4) sp *= 2;
  return sp;
}

size_t gemm_ws_bytes(int M, int N, int K, int batches) {
  if (M <= kSkinnyM) return 0;
  const int sp = gemm_splits(M, N, K, batches);
  return sp > 1 ? static_cast<size_t>(sp) * batches * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(GemmArgs a, void* ws, hipStream_t s) {
  if (a.M <= kSkinnyM) {
    // four waves per workgroup (the 16-token batch: 37.0 us against 51.3 with
    // two and 44.7 with eight waves where the column tiles are fewer than the
    // CUs; the output stage's 224 workgroups take 19.4 us with four)
    const dim3 grid(static_cast<unsigned>(a.N / 32), static_cast<unsigned>(a.batches));
    hipLaunchKernelGGL(gemm_skinny_kernel<4>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  a.n_split = gemm_splits(a.M, a.N, a.K, a.batches);
  a.steps_per_split = a.K / kGBK / a.n_split;
  a.part = a.n_split > 1 ? static_cast<float*>(ws) : nullptr;
  const int bm = gemm_bm(a.M);
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(a.N / kGBN) * ((a.M + bm - 1) / bm) *
                                        a.batches * a.n_split));
  hipLaunchKernelGGL(gemm_bf16_kernel<128>, grid, dim3(kGThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const long long n = static_cast<long long>(a.batches) * a.M * (a.N / 4);
  hipLaunchKernelGGL(gemm_split_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

size_t out_proj_workspace_bytes(int T, int n_h, int c, int g, int d_g, int d) {
  const size_t a = gemm_ws_bytes(T, d_g, n_h / g * c, g);
  const size_t b = gemm_ws_bytes(T, d, g * d_g, 1);
  return a > b ? a : b;
}

hipError_t launch_out_proj(int T, int n_h, int c, int g, int d_g, int d, const uint16_t* o,
                           const uint16_t* W_g, const uint16_t* W_o, uint16_t* z, void* out,
                           int out_fmt, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int kin = n_h / g * c;
  GemmArgs a1{};
  a1.A = o;
  a1.lda = static_cast<long long>(n_h) * c;
  a1.a_bstride = kin;
  a1.W = W_g;
  a1.w_bstride = static_cast<long long>(d_g) * kin;
  a1.C = z;
  a1.ldc = static_cast<long long>(g) * d_g;
  a1.c_bstride = d_g;
  a1.c_fmt = LCA_BF16;
  a1.M = T;
  a1.N = d_g;
  a1.K = kin;
  a1.batches = g;
  hipError_t e = launch_gemm(a1, ws, s);
  if (e != hipSuccess) return e;
  GemmArgs a2{};
  a2.A = z;
  a2.lda = static_cast<long long>(g) * d_g;
  a2.a_bstride = 0;
  a2.W = W_o;
  a2.w_bstride = 0;
  a2.C = out;
  a2.ldc = d;
  a2.c_bstride = 0;
  a2.c_fmt = out_fmt;
  a2.M = T;
  a2.N = d;
  a2.K = g * d_g;
  a2.batches = 1;
  return launch_gemm(a2, ws, s);
}

}  // namespace lca
