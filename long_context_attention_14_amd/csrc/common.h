// Shared device helpers and internal launcher declarations of the CSA/HCA
// attention library for gfx950 (CDNA4, 64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/lca.h"

namespace lca {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Device checks (a debug build: LCA_DEVICE_CHECKS = 1, build.py --device-checks).
// The kernels count the data they gather through that breaks the interface's
// rules -- a selected entry that is neither -1 nor a visible entry, a page id
// outside the pool -- and selections of the library's own that are not
// ascending visible entries followed by -1, in a counter of each source file.
// They handle such data exactly as the release build does (an absent row, a
// skipped write); the release build compiles the checks away.
#ifndef LCA_DEVICE_CHECKS
#define LCA_DEVICE_CHECKS 0
#endif
[[maybe_unused]] static __device__ unsigned int g_dbg_violations;
__device__ __forceinline__ void dbg_check(bool ok) {
  if constexpr (LCA_DEVICE_CHECKS) {
    if (!ok) atomicAdd(&g_dbg_violations, 1u);
  }
}
// Host side of one source file's counter: its value (0 without device checks)
// and, with reset, the counter set to 0.  Every source file that counts defines
// one with LCA_DBG_ACCESSOR(name).
#define LCA_DBG_ACCESSOR(name)                                                              \
  hipError_t name(unsigned long long* v, bool reset) {                                      \
    *v = 0;                                                                                 \
    if constexpr (!LCA_DEVICE_CHECKS) return hipSuccess;                                    \
    unsigned int x = 0;                                                                     \
    hipError_t e = hipMemcpyFromSymbol(&x, HIP_SYMBOL(g_dbg_violations), sizeof(x));        \
    if (e == hipSuccess && reset) {                                                         \
      const unsigned int z = 0;                                                             \
      e = hipMemcpyToSymbol(HIP_SYMBOL(g_dbg_violations), &z, sizeof(z));                   \
    }                                                                                       \
    *v = x;                                                                                 \
    return e;                                                                               \
  }
hipError_t dbg_violations_attention(unsigned long long* v, bool reset);
hipError_t dbg_violations_compress(unsigned long long* v, bool reset);
hipError_t dbg_violations_topk(unsigned long long* v, bool reset);

// ---------------------------------------------------------------------------
// stored formats

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bfloat16, round to nearest even: gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two float32 -> packed bfloat16 pair (a in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// 1/sqrt(x) with the hardware reciprocal square root (v_rsq_f32, ~1 ulp).
__device__ __forceinline__ float rsqrt_hw(float x) { return __builtin_amdgcn_rsqf(x); }

// OCP e4m3fn byte -> float32 (exact).  Exponent bias 7, exponent 0 is
// subnormal (f * 2^-9), S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t v) {
  const uint32_t s = (v & 0x80u) << 24;
  const uint32_t e = (v >> 3) & 0xfu;
  const uint32_t f = v & 0x7u;
  if (e == 0) return __uint_as_float(s | __float_as_uint(static_cast<float>(f) * 0.001953125f));
  if (e == 0xf && f == 0x7) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(s | ((e + 120u) << 23) | (f << 20));
}

// float32 -> OCP e4m3fn byte, round to nearest even, saturating at +-448.
// With E = max(exponent(|x|), -6) the quantum is 2^(E-3), and the code of
// q = rint(|x| / 2^(E-3)) is (E + 6) * 8 + q for every E (subnormals included).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t s = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a == a)) return 0x7fu;
  a = fminf(a, 448.0f);
  int E = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;
  E = E < -6 ? -6 : E;
  const float inv_q = __uint_as_float(static_cast<uint32_t>(127 - (E - 3)) << 23);  // 2^(3-E)
  const float q = rintf(a * inv_q);
  uint32_t code = static_cast<uint32_t>((E + 6) * 8 + static_cast<int>(q));
  code = code > 126u ? 126u : code;
  return s | code;
}

// ---------------------------------------------------------------------------
// Paged compressed-KV cache ("DeepSeek V4 Architecture Tricks", section
// "Heterogeneous KV Cache Layout"): entry e of sequence b is row e % epp of
// page bt[b * max_pages + e / epp] of the pool.  bt == nullptr: the contiguous
// layout, row b * N_cap + e.
struct KvPages {
  const int32_t* bt;
  int max_pages;  // row stride of bt
  int epp;        // entries per page
  int n_pages;    // pages in the pool
};

// Physical page of entry e (0 <= e < max_pages * epp), or -1 when the table
// names a page outside the pool.
__device__ __forceinline__ int kv_page(const KvPages& pg, int b, int e) {
  const int pid = pg.bt[static_cast<long long>(b) * pg.max_pages + e / pg.epp];
  return (pid >= 0 && pid < pg.n_pages) ? pid : -1;
}

// Row index (in rows from the cache base) of entry e of sequence b, or -1 when
// its page is outside the pool.
__device__ __forceinline__ long long kv_row_of(const KvPages& pg, int b, int N_cap, int e) {
  if (!pg.bt) return static_cast<long long>(b) * N_cap + e;
  const int pid = kv_page(pg, b, e);
  return pid < 0 ? -1 : static_cast<long long>(pid) * pg.epp + e % pg.epp;
}

// ---------------------------------------------------------------------------
// Partial RoPE ("DeepSeek V4 Architecture Tricks", section "Partial RoPE 和
// Attention Sink"; QbitAI article on DeepSeek-V4, hybrid attention section):
// only the last kRopeDims dims of queries, KV entries and the attention output
// carry positions.  Pair i of those dims (c - 64 + 2i, c - 64 + 2i + 1) turns by
// the angle pos * base^(-2i/64): (x, y) -> (x cos - y sin, x sin + y cos).  The
// kernels take rope_step = base^(-2/64) (pair i's frequency is rope_step^i), 0
// when RoPE is off.
constexpr int kRopeDims = 64;

// (cos, sin) of pair i's angle at position pos.  The frequency rope_step^i
// (at most 10 float64 products) and the angle are formed and reduced to
// [-pi, pi] in float64 (Cody-Waite, 2 pi in two parts): positions reach 2^21
// and beyond, where a float32 angle would be off by a tenth of a radian.  Then
// float32 sincos of the reduced angle.
__device__ inline float2 rope_cs(long long pos, int i, double rope_step) {
  double th = 1.0, sq = rope_step;
  for (int e = i; e; e >>= 1) {
    if (e & 1) th *= sq;
    sq *= sq;
  }
  const double a = static_cast<double>(pos) * th;
  const double k = rint(a * 0.15915494309189535);  // a / (2 pi)
  double r = fma(-k, 6.283185307179586, a);
  r = fma(-k, 2.4492935982947064e-16, r);
  float sn, cs;
  sincosf(static_cast<float>(r), &sn, &cs);
  return make_float2(cs, sn);
}

// Turn the pair (x, y) by the angle with cosine cs.x and sine cs.y.  The fused
// multiply-adds are written out: a sum of two products can be contracted either
// way round, and kernels that turn the same row (the state append and the
// attention that appends itself) must round it alike.
__device__ __forceinline__ void rope_turn(float& x, float& y, float2 cs) {
  const float nx = fmaf(x, cs.x, -(y * cs.y));
  const float ny = fmaf(x, cs.y, y * cs.x);
  x = nx;
  y = ny;
}

// Every lane's share of one position's angles: lane l holds pair l % 32
// (computed once per lane, in parallel; rope_lane reads it by lane shuffles).
__device__ __forceinline__ float2 rope_cs_lane(long long pos, double rope_step) {
  return rope_cs(pos, threadIdx.x & 31, rope_step);
}

// The rotary pairs among a lane's CPL consecutive channels [lane*CPL, +CPL)
// (CPL even) turned by the angles in cs_lane (rope_cs_lane of the position).
// Called by the whole wave (the shuffles need every lane).
template <int CPL>
__device__ __forceinline__ void rope_lane(float* v, int lane, int c, float2 cs_lane) {
  const int ch0 = lane * CPL;
#pragma unroll
  for (int j = 0; j < CPL; j += 2) {
    const int d = ch0 + j - (c - kRopeDims);
    const int pr = d >= 0 ? d >> 1 : 0;
    const float2 cs = make_float2(__shfl(cs_lane.x, pr, 64), __shfl(cs_lane.y, pr, 64));
    if (d >= 0) rope_turn(v[j], v[j + 1], cs);
  }
}

// ---------------------------------------------------------------------------
// row I/O: a lane owns CPL consecutive channels [lane*CPL, lane*CPL + CPL)

template <int CPL>
__device__ __forceinline__ void load_row(const void* base, int fmt, int c, int lane, float* v) {
  const int ch0 = lane * CPL;
  if (fmt == LCA_F32) {
    const float* p = static_cast<const float*>(base) + ch0;
#pragma unroll
    for (int i = 0; i < CPL; i += 2) {
      const float2 t = *reinterpret_cast<const float2*>(p + i);
      v[i] = t.x;
      v[i + 1] = t.y;
    }
  } else if (fmt == LCA_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + ch0;
#pragma unroll
    for (int i = 0; i < CPL; i += 2) {
      const uint32_t t = *reinterpret_cast<const uint32_t*>(p + i);
      v[i] = bf16_to_f32(static_cast<uint16_t>(t & 0xffffu));
      v[i + 1] = bf16_to_f32(static_cast<uint16_t>(t >> 16));
    }
  } else {  // LCA_KV_FP8_BF16ROPE
    const uint8_t* p = static_cast<const uint8_t*>(base);
    const int nope = c - 64;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int ch = ch0 + i;
      v[i] = ch < nope ? e4m3_to_f32(p[ch])
                       : bf16_to_f32(reinterpret_cast<const uint16_t*>(p + nope)[ch - nope]);
    }
  }
}

template <int CPL>
__device__ __forceinline__ void store_row(void* base, int fmt, int c, int lane, const float* v) {
  const int ch0 = lane * CPL;
  if (fmt == LCA_F32) {
    float* p = static_cast<float*>(base) + ch0;
#pragma unroll
    for (int i = 0; i < CPL; i += 2) *reinterpret_cast<float2*>(p + i) = make_float2(v[i], v[i + 1]);
  } else if (fmt == LCA_BF16) {
    uint16_t* p = static_cast<uint16_t*>(base) + ch0;
#pragma unroll
    for (int i = 0; i < CPL; i += 2) *reinterpret_cast<uint32_t*>(p + i) = pack_bf16(v[i], v[i + 1]);
  } else {  // LCA_KV_FP8_BF16ROPE
    uint8_t* p = static_cast<uint8_t*>(base);
    const int nope = c - 64;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int ch = ch0 + i;
      if (ch < nope)
        p[ch] = static_cast<uint8_t>(f32_to_e4m3(v[i]));
      else
        reinterpret_cast<uint16_t*>(p + nope)[ch - nope] = f32_to_bf16(v[i]);
    }
  }
}

__host__ __device__ inline size_t row_bytes(int fmt, int c) {
  switch (fmt) {
    case LCA_F32: return 4 * static_cast<size_t>(c);
    case LCA_BF16: return 2 * static_cast<size_t>(c);
    case LCA_FP8_E4M3: return static_cast<size_t>(c);
    case LCA_KV_FP8_BF16ROPE: return static_cast<size_t>(c) + 64;
    default: return 0;
  }
}

// DPP move of a float (row-level lane permutation, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes, returned in every lane.  Each 16-lane row is reduced
// with DPP (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror: every lane of a row ends with the same value, since each step
// adds a commuted pair), then the four row sums are read with readlane and
// added in a fixed order.  Deterministic; no LDS traffic.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0xb1>(x);
  x += dpp_f<0x4e>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

// Visible compressed entries for a query at position t: entry s needs
// (s+1)*m - 1 <= t, and s < n_entries.
// n_entries is also clamped to the cache capacity N_cap, and a negative
// position sees nothing.
__device__ __forceinline__ int visible_entries(int t, int m, int n_entries, int N_cap) {
  if (t < 0) return 0;
  int v = (t + 1) / m;
  v = v < n_entries ? v : n_entries;
  v = v < N_cap ? v : N_cap;
  return v < 0 ? 0 : v;
}

// Order-preserving uint32 key of a score: larger score <-> larger key; -0 is
// counted as +0 and NaN as -inf.  The top 12 bits are the histogram bin of the
// multi-workgroup top-k.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN -> -inf
  if (u == 0x80000000u) u = 0u;                          // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// A score as stored: fp32, or bf16 (round to nearest even of the fp32 score).
// The key of a bf16 score keeps only its top 16 bits (the key of the bf16
// value), so equal bf16 values have equal keys.
__device__ __forceinline__ void store_score(float* p, float s) { *p = s; }
__device__ __forceinline__ void store_score(uint16_t* p, float s) { *p = f32_to_bf16(s); }
__device__ __forceinline__ uint32_t stored_key(float s) { return score_key(s); }
__device__ __forceinline__ uint32_t stored_key(uint16_t h) {
  return score_key(bf16_to_f32(h)) & 0xffff0000u;
}
// key of a computed score once stored as ST
template <typename ST>
__device__ __forceinline__ uint32_t key_as_stored(float s) {
  if constexpr (sizeof(ST) == 2) return stored_key(f32_to_bf16(s));
  else return score_key(s);
}
constexpr int kScoreHistBins = 4096;
__device__ __forceinline__ uint32_t score_bin(uint32_t key) { return key >> 20; }
// Word of bin b in a row's histogram in global memory: neighbouring bins sit in
// different 128-byte lines (bin b -> line b % 32), so the few dozen bins a row's
// scores fall in do not make one hot line for the atomics of many workgroups.
__device__ __forceinline__ int hist_slot(int b) { return ((b & 31) << 7) | (b >> 5); }
__device__ __forceinline__ int hist_bin_of_slot(int w) { return ((w & 127) << 5) | (w >> 7); }
// LDS word of bin b in a row histogram copied out of global memory: one pad
// word per 64 bins.  The coalesced copy has the 64 lanes of a wave write bins
// 32 apart (two banks without the pad) and the threshold scans read bins
// 4096 / blockDim.x apart; with the pad both touch 64 distinct banks.
constexpr int kHistLdsWords = kScoreHistBins + kScoreHistBins / 64;
__device__ __forceinline__ int hist_lds(int b) { return b + (b >> 6); }

// Threshold of a row from its histogram in LDS (kScoreHistBins bins, bin
// order == key order, bin b at word hist_lds(b)): the bin holding the want-th
// largest key and the count of keys in higher bins.  All threads of the block
// call it; blockDim.x must
// divide kScoreHistBins and be a multiple of 64; scan_sh holds blockDim.x/64
// ints.  Thread t owns bins [4095 - per*t - per + 1, 4095 - per*t].
__device__ inline void find_threshold_block(const uint32_t* lh, int want, int* sh_bin,
                                            int* sh_above, int* scan_sh) {
  const int nt = blockDim.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int per = kScoreHistBins / nt;
  const int top = kScoreHistBins - 1 - per * t;
  int local = 0;
  for (int i = 0; i < per; ++i) local += static_cast<int>(lh[hist_lds(top - i)]);
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) scan_sh[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int x = 0; x < wv; ++x) before += scan_sh[x];
  int run = before + incl - local;
  if (run < want && run + local >= want) {
    for (int i = 0; i < per; ++i) {
      const int h = static_cast<int>(lh[hist_lds(top - i)]);
      if (run + h >= want) {
        *sh_bin = top - i;
        *sh_above = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
}

// Given a histogram of `nbins` bins (bin index order == key order), find the bin
// d holding the `want`-th largest element (1-based), and the number of elements
// in bins above d.  Run by one full wave (all 64 lanes); nbins % 64 == 0.
// Lane l owns bins nbins-1-l*per .. nbins-per-l*per (descending).
__device__ inline void find_bin_wave(const uint32_t* hist, int nbins, int want, int* out_bin,
                                     int* out_above) {
  const int lane = threadIdx.x & 63;
  const int per = nbins / 64;
  const int top = nbins - 1 - lane * per;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[top - i];
  // exclusive prefix over lanes (lane 0 holds the highest bins)
  uint32_t incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  uint32_t run = incl - local;
  if (run < static_cast<uint32_t>(want) && incl >= static_cast<uint32_t>(want)) {
    for (int i = 0; i < per; ++i) {
      const uint32_t h = hist[top - i];
      if (run + h >= static_cast<uint32_t>(want)) {
        *out_bin = top - i;
        *out_above = static_cast<int>(run);
        break;
      }
      run += h;
    }
  }
}

// ---------------------------------------------------------------------------
// internal launchers (defined next to their kernels, called by the C ABI)

// rope_step: base^(-2/64) of the partial RoPE, 0 for no RoPE (see rope_cs).
hipError_t launch_compress(int mode, int m, int B, int n_new, int c, const void* C, const void* Z,
                           int io_fmt, const void* prevC, const void* prevZ, const float* P,
                           void* cache, int kv_fmt, int N_cap, int first_entry, float eps,
                           double rope_step, const KvPages& pg, hipStream_t s);
hipError_t launch_rmsnorm_rows(int B, int n, int c, const void* x, int x_fmt, void* y, int y_fmt,
                               int y_seq_rows, float eps, long long pos0, double rope_step,
                               hipStream_t s);
// zero_buf (optional): zero_words uint32 words the kernel clears as a side job.
hipError_t launch_state_append(int mode, int m, int B, int c, int n_win, const void* tokC,
                               const void* tokZ, int io_fmt, void* tailC, void* tailZ, void* ring,
                               int kv_fmt, const float* P, void* cache, int N_cap,
                               int32_t* n_tokens, int32_t* q_pos, int32_t* n_entries, float eps,
                               double rope_step, const KvPages& pg, hipStream_t s,
                               uint32_t* zero_buf = nullptr, long long zero_words = 0);
// Fused indexer + selection workspace (rows = B * n_q, n_blk = ceil(N_cap / 128)).
// hist must be zero before the indexer runs (select_zero_words(rows) words).  A
// row's 128-entry blocks are dealt round-robin to its wpr workgroups;
// workgroup wi writes the (key, index) pairs of its blocks that can still be
// among the row's k largest into its own region of the row's emit array (in no
// particular order; the region starts at select_region(n_blk, wpr, wi) and
// holds 128 slots per block the workgroup owns) and their count to
// emit_cnt[row, wi]; a finish pass selects the row's top k from those pairs.
constexpr int kSelBlock = 128;
struct SelectWs {
  uint32_t* hist;      // [rows, 4096] score_bin histogram (hist_slot order)
  int32_t* emit_cnt;   // [rows, n_blk]: pairs emitted by workgroup wi of the row (wi < wpr)
  uint2* emit;         // [rows, n_blk * 128] (score key, entry index) pairs
  uint32_t* cand_key;  // [rows, N_cap] selection: threshold-bin keys when LDS overflows
  int32_t* cand_idx;   // [rows, N_cap]
  int n_blk;
  // clear_hist != 0: the finish pass zero-fills each row's histogram once it has
  // read it, so the next launch on the same hist needs no clearing first
  int clear_hist;
  // decode steps (n_q = 1) only, or NULL: the indexer takes each row's position
  // from n_tokens (p = n_tokens[b]; n_entries = min((p+1)/m, N_cap)) instead of
  // from q_pos / n_entries, and its workgroup 0 of the row writes both there for
  // the launches after it (a negative count: q_pos / n_entries are read and left
  // as they are)
  const int32_t* n_tokens;
  int32_t* q_pos_out;
  int32_t* n_entries_out;
};
// first slot of workgroup wi's region in a row's emit array: workgroups before
// wi own n_blk / wpr blocks each, one more when they come before n_blk % wpr
__host__ __device__ __forceinline__ size_t select_region(int n_blk, int wpr, int wi) {
  const int a = n_blk / wpr, r = n_blk % wpr;
  return static_cast<size_t>(wi * a + (wi < r ? wi : r)) * kSelBlock;
}
size_t select_workspace_bytes(long long rows, int N_cap);
long long select_zero_words(long long rows);
SelectWs select_ws_in(void* ws, long long rows, int N_cap);
// whether the fused path takes rows of N_cap entries and this k
bool select_supported(int N_cap, int k);
// workgroups per row (wpr) the finish pass takes
constexpr int kSelMaxWpr = 256;
// A CSA decode step's state append run by the selection finish launch: one
// more workgroup per sequence beside the finish's, on CUs the finish leaves
// idle (the indexer before it took the query positions from n_tokens itself,
// or from launch_decode_prep, which also cleared a workspace histogram).  Same
// rows, entries and counts as launch_state_append; bf16 io, c = 512, tail of
// 2m rows.
struct StateAppend {
  int m, B, n_win, kv_fmt, N_cap;
  const uint8_t* tokC;  // [B, 512] bf16
  const uint8_t* tokZ;
  uint8_t* tailC;       // [B, 2m, 512] bf16
  uint8_t* tailZ;
  uint8_t* ring;        // [B, n_win, row]
  const float* P;       // [2m, 512]
  uint8_t* cache;       // [B, N_cap, row] or a page pool
  int32_t* n_tokens;    // [B], advanced by one
  float eps;
  double rope_step;
  KvPages pg;
};
// The finish pass after the fused indexer: one workgroup per row selects the
// row's top k from the emitted pairs into idx ([rows, k], ascending, -1 after
// min(k, vis)); rows with vis <= k were written by the indexer.  app: the step's
// state append, run beside it (n_q = 1), or NULL.
hipError_t launch_select_finish(long long rows, int n_q, int N_cap, int wpr, const int32_t* q_pos, int m,
                                const int32_t* n_entries, int k, const SelectWs& w, int32_t* idx,
                                hipStream_t s, const StateAppend* app = nullptr);
// What the indexer of such a step needs first: q_pos[b] = p = n_tokens[b],
// n_entries[b] = min((p+1)/m, N_cap) (a negative count is left alone), and
// zero_buf cleared.
hipError_t launch_decode_prep(int m, int B, int N_cap, const int32_t* n_tokens, int32_t* q_pos,
                              int32_t* n_entries, uint32_t* zero_buf, long long zero_words,
                              hipStream_t s);

// hist (optional, [B*n_q, 4096], zeroed by the caller): the MFMA path adds the
// score_bin histogram of every row's visible scores into it.  sel (optional,
// MFMA formats only): the fused selecting sink; scores is then not written and
// the indexer writes every row's top k to sel_idx ([B*n_q, k], ascending entry
// indices, ties to the lower index, -1 after min(k, vis)).
hipError_t launch_indexer(int B, int n_q, int H_I, int d_I, int idx_fmt, const void* qI,
                          const uint8_t* qI_scale, const void* kI, const uint8_t* kI_scale,
                          int N_cap, const float* w, const int32_t* q_pos, int m,
                          const int32_t* n_entries, void* scores, hipStream_t s,
                          uint32_t* hist = nullptr, hipEvent_t ev_start = nullptr,
                          hipEvent_t ev_stop = nullptr, const SelectWs* sel = nullptr, int k = 0,
                          int score_fmt = LCA_F32, int32_t* sel_idx = nullptr,
                          const StateAppend* app = nullptr);
size_t topk_workspace_bytes(int B, int n_q, int N_cap, int k);
// scores: [B*n_q, N_cap] float32, or bf16 bits when score_fmt == LCA_BF16
hipError_t launch_topk(int B, int n_q, int N_cap, const void* scores, const int32_t* q_pos, int m,
                       const int32_t* n_entries, int k, int32_t* idx, void* ws, hipStream_t s,
                       int score_fmt = LCA_F32);
// For rows longer than the LDS path takes: the row histogram inside the top-k
// workspace (nullptr when the LDS path applies; its zero region is
// topk_hist_words(rows) words), and the selection from a histogram that the
// indexer already accumulated there.
long long topk_hist_words(long long rows);
uint32_t* topk_hist_in_workspace(void* ws, int B, int n_q, int N_cap, int k);
hipError_t launch_topk_from_hist(int B, int n_q, int N_cap, const float* scores,
                                 const int32_t* q_pos, int m, const int32_t* n_entries, int k,
                                 int32_t* idx, void* ws, hipStream_t s);
// fixed_split: candidate rows per split (a multiple of 64), or 0 for the plan
// that follows the number of query rows.
size_t mqa_workspace_bytes(int B, int n_q, int H, int c, int kv_fmt, int k, int N_cap, int n_win,
                           int dense, int fixed_split);
// splits per query of a fixed plan (0 for the automatic one)
int mqa_splits(int k, int N_cap, int n_win, int dense, int fixed_split);
constexpr int kMaxSplits = 256;
size_t out_proj_workspace_bytes(int T, int n_h, int c, int g, int d_g, int d);
hipError_t launch_out_proj(int T, int n_h, int c, int g, int d_g, int d, const uint16_t* o,
                           const uint16_t* W_g, const uint16_t* W_o, uint16_t* z, void* out,
                           int out_fmt, void* ws, hipStream_t s);
// Reads bytes (a multiple of 16) of device memory once; sink receives at most
// one word.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
// An HCA decode step's state append done inside the attention launch (the
// decode kernel's workgroups that hold the new token's window row or the entry
// the token completes make them, write them to the state and use them from
// LDS; the split merge, or the single workgroup, then advances n_tokens).  The
// same rows, entries and counts as launch_state_append followed by the
// attention, in one launch fewer.  m is the HCA rate; the tail has m rows;
// io is bf16; the window is the ring (W_cap = n_win, origin 0).
struct DecodeAppend {
  const uint8_t* tokC;  // [B, c] bf16: the new token's KV candidate
  const uint8_t* tokZ;  // [B, c] bf16: its gate logits
  uint8_t* tailC;       // [B, m, c] bf16
  uint8_t* tailZ;
  const float* P;       // [m, c] positional bias of the gate logits
  uint8_t* ring;        // the window ring (the attention's window) and the cache (or
  uint8_t* cache;       // page pool) it reads, for the rows the append writes
  int32_t* n_tokens;    // [B]: read, then advanced by one
  int32_t* q_pos;       // [B] written (the query position p = n_tokens)
  int32_t* n_entries;   // [B] written
};
// Whether launch_mqa can take a DecodeAppend for this shape (the few-row decode
// kernel runs the attention).
bool mqa_can_append(long long rows, int H, int c, int q_fmt, int kv_fmt, int N_cap, int n_win,
                    int fixed_split);
hipError_t launch_mqa(int B, int n_q, int H, int c, const void* q, int q_fmt, const void* cache,
                      int kv_fmt, int N_cap, const int32_t* idx, int k, const int32_t* q_pos, int m,
                      const int32_t* n_entries, const void* win, int W_cap, int64_t win_origin,
                      int n_win, float tau, float eps, const float* sink, double rope_step, void* out,
                      int out_fmt, float* lse, void* ws, const KvPages& pg, hipStream_t s,
                      int fixed_split = 0, const DecodeAppend* append = nullptr);

}  // namespace lca
