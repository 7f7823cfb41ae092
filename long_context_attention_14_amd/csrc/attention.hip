// Core attention of CSA/HCA plus the sliding-window branch, as one softmax
// merged by log-sum-exp (QbitAI article on DeepSeek-V4, hybrid attention
// section: multi-query attention over the selected compressed entries, each
// entry being both key and value; RMSNorm of queries and KV before attention;
// a sliding-window branch over the most recent tokens' uncompressed KV; an
// attention-sink logit that only enlarges the softmax denominator.  "DeepSeek
// V4 Architecture Tricks", section "Sliding Window Branch": n_win = 128).
//
// Work decomposition (flash-decoding): for a query row, the list of candidate
// rows is [compressed slots (top-k indices, or all visible entries for HCA);
// n_win window slots].  The list is cut into splits of kSplitRows slots when
// there are few query rows (decode), so that enough workgroups fill the 256
// CUs; each (query row, head group, split) workgroup streams its rows through
// LDS in tiles, keeps an online softmax per head, and writes a normalised
// partial (o, lse).  A merge kernel combines the splits of a row in a fixed
// order (deterministic).  With a single split (prefill: many query rows) the
// workgroup writes the final output directly.
#include <type_traits>

#include "common.h"
#include "pool.h"

namespace lca {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kHG = 8;          // heads per workgroup
constexpr int kRT = 16;         // rows per LDS tile
constexpr int kSplitRows = 64;  // slots per split in decode

struct SlotCtx {
  const int32_t* idx;  // [k] for this row, or nullptr (dense)
  KvPages pg;          // paged cache (pg.bt != nullptr: cache_b is the pool base)
  int b;               // the row's sequence
  int NS;              // compressed slots
  int vis;             // visible entries
  int N_cap;
  int t;               // query position
  int n_win;
  const uint8_t* cache_b;
  const uint8_t* win_b;
  int W_cap;
  long long win_origin;
  size_t kv_row;
};

// Row pointer of slot i of the candidate list, or nullptr if the slot is empty
// (or its page is outside the pool).
__device__ __forceinline__ const uint8_t* slot_row(const SlotCtx& s, int i) {
  if (i < s.NS) {
    int e = s.idx ? s.idx[i] : i;
    const int lim = s.vis < s.N_cap ? s.vis : s.N_cap;
    if (e < 0 || e >= lim) return nullptr;
    if (s.pg.bt) {
      const int pid = kv_page(s.pg, s.b, e);
      if (pid < 0) return nullptr;
      return s.cache_b + (static_cast<size_t>(pid) * s.pg.epp + e % s.pg.epp) * s.kv_row;
    }
    return s.cache_b + static_cast<size_t>(e) * s.kv_row;
  }
  const int w = i - s.NS;
  const long long j = static_cast<long long>(s.t) - s.n_win + 1 + w;
  if (j < 0) return nullptr;
  long long slot = (j - s.win_origin) % s.W_cap;
  if (slot < 0) slot += s.W_cap;
  return s.win_b + static_cast<size_t>(slot) * s.kv_row;
}

// Device checks of compressed slot i < NS whose index entry is e (and, paged,
// page pid of e): e is -1 or a visible entry, and a visible entry's page is in
// the pool (one call per slot and workgroup).
__device__ __forceinline__ void dbg_slot(const SlotCtx& s, int e, int pid) {
  const int lim = s.vis < s.N_cap ? s.vis : s.N_cap;
  const bool vis_e = e >= 0 && e < lim;
  if (s.idx) dbg_check(e == -1 || vis_e);
  if (s.pg.bt && vis_e) dbg_check(pid >= 0);
}
__device__ __forceinline__ void dbg_slot_i(const SlotCtx& s, int i) {
  if constexpr (LCA_DEVICE_CHECKS) {
    if (i < s.NS) {
      const int e = s.idx ? s.idx[i] : i;
      const int lim = s.vis < s.N_cap ? s.vis : s.N_cap;
      dbg_slot(s, e, (s.pg.bt && e >= 0 && e < lim) ? kv_page(s.pg, s.b, e) : 0);
    }
  }
}

template <int CPL>
__global__ __launch_bounds__(kAttnThreads) void attn_generic_kernel(
    int n_q, int H, int c, const uint8_t* __restrict__ q, int q_fmt, const uint8_t* __restrict__ cache,
    int kv_fmt, int N_cap, const int32_t* __restrict__ idx, int k, const int32_t* __restrict__ q_pos,
    int m, const int32_t* __restrict__ n_entries, const uint8_t* __restrict__ win, int W_cap,
    long long win_origin, int n_win, float tau, float eps, const float* __restrict__ sink,
    double rope_step, int n_splits, int split_rows, uint8_t* __restrict__ out, int out_fmt,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse, KvPages pg) {
  constexpr int C = CPL * 64;
  constexpr int CP = C + 1;                    // padded LDS row stride (floats)
  constexpr int OPT = kHG * C / kAttnThreads;  // outputs per thread
  constexpr int TPH = kAttnThreads / kHG;      // threads per head
  __shared__ float qs[kHG * CP];
  __shared__ float rows_s[kRT * CP];
  __shared__ float logit_s[kHG * kRT];
  __shared__ int valid_s[kRT];

  const int n_hg = H / kHG;
  long long bid = blockIdx.x;
  const int split = static_cast<int>(bid % n_splits);
  bid /= n_splits;
  const int hg = static_cast<int>(bid % n_hg);
  const long long row = bid / n_hg;
  const int b = static_cast<int>(row / n_q);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  SlotCtx sc;
  sc.t = q_pos[row];
  sc.vis = visible_entries(sc.t, m, n_entries[b], N_cap);
  sc.idx = idx ? idx + row * k : nullptr;
  sc.NS = idx ? k : N_cap;
  sc.N_cap = N_cap;
  sc.n_win = n_win;
  sc.kv_row = row_bytes(kv_fmt, c);
  sc.pg = pg;
  sc.b = b;
  sc.cache_b = pg.bt ? cache : cache + static_cast<size_t>(b) * N_cap * sc.kv_row;
  sc.win_b = win + static_cast<size_t>(b) * W_cap * sc.kv_row;
  sc.W_cap = W_cap;
  sc.win_origin = win_origin;
  const int NT = sc.NS + n_win;
  const int s_begin = split * split_rows;
  const int s_end = min(s_begin + split_rows, NT);

  // the query position's angles: lane l holds pair l % 32; rope_s keeps a copy
  // for the epilogue
  __shared__ float2 rope_s[kRopeDims / 2];
  float2 cs_q = make_float2(1.f, 0.f);
  if (rope_step != 0.0) {
    cs_q = rope_cs_lane(sc.t, rope_step);
    if (tid < kRopeDims / 2) rope_s[tid] = cs_q;
  }
  // normalised queries of this head group (wave wv handles heads wv, wv+4)
  const size_t q_row = row_bytes(q_fmt, c);
  for (int hh = wv; hh < kHG; hh += kAttnThreads / 64) {
    float v[CPL];
    load_row<CPL>(q + (static_cast<size_t>(row) * H + hg * kHG + hh) * q_row, q_fmt, c, lane, v);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) ss += v[i] * v[i];
    ss = wave_sum(ss);
    const float r = rsqrt_hw(ss / static_cast<float>(c) + eps);
#pragma unroll
    for (int i = 0; i < CPL; ++i) v[i] *= r;
    if (rope_step != 0.0) rope_lane<CPL>(v, lane, c, cs_q);  // the query turned to its position
#pragma unroll
    for (int i = 0; i < CPL; ++i) qs[hh * CP + lane * CPL + i] = v[i];
  }

  const int my_h = tid / TPH;
  const int my_d0 = tid % TPH;
  float o[OPT];
#pragma unroll
  for (int i = 0; i < OPT; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int base = s_begin; base < s_end; base += kRT) {
    __syncthreads();
    // stage kRT rows (each wave 4 rows) as fp32
    for (int r = wv; r < kRT; r += kAttnThreads / 64) {
      const int slot = base + r;
      const uint8_t* rp = slot < s_end ? slot_row(sc, slot) : nullptr;
      if (LCA_DEVICE_CHECKS && lane == 0 && slot < s_end) dbg_slot_i(sc, slot);
      float v[CPL];
      if (rp) {
        load_row<CPL>(rp, kv_fmt, c, lane, v);
      } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) v[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) rows_s[r * CP + lane * CPL + i] = v[i];
      if (lane == 0) valid_s[r] = rp != nullptr;
    }
    __syncthreads();
    if (tid < kHG * kRT) {
      const int h = tid / kRT, r = tid % kRT;
      float d = 0.f;
      const float* qp = qs + h * CP;
      const float* rp = rows_s + r * CP;
      for (int i = 0; i < C; ++i) d = fmaf(qp[i], rp[i], d);
      logit_s[h * kRT + r] = valid_s[r] ? d * tau : -INFINITY;
    }
    __syncthreads();
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < kRT; ++r) tmax = fmaxf(tmax, logit_s[my_h * kRT + r]);
    const float m_new = fmaxf(m_run, tmax);
    if (m_new == -INFINITY) continue;
    const float scale = __expf(m_run - m_new);
    l_run *= scale;
#pragma unroll
    for (int i = 0; i < OPT; ++i) o[i] *= scale;
#pragma unroll 4
    for (int r = 0; r < kRT; ++r) {
      const float lg = logit_s[my_h * kRT + r];
      const float p = lg == -INFINITY ? 0.f : __expf(lg - m_new);
      l_run += p;
      const float* rp = rows_s + r * CP + my_d0;
#pragma unroll
      for (int i = 0; i < OPT; ++i) o[i] = fmaf(p, rp[i * TPH], o[i]);
    }
    m_run = m_new;
  }

  const int h = hg * kHG + my_h;
  float lse_v = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  if (n_splits == 1) {
    float f = 1.f;
    if (sink && lse_v != -INFINITY) {
      const float sk = sink[h];
      const float mx = fmaxf(lse_v, sk);
      const float tot = mx + __logf(__expf(lse_v - mx) + __expf(sk - mx));
      f = __expf(lse_v - tot);
      lse_v = tot;
    } else if (sink) {
      lse_v = sink[h];
    }
    const size_t orow = (static_cast<size_t>(row) * H + h) * row_bytes(out_fmt, c);
    if (rope_step != 0.0) __syncthreads();  // rope_s written
    for (int i = 0; i < OPT; ++i) {
      const int d = my_d0 + i * TPH;
      float v = o[i] * inv * f;
      if (rope_step != 0.0) {
        // the output turned back by -t; the pair's other dim is in lane tid ^ 1
        const float other = __shfl_xor(v, 1, 64);
        const int pd = d - (c - kRopeDims);
        if (pd >= 0) {
          const float2 cs = rope_s[pd >> 1];  // angle t; turned by -t below
          v = (d & 1) ? v * cs.x - other * cs.y : v * cs.x + other * cs.y;
        }
      }
      if (out_fmt == LCA_F32)
        reinterpret_cast<float*>(out + orow)[d] = v;
      else
        reinterpret_cast<uint16_t*>(out + orow)[d] = f32_to_bf16(v);
    }
    if (lse && my_d0 == 0) lse[static_cast<size_t>(row) * H + h] = lse_v;
  } else {
    const size_t prow = (static_cast<size_t>(row) * n_splits + split) * H + h;
    for (int i = 0; i < OPT; ++i) part_o[prow * c + my_d0 + i * TPH] = o[i] * inv;
    if (my_d0 == 0) part_lse[prow] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// MFMA path: c = 512, H = 64, bf16 (or fp8 + bf16 RoPE dims) KV.
//
// A workgroup (4 waves) owns one query row and one split of its candidate list
// and all 64 heads, so each gathered KV row is read from HBM once and serves
// every head as both key and value.  Per 64-row tile: the rows are staged in
// LDS as bf16; S = Qn K^T runs on the 32x32x16 bf16 MFMA (wave w: heads
// [32*(w/2), +32) x rows [32*(w%2), +32), K = 512); the online softmax updates
// per-head max / sum in LDS and writes P as bf16; O += P V runs on the same
// MFMA (wave w: all heads x dims [128w, 128w+128), K = 64 rows), with the V
// operand read from the same LDS tile.  The softmax denominator sums the
// bf16-rounded P that the PV product uses.

typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

constexpr int kMT = 64;            // rows per tile
constexpr int kMC = 512;           // head dim
constexpr int kMH = 64;            // heads
constexpr int kQS = kMC + 8;       // LDS row stride of Q and KV tiles (bf16 elements)
constexpr int kPS = kMT + 8;       // LDS row stride of P (bf16 elements)
constexpr int kSS = kMT + 1;       // LDS row stride of S (floats)

__device__ __forceinline__ v8bf_t as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf_t, u); }

// Two OCP e4m3 bytes (the low or the high 16 bits of w) -> packed bf16 pair, with
// gfx950's scaled conversion at scale 1 (every e4m3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// gfx950's transposing LDS read: within each 16-lane group, output lane i gets
// element i%4 of the 8-byte chunks addressed by group lanes i/4 + 4j, j = 0..3.
// With group lane s pointing at row r0 + s/4, dims d0 + 4 (s%4) of a row-major
// tile, output lane i receives rows r0 .. r0+3 of dim d0 + i (checked by the
// attention parity tests).
typedef short v4s_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 tr_rows4(const uint16_t* p) {
  const v4s_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Loads through a global-address-space pointer.  Row pointers that went through
// LDS or lane reads are generic to the compiler, which would emit flat loads;
// those also count against the LDS wait counter, so every LDS wait would
// wait for the KV rows in flight as well.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ldg16(const void* p) {
  const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4_t*>(
      reinterpret_cast<uintptr_t>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ldg8(const void* p) {
  const u32x2_t v = *reinterpret_cast<const __attribute__((address_space(1))) u32x2_t*>(
      reinterpret_cast<uintptr_t>(p));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ v16f_t mfma_bf16(const v8bf_t& a, const v8bf_t& b, const v16f_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int KVFMT>
__global__ __launch_bounds__(256) void attn_mfma_kernel(
    int n_q, const uint8_t* __restrict__ q, int q_fmt, const uint8_t* __restrict__ cache,
    int N_cap, const int32_t* __restrict__ idx, int k, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, const uint8_t* __restrict__ win, int W_cap,
    long long win_origin, int n_win, float tau, float eps, const float* __restrict__ sink,
    double rope_step, int n_splits, int split_rows, uint8_t* __restrict__ out, int out_fmt,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse, KvPages pg) {
  __shared__ __attribute__((aligned(16))) uint16_t q_s[kMH * kQS];
  __shared__ float2 rope_s[kRopeDims / 2];  // (cos, sin) of the query position's angles
  __shared__ __attribute__((aligned(16))) uint16_t kv_s[kMT * kQS];
  __shared__ float s_s[kMH * kSS];
  __shared__ __attribute__((aligned(16))) uint16_t p_s[kMH * kPS];
  __shared__ float m_s[kMH], l_s[kMH], a_s[kMH];
  __shared__ const uint8_t* rowp_s[2][kMT];

  const int split = blockIdx.x % n_splits;
  const long long row = blockIdx.x / n_splits;
  const int b = static_cast<int>(row / n_q);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int j32 = lane & 31, g = lane >> 5;

  SlotCtx sc;
  sc.t = q_pos[row];
  sc.vis = visible_entries(sc.t, m, n_entries[b], N_cap);
  sc.idx = idx ? idx + row * k : nullptr;
  sc.NS = idx ? k : N_cap;
  sc.N_cap = N_cap;
  sc.n_win = n_win;
  sc.kv_row = row_bytes(KVFMT, kMC);
  sc.pg = pg;
  sc.b = b;
  sc.cache_b = pg.bt ? cache : cache + static_cast<size_t>(b) * N_cap * sc.kv_row;
  sc.win_b = win + static_cast<size_t>(b) * W_cap * sc.kv_row;
  sc.W_cap = W_cap;
  sc.win_origin = win_origin;
  const int NT = sc.NS + n_win;
  const int s_begin = split * split_rows;
  const int s_end = min(s_begin + split_rows, NT);

  // row pointers of the first tile; its row loads are issued before the query
  // phase so that both latencies overlap
  if (tid < kMT) rowp_s[0][tid] = s_begin + tid < s_end ? slot_row(sc, s_begin + tid) : nullptr;
  if (LCA_DEVICE_CHECKS && tid < kMT && s_begin + tid < s_end) dbg_slot_i(sc, s_begin + tid);
  if (rope_step != 0.0 && tid >= kMT && tid < kMT + kRopeDims / 2)
    rope_s[tid - kMT] = rope_cs(sc.t, tid - kMT, rope_step);
  __syncthreads();
  // the rotary pairs of a lane's 8 dims [8 lane, +8) turned to the query position
  auto rope8 = [&](float* v) {
    if (rope_step != 0.0 && lane >= (kMC - kRopeDims) / 8) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        rope_turn(v[2 * e], v[2 * e + 1], rope_s[4 * (lane - (kMC - kRopeDims) / 8) + e]);
    }
  };
  uint4 raw[kMT / 4];
  auto load_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kMT / 4; ++i) {
      const uint8_t* rp = rowp_s[buf][wv + 4 * i];
      raw[i] = make_uint4(0, 0, 0, 0);
      if (rp) {
        if (KVFMT == LCA_BF16) {
          raw[i] = ldg16(rp + lane * 16);
        } else if (lane < 56) {
          const uint2 f = ldg8(rp + lane * 8);
          raw[i].x = f.x;
          raw[i].y = f.y;
        } else {
          raw[i] = ldg16(rp + 448 + (lane - 56) * 16);
        }
      }
    }
  };
  load_tile(0);
  // normalised queries -> bf16 in LDS (wave wv: heads wv, wv+4, ...); all of a
  // wave's loads are issued before the first reduction
  const size_t q_row = row_bytes(q_fmt, kMC);
  if (q_fmt == LCA_BF16) {
    uint4 raw[kMH / 4];
#pragma unroll
    for (int i = 0; i < kMH / 4; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(row) * kMH + wv + 4 * i) * q_row +
                                               lane * 16);
#pragma unroll
    for (int i = 0; i < kMH / 4; ++i) {
      const uint32_t w4[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16_to_f32(static_cast<uint16_t>(w4[e] & 0xffffu));
        v[2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(w4[e] >> 16));
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
      ss = wave_sum(ss);
      const float r = rsqrt_hw(ss / static_cast<float>(kMC) + eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= r;
      rope8(v);
      uint4 pk;
      pk.x = pack_bf16(v[0], v[1]);
      pk.y = pack_bf16(v[2], v[3]);
      pk.z = pack_bf16(v[4], v[5]);
      pk.w = pack_bf16(v[6], v[7]);
      *reinterpret_cast<uint4*>(&q_s[(wv + 4 * i) * kQS + lane * 8]) = pk;
    }
  } else {
    for (int h = wv; h < kMH; h += 4) {
      float v[8];
      load_row<8>(q + (static_cast<size_t>(row) * kMH + h) * q_row, q_fmt, kMC, lane, v);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
      ss = wave_sum(ss);
      const float r = rsqrt_hw(ss / static_cast<float>(kMC) + eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= r;
      rope8(v);
      uint4 pk;
      pk.x = pack_bf16(v[0], v[1]);
      pk.y = pack_bf16(v[2], v[3]);
      pk.z = pack_bf16(v[4], v[5]);
      pk.w = pack_bf16(v[6], v[7]);
      *reinterpret_cast<uint4*>(&q_s[h * kQS + lane * 8]) = pk;
    }
  }
  if (tid < kMH) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }

  v16f_t o[2][4];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[ht][dt] = v16f_t{0};

  const int sh = wv >> 1, sr = wv & 1;  // this wave's S tile
  // transposing-read source of this lane: row (lane%16)/4, dims 16 (lane/16 % 2)
  // + 4 (lane%4) within a 4-row x 32-dim block (see tr_rows4)
  const int tr_r = (lane & 15) >> 2;
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  __syncthreads();
  int cur = 0;
  for (int base = s_begin; base < s_end; base += kMT, cur ^= 1) {
    // stage this tile's rows as bf16 and resolve the next tile's row pointers
#pragma unroll
    for (int i = 0; i < kMT / 4; ++i) {
      uint4 v = raw[i];
      if (KVFMT != LCA_BF16 && lane < 56) {  // 8 OCP e4m3 dims -> bf16 (exact)
        v.x = fp8x2_to_bf16x2<false>(raw[i].x);
        v.y = fp8x2_to_bf16x2<true>(raw[i].x);
        v.z = fp8x2_to_bf16x2<false>(raw[i].y);
        v.w = fp8x2_to_bf16x2<true>(raw[i].y);
      }
      *reinterpret_cast<uint4*>(&kv_s[(wv + 4 * i) * kQS + lane * 8]) = v;
    }
    const int nbase = base + kMT;
    if (tid < kMT) rowp_s[cur ^ 1][tid] = nbase + tid < s_end ? slot_row(sc, nbase + tid) : nullptr;
    if (LCA_DEVICE_CHECKS && tid < kMT && nbase + tid < s_end) dbg_slot_i(sc, nbase + tid);
    __syncthreads();
    if (nbase < s_end) load_tile(cur ^ 1);  // in flight during this tile's compute
    // S tile of this wave (two accumulator chains)
    {
      v16f_t acc0 = v16f_t{0}, acc1 = v16f_t{0};
      const uint16_t* qa = &q_s[(32 * sh + j32) * kQS + 8 * g];
      const uint16_t* kb = &kv_s[(32 * sr + j32) * kQS + 8 * g];
#pragma unroll 8
      for (int ks = 0; ks < kMC / 16; ks += 2) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(qa + 16 * ks);
        const uint4 b0 = *reinterpret_cast<const uint4*>(kb + 16 * ks);
        const uint4 a1 = *reinterpret_cast<const uint4*>(qa + 16 * ks + 16);
        const uint4 b1 = *reinterpret_cast<const uint4*>(kb + 16 * ks + 16);
        acc0 = mfma_bf16(as_v8bf(a0), as_v8bf(b0), acc0);
        acc1 = mfma_bf16(as_v8bf(a1), as_v8bf(b1), acc1);
      }
      const bool valid = rowp_s[cur][32 * sr + j32] != nullptr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = 32 * sh + 8 * (r >> 2) + 4 * g + (r & 3);
        s_s[h * kSS + 32 * sr + j32] = valid ? (acc0[r] + acc1[r]) * tau : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax: thread -> (head tid/4, rows 16*(tid%4) .. +16)
    {
      const int h = tid >> 2, q4 = tid & 3;
      const float* srow = &s_s[h * kSS + 16 * q4];
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, srow[r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 64));
      const float m_old = m_s[h];
      const float m_new = fmaxf(m_old, tmax);
      float psum = 0.f;
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0 = 0.f, p1 = 0.f;
        if (m_new != -INFINITY) {
          p0 = srow[r] == -INFINITY ? 0.f : __expf(srow[r] - m_new);
          p1 = srow[r + 1] == -INFINITY ? 0.f : __expf(srow[r + 1] - m_new);
        }
        pk[r / 2] = pack_bf16(p0, p1);
        psum += bf16_to_f32(static_cast<uint16_t>(pk[r / 2] & 0xffffu)) +
                bf16_to_f32(static_cast<uint16_t>(pk[r / 2] >> 16));
      }
      uint4* pd = reinterpret_cast<uint4*>(&p_s[h * kPS + 16 * q4]);
      pd[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      pd[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      psum += __shfl_xor(psum, 1, 64);
      psum += __shfl_xor(psum, 2, 64);
      if (q4 == 0) {
        const float alpha = (m_new == -INFINITY || m_old == -INFINITY) ? (m_old == -INFINITY ? 0.f : 1.f)
                                                                       : __expf(m_old - m_new);
        l_s[h] = l_s[h] * alpha + psum;
        a_s[h] = alpha;
        m_s[h] = m_new;
      }
    }
    __syncthreads();
    // O = O * alpha + P V   (wave wv: dims [128 wv, +128))
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float al = a_s[32 * ht + 8 * (r >> 2) + 4 * g + (r & 3)];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[ht][dt][r] *= al;
      }
    }
#pragma unroll
    for (int ks = 0; ks < kMT / 16; ++ks) {
      v8bf_t A[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        A[ht] = as_v8bf(*reinterpret_cast<const uint4*>(&p_s[(32 * ht + j32) * kPS + 16 * ks + 8 * g]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        // B = V rows 16 ks + 8 g .. +8 of dim 128 wv + 32 dt + j32, read transposed
        // from the row-major tile: two 4-row transposing reads (see tr_rows4)
        const uint16_t* vp = &kv_s[(16 * ks + 8 * g + tr_r) * kQS + 128 * wv + 32 * dt + tr_d];
        const uint2 lo = tr_rows4(vp);
        const uint2 hi = tr_rows4(vp + 4 * kQS);
        const v8bf_t Bv = as_v8bf(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) o[ht][dt] = mfma_bf16(A[ht], Bv, o[ht][dt]);
      }
    }
    __syncthreads();  // kv_s, p_s and rowp_s[cur] are rewritten by the next tile
  }

  // epilogue: O / l (with the sink when this is the only split); lse = m + log l.
  // Per-head factors go to LDS, then O is written through LDS (32 heads at a
  // time, fp32, reusing the KV tile buffer) so that the global stores are
  // contiguous 16-byte chunks.
  float* fac_s = s_s;  // [kMH] output factors (S is no longer needed)
  if (tid < kMH) {
    const int h = tid;
    const float l = l_s[h];
    float lse_v = l > 0.f ? m_s[h] + __logf(l) : -INFINITY;
    float f = l > 0.f ? 1.0f / l : 0.f;
    if (n_splits == 1 && sink) {
      const float sk = sink[h];
      if (lse_v == -INFINITY) {
        lse_v = sk;
      } else {
        const float mx = fmaxf(lse_v, sk);
        const float tot = mx + __logf(__expf(lse_v - mx) + __expf(sk - mx));
        f *= __expf(lse_v - tot);
        lse_v = tot;
      }
    }
    fac_s[h] = f;
    if (n_splits == 1) {
      if (lse) lse[static_cast<size_t>(row) * kMH + h] = lse_v;
    } else {
      part_lse[(static_cast<size_t>(row) * n_splits + split) * kMH + h] = lse_v;
    }
  }
  __syncthreads();
  float* ost = reinterpret_cast<float*>(kv_s);  // [32 heads][kMC] fp32 = 64 KiB
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hl = 8 * (r >> 2) + 4 * g + (r & 3);
      const float f = fac_s[32 * ht + hl];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) ost[hl * kMC + 128 * wv + 32 * dt + j32] = o[ht][dt][r] * f;
    }
    __syncthreads();
    // 32 heads x 512 fp32 = 4096 chunks of 16 B; thread tid writes chunks tid + 256 i
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int chunk = tid + 256 * i;
      const int hl = chunk >> 7, d4 = (chunk & 127) * 4;
      float4 v = *reinterpret_cast<const float4*>(&ost[hl * kMC + d4]);
      const int h = 32 * ht + hl;
      if (n_splits == 1) {
        if (rope_step != 0.0 && d4 >= kMC - kRopeDims) {  // the output turned back by -t
          const int pr = (d4 - (kMC - kRopeDims)) >> 1;
          const float2 c0 = rope_s[pr], c1 = rope_s[pr + 1];
          rope_turn(v.x, v.y, make_float2(c0.x, -c0.y));
          rope_turn(v.z, v.w, make_float2(c1.x, -c1.y));
        }
        const size_t oi = (static_cast<size_t>(row) * kMH + h) * kMC + d4;
        if (out_fmt == LCA_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + oi) = v;
        } else {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + oi) =
              make_uint2(pack_bf16(v.x, v.y), pack_bf16(v.z, v.w));
        }
      } else {
        *reinterpret_cast<float4*>(
            &part_o[((static_cast<size_t>(row) * n_splits + split) * kMH + h) * kMC + d4]) = v;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Decode kernel (few query rows, bf16 queries, 64 heads x 512): one workgroup
// of eight waves (two per SIMD) per (query row, split) with all 64 heads; wave
// w covers heads 32 hg .. +32 (hg = w & 1) and dims 128 kq .. +128 (kq = w >> 1).
//
//  * The normalised query (the wave's heads and dims) stays in registers as the
//    B operand of S^T = K Q^T (32x32x16 bf16 MFMA; lane: head 32 hg + l%32,
//    dims 128 kq + 16 ks + 8 (l/32) .. +8 of k-step ks), so the scores read only
//    K from LDS.  Each wave computes the partial S^T of all 64 tile rows over
//    its 128 dims; the four waves of a head half add their partials (in quarter
//    order) through LDS, each keeping the rows 16 kq .. +16, agree on every
//    head's tile maximum through LDS, and write P (bf16) of their rows to LDS.
//  * PV: the wave accumulates O for its 32 heads and its 128 dims (V read
//    transposed from the row-major tile).
//  * The running maximum is raised only when a tile's maximum exceeds it by
//    more than kLazyMax (natural-log units), so P stays below e^kLazyMax and O
//    is rescaled only on those tiles (the normalised result is the same).
//  * KV tiles are double-buffered in LDS.  Wave w loads the tile rows w + 8 i,
//    i < 8, through row pointers held by lanes 0..7; the next tile's rows are in
//    flight in registers during a tile's compute, and the row indices of the
//    tile after it are loaded one tile ahead.  Empty rows (outside the split,
//    past the visible entries, before the window start) load the query row,
//    are staged as zeros and masked to -inf in S.  The partial S^T of a tile
//    goes through the other KV buffer, which is free at that point.
//  * With two waves per SIMD one wave's barrier and LDS waits overlap the other
//    wave's MFMA and VALU work (four waves of twice the work each took 9% longer).
constexpr float kLazyMax = 8.0f;

// Row of slot i when its index entry e (and, paged, the page pid of e) has
// been loaded already (both unused for window slots); nullptr when the slot is
// empty.
template <bool PAGED>
__device__ __forceinline__ const uint8_t* slot_row_e(const SlotCtx& s, int i, int e, int pid) {
  if (i < s.NS) {
    const int lim = s.vis < s.N_cap ? s.vis : s.N_cap;
    if (e < 0 || e >= lim) return nullptr;
    if (PAGED) {
      if (pid < 0) return nullptr;
      return s.cache_b + (static_cast<size_t>(pid) * s.pg.epp + e % s.pg.epp) * s.kv_row;
    }
    return s.cache_b + static_cast<size_t>(e) * s.kv_row;
  }
  const int w = i - s.NS;
  const long long j = static_cast<long long>(s.t) - s.n_win + 1 + w;
  if (j < 0) return nullptr;
  long long slot = (j - s.win_origin) % s.W_cap;
  if (slot < 0) slot += s.W_cap;
  return s.win_b + static_cast<size_t>(slot) * s.kv_row;
}

constexpr int kD8Waves = 8;  // waves per decode workgroup

// The decode kernel's KV tile rows are 1 KiB apart with no padding; the
// 16-byte chunks of row r are permuted by chunk ^ dswz(r) (a function of r mod
// 16).  Both reads of a tile then spread over all 64 LDS banks: the Sᵀ reads
// (16 lanes, 16 consecutive rows, one chunk each) and the transposing V reads
// (32 lanes: 4 rows x 8 pieces of 8 bytes, two chunks per row), which with the
// padded rows met 2-way bank conflicts (a third of the kernel's LDS cycles).
constexpr int kDQS = kMC;  // LDS row stride of the decode kernel's KV tiles (bf16 elements)
__device__ __forceinline__ int dswz(int r) { return (4 * (r & 3)) ^ ((r >> 2) & 3); }
// element index of chunk-aligned column col (a multiple of 4) of row r
__device__ __forceinline__ int dkv(int r, int col) {
  return r * kDQS + ((((col >> 3) ^ dswz(r)) << 3) | (col & 7));
}

// APPEND (HCA decode steps, dense rows, n_q = 1): the step's state append runs
// here (DecodeAppend).  Every workgroup takes the query position p from
// n_tokens.  The one that holds the window slot of position p RMS-normalises
// the new token into the ring and writes its tail rows and the step's q_pos and
// n_entries; the one that holds entry (p+1)/m - 1, when the token completes a
// block, pools the block into the cache (the append's slot split and
// combination order, so the same bits).  Both keep the row they made in LDS
// and put it in place of the row loaded for that slot (which they cannot wait
// to read back).  The pooling's scratch is the second KV buffer, free before
// the first tile.
template <int KVFMT, bool PAGED, bool APPEND>
__global__ __launch_bounds__(64 * kD8Waves) void attn_decode_kernel(
    int n_q, const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int N_cap,
    const int32_t* __restrict__ idx, int k, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, const uint8_t* __restrict__ win, int W_cap,
    long long win_origin, int n_win, float tau, float eps, const float* __restrict__ sink,
    double rope_step, int n_splits, int split_rows, uint8_t* __restrict__ out, int out_fmt,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse, KvPages pg,
    DecodeAppend ap) {
  constexpr int NW = kD8Waves;
  __shared__ __attribute__((aligned(16))) uint16_t kv_s[2][kMT * kDQS];
  // APPEND: the stored bytes of the new window row [0] and of the new entry [1]
  __shared__ __attribute__((aligned(16))) uint4 app_s[APPEND ? 2 : 1][APPEND ? kMC * 2 / 16 : 1];
  __shared__ float2 rope_s[kRopeDims / 2];  // (cos, sin) of the query position's angles
  __shared__ __attribute__((aligned(16))) uint16_t p_s[kMH * kPS];
  __shared__ float ps_s[4][kMH];  // per dim quarter: query sums of squares; then P row sums
  __shared__ float mx_s[4][kMH];  // per row quarter: the tile maximum of each head
  __shared__ __attribute__((aligned(16))) uint32_t vm_s[2][NW];
  __shared__ int raise_s[2];  // tile t & 1: some head's row-quarter maximum passed the lazy bound

  const int split = blockIdx.x % n_splits;
  const long long row = blockIdx.x / n_splits;
  const int b = static_cast<int>(row / n_q);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = w & 1, kq = w >> 1;
  const int j32 = lane & 31, g = lane >> 5;
  const int head = 32 * hg + j32;  // the head of this lane's softmax state

  SlotCtx sc;
  sc.idx = idx ? idx + row * k : nullptr;
  sc.NS = idx ? k : N_cap;
  sc.N_cap = N_cap;
  sc.n_win = n_win;
  sc.kv_row = row_bytes(KVFMT, kMC);
  sc.pg = pg;
  sc.b = b;
  sc.cache_b = pg.bt ? cache : cache + static_cast<size_t>(b) * N_cap * sc.kv_row;
  sc.win_b = win + static_cast<size_t>(b) * W_cap * sc.kv_row;
  sc.W_cap = W_cap;
  sc.win_origin = win_origin;
  const int NT = sc.NS + n_win;
  const int s_begin = split * split_rows;
  const int s_end = min(s_begin + split_rows, NT);
  const int n_tiles = (s_end - s_begin + kMT - 1) / kMT;

  // lanes 0..7 (and their copies in the other lanes) hold tile row w + 8 (lane % 8)
  const int my_r = w + NW * (lane & 7);
  auto entry = [&](int tile) -> int {  // index entry of my_r in a tile (clamped load)
    const int i = s_begin + kMT * tile + my_r;
    if (sc.idx) return sc.idx[min(i, sc.NS - 1)];
    return i;
  };
  auto page_of = [&](int e) -> int {
    return kv_page(sc.pg, b, min(max(e, 0), sc.N_cap - 1));
  };
  // empty rows read the query row instead (64 KiB, always there and already in
  // the cache), so that no load depends on the cache or the window holding a row
  const uint8_t* q_bytes = reinterpret_cast<const uint8_t*>(q + static_cast<size_t>(row) * kMH * kMC);
  auto row_ptr = [&](int tile, int e, int pid, uint32_t& mask8) -> const uint8_t* {
    const int i = s_begin + kMT * tile + my_r;
    const uint8_t* p = i < s_end ? slot_row_e<PAGED>(sc, i, e, pid) : nullptr;
    if (LCA_DEVICE_CHECKS && lane < 8 && i < s_end && i < sc.NS) dbg_slot(sc, e, pid);
    mask8 = static_cast<uint32_t>(__ballot(p != nullptr)) & 0xffu;
    return p ? p : q_bytes;
  };
  const int lane_off = KVFMT == LCA_BF16 ? lane * 16 : (lane < 56 ? lane * 8 : 448 + (lane - 56) * 16);
  uint4 raw[8];
  auto load_rows = [&](const uint8_t* p) {
    const uint64_t pv = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = static_cast<uint32_t>(pv), hi = static_cast<uint32_t>(pv >> 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t pi =
          (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(hi, i))) << 32) |
          static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, i));
      raw[i] = ldg16(reinterpret_cast<const uint8_t*>(pi) + lane_off);
    }
  };
  int sp_new = -1, sp_ent = -1;  // APPEND: the slots whose rows this workgroup made
  auto stage = [&](int buf, uint32_t mask8, int tile) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = raw[i];
      if (KVFMT != LCA_BF16) {  // 8 OCP e4m3 dims -> bf16 (exact) for lanes < 56
        const uint4 c = make_uint4(fp8x2_to_bf16x2<false>(raw[i].x), fp8x2_to_bf16x2<true>(raw[i].x),
                                   fp8x2_to_bf16x2<false>(raw[i].y), fp8x2_to_bf16x2<true>(raw[i].y));
        if (lane < 56) v = c;
      }
      if (!((mask8 >> i) & 1u)) v = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&kv_s[buf][dkv(w + NW * i, lane * 8)]) = v;
    }
    if constexpr (APPEND) {
      // the rows this workgroup made replace what was loaded for their slots
      // (the same wave staged that row just above; the stored bytes are read at
      // lane_off and widened as a loaded row is)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int sp = a ? sp_ent : sp_new;
        const int r = sp - (s_begin + kMT * tile);
        if (sp >= 0 && r >= 0 && r < kMT && (r & (NW - 1)) == w) {
          const uint8_t* src = reinterpret_cast<const uint8_t*>(app_s[a]) + lane_off;
          uint4 v;
          if (KVFMT == LCA_BF16 || lane >= 56) {
            v = *reinterpret_cast<const uint4*>(src);
          } else {
            const uint2 h = *reinterpret_cast<const uint2*>(src);
            v = make_uint4(fp8x2_to_bf16x2<false>(h.x), fp8x2_to_bf16x2<true>(h.x),
                           fp8x2_to_bf16x2<false>(h.y), fp8x2_to_bf16x2<true>(h.y));
          }
          *reinterpret_cast<uint4*>(&kv_s[buf][dkv(r, lane * 8)]) = v;
        }
      }
    }
    if (lane == 0) vm_s[buf][w] = mask8;
  };

  // issue order: the index entries of the first two tiles (paged: three), the
  // query fragments, (paged: the pages of the first two tiles' entries,) then the
  // first tile's rows
  const int e_first = entry(0);
  int e_next = entry(1);
  int e_next2 = PAGED ? entry(2) : 0;
  if constexpr (APPEND) {
    sc.t = ap.n_tokens[b];  // the new token's position p (n_q = 1: row == b)
    sc.vis = visible_entries(sc.t, m, sc.t < 0 ? 0 : min((sc.t + 1) / m, N_cap), N_cap);
  } else {
    sc.t = q_pos[row];
    sc.vis = visible_entries(sc.t, m, n_entries[b], N_cap);
  }
  uint4 qf[kMC / 64];
  {
    const uint16_t* qh = q + (static_cast<size_t>(row) * kMH + head) * kMC + 128 * kq + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kMC / 64; ++ks) qf[ks] = *reinterpret_cast<const uint4*>(qh + 16 * ks);
  }
  uint32_t mask_cur;
  int pid_first = 0, pid_next = 0;
  if constexpr (PAGED) {
    pid_first = page_of(e_first);
    pid_next = page_of(e_next);
  }
  load_rows(row_ptr(0, e_first, pid_first, mask_cur));

  if constexpr (APPEND) {
    // the state append of the step (while the first tile's rows are in flight)
    const int p = sc.t;
    const int s_new = p >= 0 && (p + 1) % m == 0 ? (p + 1) / m - 1 : -1;  // the entry p completes
    if (p >= 0 && NT - 1 >= s_begin && NT - 1 < s_end) sp_new = NT - 1;      // window slot of p
    if (s_new >= 0 && s_new < N_cap && s_new >= s_begin && s_new < s_end) sp_ent = s_new;
    constexpr int CPL = kMC / kWave;
    const size_t io_row = row_bytes(LCA_BF16, kMC);
    float tc[CPL], tz[CPL];
    if (sp_new >= 0 || sp_ent >= 0) {
      load_row<CPL>(ap.tokC + static_cast<size_t>(b) * io_row, LCA_BF16, kMC, lane, tc);
      load_row<CPL>(ap.tokZ + static_cast<size_t>(b) * io_row, LCA_BF16, kMC, lane, tz);
    }
    const float2 rope_p = rope_step != 0.0 ? rope_cs_lane(p, rope_step) : make_float2(1.f, 0.f);
    uint8_t* tCb = ap.tailC + static_cast<size_t>(b) * m * io_row;
    uint8_t* tZb = ap.tailZ + static_cast<size_t>(b) * m * io_row;
    if (sp_new >= 0) {
      if (w == 0) {  // window row: into the ring and into LDS
        float u[CPL];
        window_row<CPL>(tc, kMC, eps, u);
        if (rope_step != 0.0) rope_lane<CPL>(u, lane, kMC, rope_p);
        store_row<CPL>(ap.ring + (static_cast<size_t>(b) * W_cap + p % n_win) * sc.kv_row, KVFMT, kMC,
                       lane, u);
        store_row<CPL>(app_s[0], KVFMT, kMC, lane, u);
        if (lane == 0) {
          ap.q_pos[b] = p;
          ap.n_entries[b] = min((p + 1) / m, N_cap);
        }
      } else if (w == 1) {  // the token's tail rows
        store_row<CPL>(tCb + static_cast<size_t>(p % m) * io_row, LCA_BF16, kMC, lane, tc);
      } else if (w == 2) {
        store_row<CPL>(tZb + static_cast<size_t>(p % m) * io_row, LCA_BF16, kMC, lane, tz);
      }
    }
    if (sp_ent >= 0) {  // the completed block, pooled by all eight waves
      Pool pool[CPL];
      pool_init<CPL>(pool);
      pool_tail<CPL, LCA_BF16>(0, m, m, 0, s_new, p % m, tCb, tZb, ap.P, kMC, lane, w, tc, tz, pool);
      int order[kPoolWaves];
#pragma unroll
      for (int x = 0; x < kPoolWaves; ++x) order[x] = x;
      static_assert(kPoolWaves == NW, "one pooling wave per decode wave");
      static_assert(sizeof(float) * kPoolWaves * 3 * CPL * kWave <= sizeof(kv_s[1]), "pool scratch");
      auto part = reinterpret_cast<float (*)[3][CPL][kWave]>(&kv_s[1][0]);
      float e[CPL];
      if (pool_combine_norm<CPL>(part, pool, order, w, lane, kMC, eps, e)) {
        if (rope_step != 0.0) rope_lane<CPL>(e, lane, kMC, rope_p);  // the entry's last token is p
        const long long out_row = kv_row_of(pg, b, N_cap, s_new);
        if (LCA_DEVICE_CHECKS && lane == 0) dbg_check(out_row >= 0);
        if (out_row >= 0)
          store_row<CPL>(ap.cache + static_cast<size_t>(out_row) * sc.kv_row, KVFMT, kMC, lane, e);
        store_row<CPL>(app_s[1], KVFMT, kMC, lane, e);
      }
    }
    // app_s is read after the query's normalisation barrier below
  }

  // RMSNorm of the query over its 512 dims: lane halves and the four waves of a
  // head half hold an eighth each; the wave sums go through LDS
  {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < kMC / 64; ++ks) {
      const uint32_t w4[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16_to_f32(static_cast<uint16_t>(w4[e] & 0xffffu));
        const float c = bf16_to_f32(static_cast<uint16_t>(w4[e] >> 16));
        ss = fmaf(a, a, ss);
        ss = fmaf(c, c, ss);
      }
    }
    ss += __shfl_xor(ss, 32, 64);
    if (g == 0) ps_s[kq][head] = ss;
    if (rope_step != 0.0 && w == 0 && lane < kRopeDims / 2) rope_s[lane] = rope_cs(sc.t, lane, rope_step);
    if (tid == 0) raise_s[0] = 0;
    __syncthreads();
    const float r = rsqrt_hw(((ps_s[0][head] + ps_s[1][head]) + (ps_s[2][head] + ps_s[3][head])) /
                                 static_cast<float>(kMC) + eps);
    // the rotary dims 448..511 (k-steps 4..7 of the kq = 3 waves) turned to the
    // query position
    const bool rope_q = rope_step != 0.0 && kq == 3;
    constexpr int kRopeStep = (kMC - kRopeDims - 384) / 16;
#pragma unroll
    for (int ks = 0; ks < kMC / 64; ++ks) {
      uint32_t w4[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = bf16_to_f32(static_cast<uint16_t>(w4[e] & 0xffffu)) * r;
        float y = bf16_to_f32(static_cast<uint16_t>(w4[e] >> 16)) * r;
        if (ks >= kRopeStep && rope_q) rope_turn(x, y, rope_s[8 * (ks - kRopeStep) + 4 * g + e]);
        w4[e] = pack_bf16(x, y);
      }
      qf[ks] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;  // softmax state of `head`
  v16f_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = v16f_t{0};
  const int tr_r = (lane & 15) >> 2;
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int rb = kq >> 1, rh = kq & 1;  // this wave's 16 rows: block rb, registers 8 rh .. +8

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    stage(buf, mask_cur, t);
    uint32_t mask_next = 0;
    const uint8_t* p_next = row_ptr(t + 1, e_next, pid_next, mask_next);
    if constexpr (PAGED) {
      pid_next = page_of(e_next2);
      e_next = e_next2;
      e_next2 = entry(t + 3);
    } else {
      e_next = entry(t + 2);
    }
    __syncthreads();  // B1: tile t staged (ps_s of the last tile read)
    if (t + 1 < n_tiles) load_rows(p_next);  // in flight during this tile's compute
    mask_cur = mask_next;

    // partial S^T over this wave's 128 dims for the rows 0..31 (acc[0]) and
    // 32..63 (acc[1])
    v16f_t acc[2];
    {
      acc[0] = v16f_t{0};
      acc[1] = v16f_t{0};
      // rows j32 and 32 + j32 share their swizzle (it depends on r mod 16)
      const uint16_t* kb0 = &kv_s[buf][j32 * kDQS];
      const uint16_t* kb1 = &kv_s[buf][(32 + j32) * kDQS];
      const int kc = 16 * kq + g, sw = dswz(j32);
#pragma unroll
      for (int ks = 0; ks < kMC / 64; ++ks) {
        const int off = ((kc + 2 * ks) ^ sw) << 3;  // chunk 16 kq + g + 2 ks, permuted
        const uint4 a0 = *reinterpret_cast<const uint4*>(kb0 + off);
        const uint4 a1 = *reinterpret_cast<const uint4*>(kb1 + off);
        acc[0] = mfma_bf16(as_v8bf(a0), as_v8bf(qf[ks]), acc[0]);
        acc[1] = mfma_bf16(as_v8bf(a1), as_v8bf(qf[ks]), acc[1]);
      }
    }
    // exchange through the free KV buffer: sx[wave][16 blk + r][lane]
    float* sx = reinterpret_cast<float*>(kv_s[buf ^ 1]);
    {
      float* sw = sx + w * 2048 + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sw[r * 64] = acc[0][r];
        sw[(16 + r) * 64] = acc[1][r];
      }
    }
    __syncthreads();  // B2: partial scores
    // full scores of this wave's rows 16 kq + 8 (i/4) + 4 g + i%4, summed over the
    // four dim quarters in quarter order
    // (the wave's own partial is read back from LDS too, so every row sums in the
    // same order whichever wave holds it)
    float s8[8];
    {
      float tot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const float* pw = sx + (hg + 2 * qq) * 2048 + (16 * rb + 8 * rh) * 64 + lane;
#pragma unroll
        for (int i = 0; i < 8; ++i) tot[i] += pw[i * 64];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) s8[i] = tot[i] * tau;
    }
    {
      // empty rows -> -inf.  Tile row 16 kq + 8 (i/4) + 4 g + i%4 was loaded by
      // wave 4 g + i%4 as its row number 2 kq + i/4.
      const uint4 v0 = *reinterpret_cast<const uint4*>(&vm_s[buf][0]);
      const uint4 v1 = *reinterpret_cast<const uint4*>(&vm_s[buf][4]);
      if (((v0.x & v0.y & v0.z & v0.w & v1.x & v1.y & v1.z & v1.w) & 0xffu) != 0xffu) {
        const uint32_t vmw[4] = {g ? v1.x : v0.x, g ? v1.y : v0.y, g ? v1.z : v0.z, g ? v1.w : v0.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (!((vmw[i & 3] >> (2 * kq + (i >> 2))) & 1u)) s8[i] = -INFINITY;
      }
    }
    float tq = s8[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tq = fmaxf(tq, s8[i]);
    tq = fmaxf(tq, __shfl_xor(tq, 32, 64));
    // The running maximum moves only when a head's tile maximum passes it by
    // more than kLazyMax (always on a split's first tile with a visible row).
    // The first tile exchanges the row quarters' maxima as the rule needs.
    // Later tiles: each wave checks its own row quarter and raises a flag, P is
    // written with the running maximum, and only a raised flag (seen by every
    // wave after B3) costs the exchange and a second P pass -- the same maxima,
    // P and sums as exchanging on every tile, one barrier fewer on the tiles
    // that do not raise it.
    auto write_p = [&](float m_use) {
      // P of this wave's 16 rows
      float psum = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        uint32_t pk[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float p0 = __expf(s8[4 * q4 + 2 * u] - m_use);
          const float p1 = __expf(s8[4 * q4 + 2 * u + 1] - m_use);
          pk[u] = pack_bf16(p0, p1);
          psum += bf16_to_f32(static_cast<uint16_t>(pk[u] & 0xffffu)) +
                  bf16_to_f32(static_cast<uint16_t>(pk[u] >> 16));
        }
        *reinterpret_cast<uint2*>(&p_s[head * kPS + 16 * kq + 8 * q4 + 4 * g]) = make_uint2(pk[0], pk[1]);
      }
      psum += __shfl_xor(psum, 32, 64);
      if (g == 0) ps_s[kq][head] = psum;
    };
    bool exchange = t == 0;
    if (!exchange) {  // (t is the same for every thread)
      if (__ballot(tq > m_run + kLazyMax) && lane == 0) raise_s[t & 1] = 1;
      write_p(m_run == -INFINITY ? 0.f : m_run);
      __syncthreads();  // B3: P and the row-quarter sums (and the flag)
      exchange = raise_s[t & 1] != 0;
    }
    float m_new = m_run, alpha = 1.f;
    if (exchange) {  // (the same for every thread)
      if (g == 0) mx_s[kq][head] = tq;
      __syncthreads();  // B3a: the row quarters' maxima
      const float tmax = fmaxf(fmaxf(mx_s[0][head], mx_s[1][head]), fmaxf(mx_s[2][head], mx_s[3][head]));
      m_new = (m_run == -INFINITY || tmax > m_run + kLazyMax) ? tmax : m_run;
      alpha = (m_run == -INFINITY || m_new == m_run) ? 1.f : __expf(m_run - m_new);
      write_p(m_new == -INFINITY ? 0.f : m_new);
      __syncthreads();  // B3b: P and the sums again
    }
    if (tid == 0) raise_s[(t + 1) & 1] = 0;  // (read again after tile t + 1's B3 only)
    l_run = l_run * alpha + ((ps_s[0][head] + ps_s[1][head]) + (ps_s[2][head] + ps_s[3][head]));
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float al = __shfl(alpha, 8 * (r >> 2) + 4 * g + (r & 3), 64);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db][r] *= al;
      }
    }
    // O[heads 32 hg + .., dims 128 kq + ..] += P V
#pragma unroll
    for (int ks = 0; ks < kMT / 16; ++ks) {
      const v8bf_t A = as_v8bf(*reinterpret_cast<const uint4*>(&p_s[head * kPS + 16 * ks + 8 * g]));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int vr = 16 * ks + 8 * g + tr_r, vc = 128 * kq + 32 * db + tr_d;
        const uint2 lo = tr_rows4(&kv_s[buf][dkv(vr, vc)]);
        const uint2 hi = tr_rows4(&kv_s[buf][dkv(vr + 4, vc)]);
        o[db] = mfma_bf16(A, as_v8bf(make_uint4(lo.x, lo.y, hi.x, hi.y)), o[db]);
      }
    }
  }

  // epilogue: O / l (with the sink when this is the only split); lse = m + log l
  float lse_v = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
  float f = l_run > 0.f ? 1.0f / l_run : 0.f;
  if (n_splits == 1 && sink) {
    const float sk = sink[head];
    if (lse_v == -INFINITY) {
      lse_v = sk;
    } else {
      const float mx = fmaxf(lse_v, sk);
      const float tot = mx + __logf(__expf(lse_v - mx) + __expf(sk - mx));
      f *= __expf(lse_v - tot);
      lse_v = tot;
    }
  }
  if (kq == 0 && g == 0) {
    if (n_splits == 1) {
      if (lse) lse[static_cast<size_t>(row) * kMH + head] = lse_v;
    } else {
      part_lse[(static_cast<size_t>(row) * n_splits + split) * kMH + head] = lse_v;
    }
  }
  if (n_splits > 1) {
    // fp16 partial rows straight from the accumulators (a lane's 32 columns of
    // a head are 64 contiguous bytes; the merge turns the output back).  A
    // split's normalised O is a convex combination of RMS-normalised rows, so
    // |O| <= sqrt(512) and fp16 holds it to 2^-11 relative (round to nearest)
    _Float16* pb = reinterpret_cast<_Float16*>(part_o) +
                   (static_cast<size_t>(row) * n_splits + split) * kMH * kMC + 128 * kq + j32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = 32 * hg + 8 * (r >> 2) + 4 * g + (r & 3);
      const float fr = __shfl(f, 8 * (r >> 2) + 4 * g + (r & 3), 64);
#pragma unroll
      for (int db = 0; db < 4; ++db) pb[h * kMC + 32 * db] = static_cast<_Float16>(o[db][r] * fr);
    }
    return;
  }
  // one split: O * f -> LDS as fp32 [64 heads][512] (over both KV buffers, once
  // every wave is done with them), then contiguous 16-byte stores
  float* ost = reinterpret_cast<float*>(&kv_s[0][0]);
  __syncthreads();
  // APPEND with one split: no merge follows, and every wave read n_tokens
  // before the barriers behind it
  if (APPEND && tid == 0 && sc.t >= 0) ap.n_tokens[b] = sc.t + 1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int h = 32 * hg + 8 * (r >> 2) + 4 * g + (r & 3);
    const float fr = __shfl(f, 8 * (r >> 2) + 4 * g + (r & 3), 64);
#pragma unroll
    for (int db = 0; db < 4; ++db) ost[h * kMC + 128 * kq + 32 * db + j32] = o[db][r] * fr;
  }
  __syncthreads();
  const size_t obase = static_cast<size_t>(row) * kMH * kMC;
  // 64 x 512 fp32 = 8192 chunks of 16 B; thread tid writes chunks tid + 512 i
#pragma unroll 4
  for (int i = 0; i < kMH * kMC / 4 / (64 * NW); ++i) {
    const int c4 = (tid + 64 * NW * i) * 4;
    float4 v = *reinterpret_cast<const float4*>(&ost[c4]);
    if (rope_step != 0.0 && (c4 & (kMC - 1)) >= kMC - kRopeDims) {  // the output turned back by -t
      const int pr = ((c4 & (kMC - 1)) - (kMC - kRopeDims)) >> 1;
      const float2 c0 = rope_s[pr], c1 = rope_s[pr + 1];
      rope_turn(v.x, v.y, make_float2(c0.x, -c0.y));
      rope_turn(v.z, v.w, make_float2(c1.x, -c1.y));
    }
    if (out_fmt == LCA_F32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + obase + c4) = v;
    } else {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + obase + c4) =
          make_uint2(pack_bf16(v.x, v.y), pack_bf16(v.z, v.w));
    }
  }
}

// Splits per query row are capped so that each split stays a few tiles long.
constexpr int kMaxMergeSplits = 256;

// Split merge with one thread per 4 consecutive dims of a (query row, head).
// The lse values and partial rows of up to CH splits are loaded together, so a
// merge of that many splits takes one memory round trip; more splits go CH at a
// time with a running maximum.  Splits are combined in split order
// (deterministic).  CH (4 .. 20) is the split count rounded up to a multiple of
// 4, so few loads are clamped repeats of the last split; more than 20 splits go
// 16 at a time.  H16: the partial rows are fp16 (the decode kernel's), else
// fp32; fp16 rows stay packed until used, which leaves registers for 32- and
// 48-split instances.
// One-wave workgroups: a small batch's merge (4 query rows: 32K threads) then
// spreads over every CU instead of half of them (256-thread groups made the
// hybrid stack's merges 2.4 us slower per step).
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
constexpr int kMergeThreads = 64;
template <int CH, bool H16>
__global__ __launch_bounds__(kMergeThreads) void attn_merge4_kernel(
    long long rows, int H, int c, int n_splits, const void* __restrict__ part_o,
    const float* __restrict__ part_lse, const float* __restrict__ sink, uint8_t* __restrict__ out,
    int out_fmt, float* __restrict__ lse, const int32_t* __restrict__ q_pos, double rope_step,
    int32_t* __restrict__ advance) {
  const int c4n = c / 4;
  const long long gid = static_cast<long long>(blockIdx.x) * kMergeThreads + threadIdx.x;
  // the angles of -t for the output's turn back: a block covers one query row
  // (H * c / 4 is a multiple of 256, checked by the launcher)
  __shared__ float2 rope_s[kRopeDims / 2];
  if (rope_step != 0.0) {
    const long long row0 = static_cast<long long>(blockIdx.x) * kMergeThreads / (static_cast<long long>(H) * c4n);
    if (threadIdx.x < kRopeDims / 2)
      rope_s[threadIdx.x] = rope_cs(-static_cast<long long>(q_pos[row0]), threadIdx.x, rope_step);
    __syncthreads();
  }
  // a decode step whose attention appended the token: n_tokens[row] += 1 (no
  // other launch of the step reads it any more; a negative count stays)
  if (advance && gid < rows && advance[gid] >= 0) advance[gid] += 1;
  if (gid >= rows * H * c4n) return;
  const long long rh = gid / c4n;
  const int d4 = static_cast<int>(gid % c4n) * 4;
  const long long row = rh / H;
  const int h = static_cast<int>(rh % H);
  // the sink is one more logit in the denominator, with no value row
  float m = sink ? sink[h] : -INFINITY;
  float den = sink ? 1.f : 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < n_splits; s0 += CH) {
    float l[CH];
    [[maybe_unused]] float4 v[H16 ? 1 : CH];
    [[maybe_unused]] h4_t vh[H16 ? CH : 1];  // fp16 rows kept packed until used
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int sp = min(s0 + u, n_splits - 1);
      const size_t base = (static_cast<size_t>(row) * n_splits + sp) * H + h;
      l[u] = part_lse[base];
      if constexpr (H16)
        vh[u] = *reinterpret_cast<const h4_t*>(static_cast<const _Float16*>(part_o) + base * c + d4);
      else
        v[u] = *reinterpret_cast<const float4*>(static_cast<const float*>(part_o) + base * c + d4);
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (s0 + u >= n_splits) l[u] = -INFINITY;
      mc = fmaxf(mc, l[u]);
    }
    if (mc == -INFINITY) continue;  // no rows so far
    const float sc = m == -INFINITY ? 0.f : __expf(m - mc);
    den *= sc;
    acc.x *= sc;
    acc.y *= sc;
    acc.z *= sc;
    acc.w *= sc;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float wgt = l[u] == -INFINITY ? 0.f : __expf(l[u] - mc);
      den += wgt;
      float4 vu;
      if constexpr (H16)
        vu = make_float4(static_cast<float>(vh[u][0]), static_cast<float>(vh[u][1]),
                         static_cast<float>(vh[u][2]), static_cast<float>(vh[u][3]));
      else
        vu = v[u];
      acc.x = fmaf(wgt, vu.x, acc.x);
      acc.y = fmaf(wgt, vu.y, acc.y);
      acc.z = fmaf(wgt, vu.z, acc.z);
      acc.w = fmaf(wgt, vu.w, acc.w);
    }
    m = mc;
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (rope_step != 0.0 && d4 >= c - kRopeDims) {  // the output turned back by -t
    const int pr = (d4 - (c - kRopeDims)) >> 1;
    rope_turn(o.x, o.y, rope_s[pr]);
    rope_turn(o.z, o.w, rope_s[pr + 1]);
  }
  const size_t oi = static_cast<size_t>(rh) * c + d4;
  if (out_fmt == LCA_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + oi) = o;
  } else {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + oi) =
        make_uint2(pack_bf16(o.x, o.y), pack_bf16(o.z, o.w));
  }
  if (lse && d4 == 0) lse[rh] = den > 0.f ? m + __logf(den) : -INFINITY;
}

struct Plan {
  int n_splits, split_rows;
  bool mfma;    // 64 heads x 512 on the MFMA kernels
  bool decode;  // ... with the decode kernel (few rows, bf16 queries)
};

bool use_mfma(int H, int c, int q_fmt, int kv_fmt) {
  return H == kMH && c == kMC && (q_fmt == LCA_BF16 || q_fmt == LCA_F32) &&
         (kv_fmt == LCA_BF16 || kv_fmt == LCA_KV_FP8_BF16ROPE);
}

// fixed_split > 0 (a multiple of kMT): that many candidate rows per split,
// whatever the number of query rows, so a query's result does not depend on
// the batch; 0: the automatic plan below.
Plan make_plan(long long rows, int H, int c, int q_fmt, int kv_fmt, int k, int N_cap, int n_win,
               int dense, int fixed_split) {
  const int NT = (dense ? N_cap : k) + n_win;
  Plan p;
  p.mfma = use_mfma(H, c, q_fmt, kv_fmt);
  p.decode = p.mfma && q_fmt == LCA_BF16;
  if (fixed_split > 0) {
    p.split_rows = fixed_split < NT ? fixed_split : NT;
    p.n_splits = (NT + fixed_split - 1) / fixed_split;
    if (p.n_splits < 1) p.n_splits = 1;
    return p;
  }
  if (rows >= 512) {
    p.n_splits = 1;
    p.split_rows = NT;
    return p;
  }
  int split_rows;
  if (p.mfma) {
    // one workgroup per CU and one round: about 256 / rows splits per row, each a
    // whole number of 64-row tiles
    const long long want = rows >= 256 ? 1 : 256 / rows;
    const long long per = (NT + want - 1) / want;
    split_rows = static_cast<int>(((per + kMT - 1) / kMT) * kMT);
  } else {
    split_rows = kSplitRows;
  }
  if (split_rows < kMT) split_rows = kMT;
  const int min_rows = (NT + kMaxMergeSplits - 1) / kMaxMergeSplits;
  if (split_rows < min_rows) split_rows = ((min_rows + kMT - 1) / kMT) * kMT;
  p.split_rows = split_rows;
  p.n_splits = (NT + split_rows - 1) / split_rows;
  return p;
}

}  // namespace

bool mqa_can_append(long long rows, int H, int c, int q_fmt, int kv_fmt, int N_cap, int n_win,
                    int fixed_split) {
  return n_win >= 1 && make_plan(rows, H, c, q_fmt, kv_fmt, 0, N_cap, n_win, 1, fixed_split).decode;
}

int mqa_splits(int k, int N_cap, int n_win, int dense, int fixed_split) {
  const int NT = (dense ? N_cap : k) + n_win;
  return fixed_split > 0 ? (NT + fixed_split - 1) / fixed_split : 0;
}

size_t mqa_workspace_bytes(int B, int n_q, int H, int c, int kv_fmt, int k, int N_cap, int n_win,
                           int dense, int fixed_split) {
  const long long rows = static_cast<long long>(B) * n_q;
  // the plan does not depend on q_fmt beyond F32/BF16, which both allow the MFMA path
  const Plan p = make_plan(rows, H, c, LCA_BF16, kv_fmt, k, N_cap, n_win, dense, fixed_split);
  if (p.n_splits == 1) return 0;
  const size_t n = static_cast<size_t>(rows) * p.n_splits * H;
  return n * c * sizeof(float) + ((n * sizeof(float) + 255) & ~static_cast<size_t>(255)) + 256;
}

#define LCA_ATTN_CPL(c, KERNEL, GRID, BLOCK, ...)                                         \
  do {                                                                                    \
    switch ((c) / 64) {                                                                   \
      case 2: hipLaunchKernelGGL(KERNEL<2>, GRID, BLOCK, 0, s, __VA_ARGS__); break;       \
      case 4: hipLaunchKernelGGL(KERNEL<4>, GRID, BLOCK, 0, s, __VA_ARGS__); break;       \
      case 8: hipLaunchKernelGGL(KERNEL<8>, GRID, BLOCK, 0, s, __VA_ARGS__); break;       \
      default: return hipErrorInvalidValue;                                               \
    }                                                                                     \
  } while (0)

hipError_t launch_mqa(int B, int n_q, int H, int c, const void* q, int q_fmt, const void* cache,
                      int kv_fmt, int N_cap, const int32_t* idx, int k, const int32_t* q_pos, int m,
                      const int32_t* n_entries, const void* win, int W_cap, int64_t win_origin,
                      int n_win, float tau, float eps, const float* sink, double rope_step, void* out,
                      int out_fmt, float* lse, void* ws, const KvPages& pg, hipStream_t s,
                      int fixed_split, const DecodeAppend* append) {
  const long long rows = static_cast<long long>(B) * n_q;
  if (rows == 0) return hipSuccess;
  const int dense = idx == nullptr;
  const Plan p = make_plan(rows, H, c, q_fmt, kv_fmt, k, N_cap, n_win, dense, fixed_split);
  // the in-kernel append: the decode kernel over dense rows, one query per
  // sequence, the ring as the window (W_cap = n_win, origin 0)
  if (append && (!p.decode || !dense || n_q != 1 || W_cap != n_win || win_origin != 0 || n_win < 1 ||
                 win != append->ring || cache != append->cache))
    return hipErrorInvalidValue;
  const DecodeAppend ap = append ? *append : DecodeAppend{};
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (p.n_splits > 1) {
    const size_t n = static_cast<size_t>(rows) * p.n_splits * H;
    part_o = static_cast<float*>(ws);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + n * c * sizeof(float));
  }
  if (p.decode) {
    const dim3 grid(static_cast<unsigned>(rows * p.n_splits));
    const dim3 block(64 * kD8Waves);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, block, 0, s, n_q, static_cast<const uint16_t*>(q),
                         static_cast<const uint8_t*>(cache), N_cap, idx, k, q_pos, m, n_entries,
                         static_cast<const uint8_t*>(win), W_cap, static_cast<long long>(win_origin),
                         n_win, tau, eps, sink, rope_step, p.n_splits, p.split_rows,
                         static_cast<uint8_t*>(out), out_fmt, lse, part_o, part_lse, pg, ap);
    };
    const bool paged = pg.bt != nullptr;
    if (append) {
      if (kv_fmt == LCA_BF16)
        paged ? go(attn_decode_kernel<LCA_BF16, true, true>) : go(attn_decode_kernel<LCA_BF16, false, true>);
      else
        paged ? go(attn_decode_kernel<LCA_KV_FP8_BF16ROPE, true, true>)
              : go(attn_decode_kernel<LCA_KV_FP8_BF16ROPE, false, true>);
    } else if (kv_fmt == LCA_BF16) {
      paged ? go(attn_decode_kernel<LCA_BF16, true, false>) : go(attn_decode_kernel<LCA_BF16, false, false>);
    } else {
      paged ? go(attn_decode_kernel<LCA_KV_FP8_BF16ROPE, true, false>)
            : go(attn_decode_kernel<LCA_KV_FP8_BF16ROPE, false, false>);
    }
  } else if (p.mfma) {
    const dim3 grid(static_cast<unsigned>(rows * p.n_splits));
    if (kv_fmt == LCA_BF16)
      hipLaunchKernelGGL(attn_mfma_kernel<LCA_BF16>, grid, dim3(256), 0, s, n_q,
                         static_cast<const uint8_t*>(q), q_fmt, static_cast<const uint8_t*>(cache),
                         N_cap, idx, k, q_pos, m, n_entries, static_cast<const uint8_t*>(win), W_cap,
                         static_cast<long long>(win_origin), n_win, tau, eps, sink, rope_step, p.n_splits,
                         p.split_rows, static_cast<uint8_t*>(out), out_fmt, lse, part_o, part_lse, pg);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<LCA_KV_FP8_BF16ROPE>, grid, dim3(256), 0, s, n_q,
                         static_cast<const uint8_t*>(q), q_fmt, static_cast<const uint8_t*>(cache),
                         N_cap, idx, k, q_pos, m, n_entries, static_cast<const uint8_t*>(win), W_cap,
                         static_cast<long long>(win_origin), n_win, tau, eps, sink, rope_step, p.n_splits,
                         p.split_rows, static_cast<uint8_t*>(out), out_fmt, lse, part_o, part_lse, pg);
  } else {
  const dim3 grid(static_cast<unsigned>(rows * (H / kHG) * p.n_splits));
  LCA_ATTN_CPL(c, attn_generic_kernel, grid, dim3(kAttnThreads), n_q, H, c,
               static_cast<const uint8_t*>(q), q_fmt, static_cast<const uint8_t*>(cache), kv_fmt,
               N_cap, idx, k, q_pos, m, n_entries, static_cast<const uint8_t*>(win), W_cap,
               static_cast<long long>(win_origin), n_win, tau, eps, sink, rope_step, p.n_splits, p.split_rows,
               static_cast<uint8_t*>(out), out_fmt, lse, part_o, part_lse, pg);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  if (rope_step != 0.0 && (static_cast<long long>(H) * (c / 4)) % 256 != 0) return hipErrorInvalidValue;
  int32_t* advance = append ? append->n_tokens : nullptr;
  const dim3 g2(static_cast<unsigned>((rows * H * (c / 4) + kMergeThreads - 1) / kMergeThreads));
  auto merge = [&](auto kern) {
    hipLaunchKernelGGL(kern, g2, dim3(kMergeThreads), 0, s, rows, H, c, p.n_splits, static_cast<const void*>(part_o),
                       part_lse, sink, static_cast<uint8_t*>(out), out_fmt, lse, q_pos, rope_step,
                       advance);
  };
  // the decode kernel writes fp16 partials, the other kernels fp32
  auto merge_ch = [&](auto h16) {
    constexpr bool H16 = decltype(h16)::value;
    if (p.n_splits <= 4) merge(attn_merge4_kernel<4, H16>);
    else if (p.n_splits <= 8) merge(attn_merge4_kernel<8, H16>);
    else if (p.n_splits <= 12) merge(attn_merge4_kernel<12, H16>);
    else if (p.n_splits <= 16) merge(attn_merge4_kernel<16, H16>);
    else if (p.n_splits <= 20) merge(attn_merge4_kernel<20, H16>);
    else if (H16 && p.n_splits <= 32) merge(attn_merge4_kernel<32, H16>);
    else if (H16 && p.n_splits <= 48) merge(attn_merge4_kernel<48, H16>);
    else merge(attn_merge4_kernel<16, H16>);
  };
  if (p.decode) merge_ch(std::true_type{});
  else merge_ch(std::false_type{});
  return hipGetLastError();
}

LCA_DBG_ACCESSOR(dbg_violations_attention)

}  // namespace lca
