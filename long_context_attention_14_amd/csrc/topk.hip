// Per-query top-k selection of indexer scores ("DeepSeek V4 Architecture
// Tricks", section "CSA": top-k = 1024; QbitAI article on DeepSeek-V4, hybrid
// attention section: at 1M tokens a query attends 1024 compressed blocks).
//
// Scores become order-preserving uint32 keys (-0 -> +0, NaN -> -inf first), so
// "largest score, lower index first among equals" is "largest key, lowest index
// first".  The k-th largest key T is found by MSB-first radix select on integer
// histograms (no floating-point atomics: the result is deterministic), then the
// selected indices are compacted in index order: every key > T, plus the first
// (k - #{key > T}) keys equal to T.  The output is therefore ascending.
//
// Two paths:
//  * rows of at most kLdsMaxRow entries (prefill): one 1024-thread workgroup
//    per row keeps the whole row's keys in LDS (up to 144 KiB of gfx950's
//    160 KiB) and runs four 8-bit radix passes there;
//  * longer rows (decode at 1M context: 262144 entries): many workgroups per
//    row build a 4096-bin histogram of the top 12 key bits; the bin holding the
//    k-th key splits the row into "surely selected" (higher bins) and
//    "candidates" (that bin); a second pass compacts both per segment in index
//    order; a last one-workgroup-per-row pass radix-selects among the
//    candidates on the remaining 20 bits and merges the two sorted lists.
#include "common.h"
#include "pool.h"

namespace lca {
namespace {

constexpr int kLdsMaxRow = 36864;
constexpr int kRowThreads = 1024;
constexpr int kSeg = 8192;
constexpr int kSegThreads = 256;
constexpr int kHistBins = kScoreHistBins;

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// ---------------------------------------------------------------------------
// LDS path

// Block-wide exclusive prefix of two per-thread counts (kRowThreads threads);
// also returns the totals.  scan_a/scan_b hold kRowThreads/64 ints each.
__device__ __forceinline__ void block_scan2(int a, int b, int* ea, int* eb, int* ta, int* tb,
                                            int* scan_a, int* scan_b) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int va = __shfl_up(ia, o, 64), vb = __shfl_up(ib, o, 64);
    if (lane >= o) {
      ia += va;
      ib += vb;
    }
  }
  if (lane == 63) {
    scan_a[wv] = ia;
    scan_b[wv] = ib;
  }
  __syncthreads();
  int oa = ia - a, ob = ib - b, sa = 0, sb = 0;
  for (int x = 0; x < kRowThreads / 64; ++x) {
    if (x < wv) {
      oa += scan_a[x];
      ob += scan_b[x];
    }
    sa += scan_a[x];
    sb += scan_b[x];
  }
  *ea = oa;
  *eb = ob;
  *ta = sa;
  *tb = sb;
}


// ST: float, or uint16_t for bf16 scores (16-bit keys: two 8-bit passes).
// One workgroup per row, the row's keys in LDS.  The radix histograms have
// kHistCopies copies (lane l adds to copy l % kHistCopies, copies 257 words
// apart so that a bin's copies sit in different banks): the top key bits of a
// row of scores take very few distinct values, and LDS atomics to one address
// within an instruction are serialised.  The index-order compaction counts
// every round's selected entries per wave first, so one block scan gives all
// output offsets (no barrier per 1024 entries).
constexpr int kHistCopies = 8;
constexpr int kHistStride = 257;
constexpr int kMaxRounds = (kLdsMaxRow + kRowThreads - 1) / kRowThreads;  // 36
constexpr int kRowWaves = kRowThreads / 64;

template <typename ST>
__global__ __launch_bounds__(kRowThreads) void topk_lds_kernel(
    const ST* __restrict__ scores, int N_cap, int n_q, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, int k, int32_t* __restrict__ idx) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hc[kHistCopies * kHistStride];
  __shared__ uint32_t hist[256];
  __shared__ int sh_bin, sh_above;
  __shared__ int cg[kMaxRounds * kRowWaves], ce[kMaxRounds * kRowWaves];
  __shared__ int scan_a[kRowWaves], scan_b[kRowWaves];
  const long long row = blockIdx.x;
  const int b = static_cast<int>(row / n_q);
  const int vis = visible_entries(q_pos[row], m, n_entries[b], N_cap);
  int32_t* out = idx + row * k;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (vis <= k) {
    for (int i = tid; i < k; i += kRowThreads) out[i] = i < vis ? i : -1;
    return;
  }
  // keys to LDS: every load of the row goes out at once (at most kMaxRounds
  // per thread; with eight at a time the row took four to five dependent
  // memory round trips), and the first radix pass (the top 8 bits of every
  // key) is counted as the keys are stored
  const ST* src = scores + row * N_cap;
  const int n_rounds = (vis + kRowThreads - 1) / kRowThreads;
  ST v[kMaxRounds];
#pragma unroll
  for (int u = 0; u < kMaxRounds; ++u)
    if (u < n_rounds) v[u] = src[min(u * kRowThreads + tid, vis - 1)];
  for (int i = tid; i < kHistCopies * kHistStride; i += kRowThreads) hc[i] = 0;
  __syncthreads();
  uint32_t* my_copy = hc + (lane % kHistCopies) * kHistStride;
#pragma unroll
  for (int u = 0; u < kMaxRounds; ++u) {
    const int i = u * kRowThreads + tid;
    if (u < n_rounds && i < vis) {
      const uint32_t key = stored_key(v[u]);
      keys[i] = key;
      atomicAdd(&my_copy[key >> 24], 1u);
    }
  }
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
  constexpr int kLowShift = sizeof(ST) == 2 ? 16 : 0;  // bf16 keys have no low 16 bits
  for (int shift = 24; shift >= kLowShift; shift -= 8) {
    if (shift != 24) {  // (the first pass was counted with the loads)
      for (int i = tid; i < kHistCopies * kHistStride; i += kRowThreads) hc[i] = 0;
      __syncthreads();
      for (int i = tid; i < vis; i += kRowThreads) {
        const uint32_t key = keys[i];
        if ((key & mask) == prefix) atomicAdd(&my_copy[(key >> shift) & 0xffu], 1u);
      }
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t t = 0;
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) t += hc[c * kHistStride + tid];
      hist[tid] = t;
    }
    __syncthreads();
    if (tid < 64) find_bin_wave(hist, 256, remaining, &sh_bin, &sh_above);
    __syncthreads();
    prefix |= static_cast<uint32_t>(sh_bin) << shift;
    mask |= 0xffu << shift;
    remaining -= sh_above;
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;

  // compaction in index order: entry i = 1024 r + tid.  Per-wave counts of
  // every round, one scan over (round, wave), then the writes.
  for (int r = 0; r < n_rounds; ++r) {
    const int i = r * kRowThreads + tid;
    const uint32_t key = i < vis ? keys[i] : 0u;
    const uint64_t bg = __ballot(i < vis && key > T), be = __ballot(i < vis && key == T);
    if (lane == 0) {
      cg[r * kRowWaves + wv] = __popcll(bg);
      ce[r * kRowWaves + wv] = __popcll(be);
    }
  }
  __syncthreads();
  {
    const int t = tid;  // n_rounds * kRowWaves <= kRowThreads entries, round-major
    const bool in = t < n_rounds * kRowWaves;
    const int a = in ? cg[t] : 0, c = in ? ce[t] : 0;
    int ea, ec, ta, tc;
    block_scan2(a, c, &ea, &ec, &ta, &tc, scan_a, scan_b);
    __syncthreads();  // every count read before the offsets replace them
    if (in) {
      cg[t] = ea;
      ce[t] = ec;
    }
  }
  __syncthreads();
  for (int r = 0; r < n_rounds; ++r) {
    const int i = r * kRowThreads + tid;
    const uint32_t key = i < vis ? keys[i] : 0u;
    const bool gt = i < vis && key > T;
    const bool eq = i < vis && key == T;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const int gt_before = cg[r * kRowWaves + wv] + lanes_below(bg);
    const int eq_before = ce[r * kRowWaves + wv] + lanes_below(be);
    const int pos = gt_before + min(eq_before, need_eq);
    if ((gt || (eq && eq_before < need_eq)) && pos < k) out[pos] = i;
  }
}

// ---------------------------------------------------------------------------
// histogram path for long rows

struct WideWs {
  uint32_t* hist;      // [rows, 4096]
  int32_t* sure;       // [rows, n_seg, k]
  uint32_t* cand_key;  // [rows, n_seg, kSeg]
  int32_t* cand_idx;   // [rows, n_seg, kSeg]
  int32_t* sure_cnt;   // [rows, n_seg]
  int32_t* cand_cnt;   // [rows, n_seg]
};

// Workspace carve-up; every array starts on a 256-byte boundary.
struct WideLayout {
  size_t hist, sure, cand_key, cand_idx, sure_cnt, cand_cnt, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

inline WideLayout wide_layout(long long rows, int n_seg, int k) {
  WideLayout L;
  const size_t r = static_cast<size_t>(rows), ns = static_cast<size_t>(n_seg);
  size_t off = 0;
  L.hist = off;     off += align256(r * kHistBins * 4);
  L.sure = off;     off += align256(r * ns * static_cast<size_t>(k) * 4);
  L.cand_key = off; off += align256(r * ns * kSeg * 4);
  L.cand_idx = off; off += align256(r * ns * kSeg * 4);
  L.sure_cnt = off; off += align256(r * ns * 4);
  L.cand_cnt = off; off += align256(r * ns * 4);
  L.total = off;
  return L;
}

inline WideWs wide_ws(void* base, long long rows, int n_seg, int k) {
  const WideLayout L = wide_layout(rows, n_seg, k);
  char* p = static_cast<char*>(base);
  WideWs w;
  w.hist = reinterpret_cast<uint32_t*>(p + L.hist);
  w.sure = reinterpret_cast<int32_t*>(p + L.sure);
  w.cand_key = reinterpret_cast<uint32_t*>(p + L.cand_key);
  w.cand_idx = reinterpret_cast<int32_t*>(p + L.cand_idx);
  w.sure_cnt = reinterpret_cast<int32_t*>(p + L.sure_cnt);
  w.cand_cnt = reinterpret_cast<int32_t*>(p + L.cand_cnt);
  return w;
}

__global__ void zero_u32_kernel(uint32_t* p, long long n) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <typename ST>
__global__ __launch_bounds__(kSegThreads) void topk_hist_kernel(
    const ST* __restrict__ scores, int N_cap, int n_q, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, int k, int n_seg, uint32_t* __restrict__ ghist) {
  __shared__ uint32_t h[kHistBins];
  const long long row = blockIdx.x / n_seg;
  const int seg = blockIdx.x % n_seg;
  const int b = static_cast<int>(row / n_q);
  const int vis = visible_entries(q_pos[row], m, n_entries[b], N_cap);
  if (vis <= k) return;
  const int s0 = seg * kSeg;
  if (s0 >= vis) return;
  const int s1 = min(s0 + kSeg, vis);
  for (int i = threadIdx.x; i < kHistBins; i += kSegThreads) h[i] = 0;
  __syncthreads();
  const ST* src = scores + row * N_cap;
  for (int i = s0 + threadIdx.x; i < s1; i += kSegThreads) atomicAdd(&h[score_bin(stored_key(src[i]))], 1u);
  __syncthreads();
  uint32_t* gh = ghist + row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kSegThreads)
    if (h[i]) atomicAdd(&gh[hist_slot(i)], h[i]);
}

// Threshold of a row: (bin of the k-th largest key, count of keys in higher
// bins), or (-1, vis) when every visible entry is kept.  The row histogram is
// copied to LDS (lh) with coalesced loads and searched by the whole block.
// All threads call it; the result is valid after it returns.
__device__ void row_threshold(const uint32_t* gh, uint32_t* lh, int vis, int k, int* sh_bin,
                              int* sh_above, int* scan_sh) {
  if (vis <= k) {
    if (threadIdx.x == 0) {
      *sh_bin = -1;
      *sh_above = vis;
    }
    __syncthreads();
    return;
  }
  // read in word order (coalesced), place by bin
  for (int w = threadIdx.x; w < kHistBins; w += blockDim.x) lh[hist_lds(hist_bin_of_slot(w))] = gh[w];
  __syncthreads();
  find_threshold_block(lh, k, sh_bin, sh_above, scan_sh);
}

// One workgroup per (row, segment of kSeg scores); wave wv owns the quarter
// [s0 + wv*kSeg/4, +kSeg/4) and loads it with coalesced loads (element
// base + 64 r + lane in register r).  Pass 1 counts the surely selected and the
// candidate entries of each wave with ballots; a scan of the four wave totals
// gives every wave its output offsets; pass 2 writes the indices in order.
constexpr int kQuarter = kSeg / (kSegThreads / 64);  // 2048
constexpr int kPerLane = kQuarter / 64;                // 32

template <typename ST>
__global__ __launch_bounds__(kSegThreads) void topk_collect_kernel(
    const ST* __restrict__ scores, int N_cap, int n_q, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, int k, int n_seg, WideWs ws) {
  __shared__ int wtot_s[kSegThreads / 64], wtot_c[kSegThreads / 64];
  __shared__ uint32_t lh[kHistLdsWords];
  __shared__ int sh_bin, sh_above, scan_sh[kSegThreads / 64];
  const long long row = blockIdx.x / n_seg;
  const int seg = blockIdx.x % n_seg;
  const int b = static_cast<int>(row / n_q);
  const int vis = visible_entries(q_pos[row], m, n_entries[b], N_cap);
  const int s0 = seg * kSeg;
  const int s1 = min(s0 + kSeg, vis);
  const long long rs = row * n_seg + seg;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wbase = s0 + wv * kQuarter;
  const ST* src = scores + row * N_cap;
  uint32_t kv[kPerLane];
#pragma unroll
  for (int r = 0; r < kPerLane; ++r) {
    const int i = wbase + 64 * r + lane;
    kv[r] = i < s1 ? stored_key(src[i]) : 0u;
  }
  row_threshold(ws.hist + row * kHistBins, lh, vis, k, &sh_bin, &sh_above, scan_sh);
  const int bstar = sh_bin;
  int ns = 0, nc = 0;
#pragma unroll
  for (int r = 0; r < kPerLane; ++r) {
    const int i = wbase + 64 * r + lane;
    const int bin = static_cast<int>(score_bin(kv[r]));
    ns += __popcll(__ballot(i < s1 && bin > bstar));
    nc += __popcll(__ballot(i < s1 && bin == bstar));
  }
  if (lane == 0) {
    wtot_s[wv] = ns;
    wtot_c[wv] = nc;
  }
  __syncthreads();
  int os = 0, oc = 0, ts = 0, tc = 0;
#pragma unroll
  for (int x = 0; x < kSegThreads / 64; ++x) {
    if (x < wv) {
      os += wtot_s[x];
      oc += wtot_c[x];
    }
    ts += wtot_s[x];
    tc += wtot_c[x];
  }
  int32_t* sure = ws.sure + rs * k;
  uint32_t* ckey = ws.cand_key + rs * kSeg;
  int32_t* cidx = ws.cand_idx + rs * kSeg;
#pragma unroll
  for (int r = 0; r < kPerLane; ++r) {
    const int i = wbase + 64 * r + lane;
    const uint32_t key = kv[r];
    const int bin = static_cast<int>(score_bin(key));
    const bool is_s = i < s1 && bin > bstar;
    const bool is_c = i < s1 && bin == bstar;
    const uint64_t bs = __ballot(is_s), bc = __ballot(is_c);
    const int ps = os + lanes_below(bs), pc = oc + lanes_below(bc);
    if (is_s && ps < k) sure[ps] = i;
    if (is_c) {
      ckey[pc] = key;
      cidx[pc] = i;
    }
    os += __popcll(bs);
    oc += __popcll(bc);
  }
  if (tid == 0) {
    ws.sure_cnt[rs] = s0 < vis ? ts : 0;
    ws.cand_cnt[rs] = s0 < vis ? tc : 0;
  }
}


// Radix-select the `need` largest candidates (all in one 12-bit top bin, so only
// the low 20 key bits differ; passes of 8, 8 and 4 bits) and write their indices
// to Ch in candidate order (ties: earlier candidates first).  The candidates are
// in ascending index order, so Ch is ascending.  All threads of a kRowThreads
// block call it.
template <class KeyF, class IdxF>
__device__ int select_candidates(int nCand, int need, KeyF cand_key, IdxF cand_idx, int32_t* Ch,
                                 uint32_t* hist, int* sh_b2, int* sh_a2, uint32_t* wgt,
                                 uint32_t* weq) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (need <= 0) return 0;
  uint32_t prefix = 0, mask = 0;
  int remaining = need;
  const int shifts[3] = {12, 4, 0};
  const int widths[3] = {8, 8, 4};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t dm = (1u << widths[pass]) - 1u;
    for (int i = tid; i < 256; i += kRowThreads) hist[i] = 0;
    __syncthreads();
    for (int p = tid; p < nCand; p += kRowThreads) {
      const uint32_t key = cand_key(p);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> sh) & dm], 1u);
    }
    __syncthreads();
    if (tid < 64) find_bin_wave(hist, 256, remaining, sh_b2, sh_a2);
    __syncthreads();
    prefix |= static_cast<uint32_t>(*sh_b2) << sh;
    mask |= dm << sh;
    remaining -= *sh_a2;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;
  int run_gt = 0, run_eq = 0;
  for (int base = 0; base < nCand; base += kRowThreads) {
    const int p = base + tid;
    const uint32_t key = p < nCand ? (cand_key(p) & 0xfffffu) : 0u;
    const bool gt = p < nCand && key > T;
    const bool eq = p < nCand && key == T;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      wgt[wv] = __popcll(bg);
      weq[wv] = __popcll(be);
    }
    __syncthreads();
    int og = run_gt, oe = run_eq, tg = 0, te = 0;
    for (int x = 0; x < kRowThreads / 64; ++x) {
      if (x < wv) {
        og += wgt[x];
        oe += weq[x];
      }
      tg += wgt[x];
      te += weq[x];
    }
    const int gb = og + lanes_below(bg), eb = oe + lanes_below(be);
    const int pc = gb + min(eb, need_eq);
    if ((gt || (eq && eb < need_eq)) && pc < need) Ch[pc] = cand_idx(p);
    run_gt += tg;
    run_eq += te;
    __syncthreads();
  }
  __syncthreads();
  return need;
}

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Merge the ascending lists S[0..nS) and Ch[0..nC) into out[0..k), -1 after.
__device__ void merge_to_output(const int32_t* S, int nS, const int32_t* Ch, int nC, int32_t* out,
                                int k) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nS; i += kRowThreads) {
    const int pos = i + lower_bound_i32(Ch, nC, S[i]);
    if (pos < k) out[pos] = S[i];
  }
  for (int i = tid; i < nC; i += kRowThreads) {
    const int pos = i + lower_bound_i32(S, nS, Ch[i]);
    if (pos < k) out[pos] = Ch[i];
  }
  for (int i = nS + nC + tid; i < k; i += kRowThreads) out[i] = -1;
}

constexpr int kMaxK = 4096;
constexpr int kMaxSeg = 1024;
constexpr int kCandLds = 8192;

// segment containing flat position p of a concatenation with exclusive
// prefix offsets off[0..n] (off[n] = total)
__device__ __forceinline__ int seg_of(const int* off, int n, int p) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One workgroup per row: gather the surely selected indices and the candidate
// (key, index) pairs of all segments into LDS with independent loads, radix-
// select the remaining `need` among the candidates on the low 20 key bits, and
// merge the two ascending lists into the row's output.
__global__ __launch_bounds__(kRowThreads) void topk_finish_kernel(
    int N_cap, int n_q, const int32_t* __restrict__ q_pos, int m, const int32_t* __restrict__ n_entries,
    int k, int n_seg, WideWs ws, int32_t* __restrict__ idx) {
  __shared__ int32_t S[kMaxK], Ch[kMaxK];
  __shared__ int seg_s[kMaxSeg + 1], seg_c[kMaxSeg + 1];
  __shared__ uint32_t hist[256];
  __shared__ int sh_bin, sh_above, sh_b2, sh_a2;
  __shared__ uint32_t wgt[kRowThreads / 64], weq[kRowThreads / 64];
  __shared__ uint32_t lh[kHistLdsWords];
  __shared__ int scan_sh[kRowThreads / 64];
  __shared__ uint32_t ck_s[kCandLds];
  __shared__ int32_t ci_s[kCandLds];
  const long long row = blockIdx.x;
  const int b = static_cast<int>(row / n_q);
  const int vis = visible_entries(q_pos[row], m, n_entries[b], N_cap);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* out = idx + row * k;
  row_threshold(ws.hist + row * kHistBins, lh, vis, k, &sh_bin, &sh_above, scan_sh);
  for (int s = tid; s < n_seg; s += kRowThreads) {
    seg_s[s] = ws.sure_cnt[row * n_seg + s];
    seg_c[s] = ws.cand_cnt[row * n_seg + s];
  }
  __syncthreads();
  if (wv == 0) {  // exclusive prefix sums, 64 segments a round
    int run_s = 0, run_c = 0;
    for (int base = 0; base < n_seg; base += 64) {
      const int s = base + lane;
      const int vs = s < n_seg ? seg_s[s] : 0, vc = s < n_seg ? seg_c[s] : 0;
      int is = vs, ic = vc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int ts = __shfl_up(is, o, 64), tc = __shfl_up(ic, o, 64);
        if (lane >= o) {
          is += ts;
          ic += tc;
        }
      }
      if (s < n_seg) {
        seg_s[s] = run_s + is - vs;
        seg_c[s] = run_c + ic - vc;
      }
      run_s += __shfl(is, 63, 64);
      run_c += __shfl(ic, 63, 64);
    }
    if (lane == 0) {
      seg_s[n_seg] = run_s;
      seg_c[n_seg] = run_c;
    }
  }
  __syncthreads();
  const int nS = min(seg_s[n_seg], k);
  const int nCand = seg_c[n_seg];
  const bool cand_in_lds = nCand <= kCandLds;
  // parallel gathers (ascending index order is the concatenation order)
  for (int p = tid; p < nS; p += kRowThreads) {
    const int s = seg_of(seg_s, n_seg, p);
    S[p] = ws.sure[(row * n_seg + s) * k + (p - seg_s[s])];
  }
  if (cand_in_lds) {
    for (int p = tid; p < nCand; p += kRowThreads) {
      const int s = seg_of(seg_c, n_seg, p);
      const long long off = (row * n_seg + s) * kSeg + (p - seg_c[s]);
      ck_s[p] = ws.cand_key[off];
      ci_s[p] = ws.cand_idx[off];
    }
  }
  __syncthreads();
  auto cand_key = [&](int p) -> uint32_t {
    if (cand_in_lds) return ck_s[p];
    const int s = seg_of(seg_c, n_seg, p);
    return ws.cand_key[(row * n_seg + s) * kSeg + (p - seg_c[s])];
  };
  auto cand_idx = [&](int p) -> int32_t {
    if (cand_in_lds) return ci_s[p];
    const int s = seg_of(seg_c, n_seg, p);
    return ws.cand_idx[(row * n_seg + s) * kSeg + (p - seg_c[s])];
  };
  const int need = vis <= k ? 0 : k - sh_above;
  const int nC = select_candidates(nCand, need, cand_key, cand_idx, Ch, hist, &sh_b2, &sh_a2, wgt, weq);
  merge_to_output(S, nS, Ch, nC, out, k);
}


// ---------------------------------------------------------------------------
// Workspace of the fused indexer selection (SelectWs; the selection itself
// runs inside the indexer).
constexpr int kMaxBlk = 8192;  // blocks per row (N_cap <= 1 Mi entries)

// ---------------------------------------------------------------------------
// Finish of the fused selection: one workgroup per row selects the row's top k
// from the pairs the row's workgroups emitted (every entry of the final top k
// is among them).  The row's final histogram gives the bin b* of the k-th
// largest key and the count of keys above it; every emitted entry above b* is
// selected, and the rest come from the entries in b* (the candidates; their
// number is the bin's count): a radix select on the low 20 key bits finds the
// key T of the last one taken, and when more candidates than needed carry T, a
// second radix select on the entry index takes the lowest ones.  The selected
// indices, in no order so far, are written out in ascending order through a
// bitmap over the row's visible entries (2^19 entries per pass).  Wave w reads
// the pairs of regions w, w + 16, ...; the histogram, the counts and the first
// 512 pairs of the wave's regions (up to 8 regions) do not depend on the row's
// length, so they are loaded at once with it: the common case takes one memory
// round trip before the selection.
constexpr int kFinWaves = 16;
constexpr int kFinThreads = kFinWaves * kWave;
constexpr int kFinSpec = 8;             // pairs per lane loaded with the counts
constexpr int kFinCand = 4096;          // candidates held in LDS (else in global memory)
constexpr int kFinBitmapWords = 16384;  // one output pass: 2^19 entries
constexpr uint32_t kSkipKey = 0x80000000u;

// exclusive block-wide prefix of one int per thread (NW full waves); *total is
// the sum over the block.  Ends with a barrier, so scan_sh can be reused.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* scan_sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) scan_sh[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    const int t = scan_sh[x];
    before += x < wave ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();
  return before + incl - v;
}

// Among the n elements whose key(e) lacks kSkipKey (keys of 20 bits), the
// want-th largest (1 <= want <= their number), by passes over bits 19..12,
// 11..4 and 3..0.  Returns the key prefix found and sets *mask to the bits it
// fixes: elements with (key & mask) > prefix are all taken, *gt of them, and
// *eq elements have (key & mask) == prefix, of which want - *gt are taken.
// The passes stop early once every element of the chosen digit is taken
// (*eq == want - *gt).
template <int NW, class KeyF>
__device__ uint32_t radix_select20(int n, int want, KeyF key, uint32_t* rh, int* sh_rb, int* sh_ra,
                                   uint32_t* mask_out, int* gt, int* eq) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int remaining = want, in_bin = 0;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 12 : (pass == 1 ? 4 : 0);
    const uint32_t dm = pass == 2 ? 0xfu : 0xffu;
    for (int i = tid; i < 256; i += NT) rh[i] = 0;
    if (tid == 0) {  // (set by the bin search; defined even if it found none)
      *sh_rb = 0;
      *sh_ra = 0;
    }
    __syncthreads();
    for (int e = tid; e < n; e += NT) {
      const uint32_t kk = key(e);
      if (!(kk & kSkipKey) && (kk & mask) == prefix) atomicAdd(&rh[(kk >> sh) & dm], 1u);
    }
    __syncthreads();
    if (tid < kWave) find_bin_wave(rh, 256, remaining, sh_rb, sh_ra);
    __syncthreads();
    const int bsel = *sh_rb;
    prefix |= static_cast<uint32_t>(bsel) << sh;
    mask |= dm << sh;
    remaining -= *sh_ra;
    in_bin = static_cast<int>(rh[bsel]);
    __syncthreads();
    if (in_bin == remaining) break;  // the same for every thread
  }
  *mask_out = mask;
  *gt = want - remaining;
  *eq = in_bin;
  return prefix;
}

// Workgroups rows .. rows + B - 1 (when app.tokC is set) run the decode step's
// state append of sequence blockIdx.x - rows instead, with the candidates' LDS
// as the pooling scratch.
__global__ __launch_bounds__(kFinThreads) void select_finish_kernel(
    int n_q, int N_cap, int wpr, const int32_t* __restrict__ q_pos, int m,
    const int32_t* __restrict__ n_entries, int k, SelectWs o, int32_t* __restrict__ sel_idx,
    long long rows, StateAppend app) {
  constexpr int NT = kFinThreads;
  __shared__ uint32_t lh[kHistLdsWords];
  __shared__ int32_t sel[kMaxK];
  __shared__ __attribute__((aligned(16))) uint32_t cand[2 * kFinCand];  // keys, indices
  // the output bitmap (one pass: 2^19 entries) and its counts per 128 entries
  __shared__ __attribute__((aligned(16))) uint32_t obm[kFinBitmapWords];
  __shared__ __attribute__((aligned(16))) uint32_t bcnt[kFinBitmapWords / 4];
  if (app.tokC && static_cast<long long>(blockIdx.x) >= rows) {
    constexpr int CPL = 512 / kWave;
    static_assert(sizeof(float) * kAppendWaves * 3 * CPL * kWave <= sizeof(obm), "append scratch");
    static_assert(kFinThreads >= kWave * kAppendWaves, "append waves");
    state_append_body<CPL, LCA_BF16, true>(static_cast<int>(blockIdx.x - rows), app.B,
                                     reinterpret_cast<float (*)[3][CPL][kWave]>(obm), 1, app.m, 512,
                                     app.n_win, app.tokC, app.tokZ, app.tailC, app.tailZ, app.ring,
                                     app.kv_fmt, app.P, app.cache, app.N_cap, app.n_tokens, nullptr,
                                     nullptr, app.eps, app.rope_step, app.pg, nullptr, 0);
    return;
  }
  __shared__ int sh_bin, sh_above, sh_nsel, sh_ncand, sh_rb, sh_ra;
  __shared__ int scan_sh[kFinWaves];
  __shared__ uint32_t rh[256];
  uint32_t* ck = cand;
  int32_t* ci = reinterpret_cast<int32_t*>(cand + kFinCand);
  const long long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint2* em = o.emit + static_cast<size_t>(row) * o.n_blk * kSelBlock;
  // the histogram words, and the counts and first pairs of the wave's regions
  // w, w + 16, ... (up to 8 of them; the 8 pair slots of a lane are shared
  // out, 64 pairs each, slots clamped to the region; every one of the wpr
  // regions exists, the row's length decides below which are used)
  const uint32_t* gh = o.hist + row * kScoreHistBins;
  constexpr int kHv = kScoreHistBins / NT;
  uint32_t hv[kHv];
#pragma unroll
  for (int u = 0; u < kHv; ++u) hv[u] = gh[tid + u * NT];
  const int spr_lg = wpr > 4 * kFinWaves ? 0 : (wpr > 2 * kFinWaves ? 1 : (wpr > kFinWaves ? 2 : 3));
  const int rpw = kFinSpec >> spr_lg;  // regions per wave read speculatively
  // region wi: blocks [wi a + min(wi, r), +a + (wi < r)) of the row (see select_region)
  const int ra = o.n_blk / wpr, rr = o.n_blk % wpr;
  auto region_first = [&](int wi) -> int { return (wi * ra + min(wi, rr)) * kSelBlock; };
  // lane l < 8 loads the count of the wave's region l (clamped to an existing
  // region; which regions are used is decided below)
  const int cnt_l = o.emit_cnt[row * o.n_blk + min(wave + kFinWaves * min(lane, kFinSpec - 1), wpr - 1)];
  uint2 pr[kFinSpec];
#pragma unroll
  for (int u = 0; u < kFinSpec; ++u) {
    const int sgc = min(wave + kFinWaves * (u >> spr_lg), wpr - 1), sl = u & ((1 << spr_lg) - 1);
    const int rb = region_first(sgc);
    const int capc = (ra + (sgc < rr ? 1 : 0)) * kSelBlock;
    pr[u] = em[rb + min(sl * kWave + lane, capc - 1)];
  }
  // the output bitmap and block counts start cleared (while the loads above
  // are in flight; ordered before their first use by the barrier below)
  for (int w = 4 * tid; w < kFinBitmapWords; w += 4 * NT)
    *reinterpret_cast<uint4*>(obm + w) = make_uint4(0u, 0u, 0u, 0u);
  for (int w = 4 * tid; w < kFinBitmapWords / 4; w += 4 * NT)
    *reinterpret_cast<uint4*>(bcnt + w) = make_uint4(0u, 0u, 0u, 0u);
  const int b = static_cast<int>(row / n_q);
  const int vis = visible_entries(q_pos[row], m, n_entries[b], N_cap);
  if (vis <= k) return;  // written by the indexer
  int32_t* out = sel_idx + row * k;
  // one output pass: every selected entry sets its bitmap bit and counts in
  // its 128-entry block as it is selected
  const bool inl = vis <= 32 * kFinBitmapWords;
  auto mark = [&](int32_t x) {
    if (inl) {
      atomicOr(&obm[x >> 5], 1u << (x & 31));
      atomicAdd(&bcnt[x >> 7], 1u);
    }
  };
  const int n_part = min(wpr, (vis + kSelBlock - 1) / kSelBlock);
#pragma unroll
  for (int u = 0; u < kHv; ++u) lh[hist_lds(hist_bin_of_slot(tid + u * NT))] = hv[u];
  if (o.clear_hist) {  // (after the words' own loads: their values were used just above)
    uint32_t* ghw = o.hist + row * kScoreHistBins;
#pragma unroll
    for (int u = 0; u < kHv; ++u) ghw[tid + u * NT] = 0u;
  }
  if (tid == 0) {
    sh_nsel = 0;
    sh_ncand = 0;
    sh_bin = 0;  // (set below; defined even if the histogram were short of k)
    sh_above = 0;
  }
  __syncthreads();
  // threshold bin b*: thread t sums bins [4095 - 4t - 3, 4095 - 4t]
  constexpr int per = kScoreHistBins / NT;
  const int topb = kScoreHistBins - 1 - per * tid;
  int local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) local += static_cast<int>(lh[hist_lds(topb - i)]);
  int total;
  int run = block_excl_scan<kFinWaves>(local, &total, scan_sh);
  if (run < k && run + local >= k) {
    for (int i = 0; i < per; ++i) {
      const int h = static_cast<int>(lh[hist_lds(topb - i)]);
      if (run + h >= k) {
        sh_bin = topb - i;
        sh_above = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  const int bstar = sh_bin, above = sh_above;
  const int C = static_cast<int>(lh[hist_lds(bstar)]);
  const int need = k - above;  // 1 <= need <= C
  const bool cand_lds = C <= kFinCand;
  uint32_t* gck = o.cand_key + row * N_cap;
  int32_t* gci = o.cand_idx + row * N_cap;
  const int cap = cand_lds ? kFinCand : N_cap;
  // above b* -> sel, in b* -> candidates; one LDS atomic per kind and wave per
  // kFinSpec * 64 pairs
  // (slot u of a lane holds a pair when lane < lim[u])
  auto classify = [&](const uint2* p, const int* lim) {
    uint64_t ms[kFinSpec], mc[kFinSpec];
    int ns = 0, nc = 0;
#pragma unroll
    for (int u = 0; u < kFinSpec; ++u) {
      const bool valid = lane < lim[u];
      const int bin = static_cast<int>(score_bin(p[u].x));
      ms[u] = __ballot(valid && bin > bstar);
      mc[u] = __ballot(valid && bin == bstar);
      ns += __popcll(ms[u]);
      nc += __popcll(mc[u]);
    }
    int bs = 0, bc = 0;
    if (lane == 0) {
      if (ns) bs = atomicAdd(&sh_nsel, ns);
      if (nc) bc = atomicAdd(&sh_ncand, nc);
    }
    bs = __shfl(bs, 0, kWave);
    bc = __shfl(bc, 0, kWave);
#pragma unroll
    for (int u = 0; u < kFinSpec; ++u) {
      if ((ms[u] >> lane) & 1) {
        const int q = bs + lanes_below(ms[u]);
        if (q < k) {
          sel[q] = static_cast<int32_t>(p[u].y);
          mark(static_cast<int32_t>(p[u].y));
        }
      }
      bs += __popcll(ms[u]);
      if ((mc[u] >> lane) & 1) {
        const int q = bc + lanes_below(mc[u]);
        if (q < cap) {
          if (cand_lds) {
            ck[q] = p[u].x;
            ci[q] = static_cast<int32_t>(p[u].y);
          } else {
            gck[q] = p[u].x;
            gci[q] = static_cast<int32_t>(p[u].y);
          }
        }
      }
      bc += __popcll(mc[u]);
    }
  };
  constexpr int kChunk = kFinSpec * kWave;
  int lim[kFinSpec];
#pragma unroll
  for (int u = 0; u < kFinSpec; ++u) {
    const int sg = wave + kFinWaves * (u >> spr_lg), sl = u & ((1 << spr_lg) - 1);
    const int cnt = __shfl(cnt_l, u >> spr_lg, kWave);
    lim[u] = sg < n_part ? cnt - sl * kWave : 0;
  }
  classify(pr, lim);
  // pairs of those regions past the slots they were given, then the regions
  // past the first 8 of the wave (the same for the whole wave)
  for (int j = 0; j < rpw; ++j) {
    const int sg = wave + kFinWaves * j;
    if (sg >= n_part) break;
    const int cnt = o.emit_cnt[row * o.n_blk + sg];
    const size_t rb = select_region(o.n_blk, wpr, sg);
    for (int c0 = kWave << spr_lg; c0 < cnt; c0 += kChunk) {
#pragma unroll
      for (int u = 0; u < kFinSpec; ++u) {
        pr[u] = em[rb + min(c0 + u * kWave + lane, cnt - 1)];
        lim[u] = cnt - c0 - u * kWave;
      }
      classify(pr, lim);
    }
  }
  for (int sg = wave + kFinWaves * rpw; sg < n_part; sg += kFinWaves) {
    const int cnt = o.emit_cnt[row * o.n_blk + sg];
    const size_t rb = select_region(o.n_blk, wpr, sg);
    for (int c0 = 0; c0 < cnt; c0 += kChunk) {
#pragma unroll
      for (int u = 0; u < kFinSpec; ++u) {
        pr[u] = em[rb + min(c0 + u * kWave + lane, cnt - 1)];
        lim[u] = cnt - c0 - u * kWave;
      }
      classify(pr, lim);
    }
  }
  __syncthreads();
  const int nC = min(sh_ncand, cap);
  auto ckey = [&](int e) -> uint32_t { return (cand_lds ? ck[e] : gck[e]) & 0xfffffu; };
  auto cidx = [&](int e) -> int32_t { return cand_lds ? ci[e] : gci[e]; };
  // the need largest candidates (low 20 key bits; ties to the lower index)
  uint32_t T = 0, tmask = 0;
  // candidates with (key & tmask) == T are taken when ((0xfffff - index) & xmask) >= X
  uint32_t X = 0, xmask = 0;
  if (need < nC) {
    int gt, eq;
    T = radix_select20<kFinWaves>(nC, need, ckey, rh, &sh_rb, &sh_ra, &tmask, &gt, &eq);
    const int need_eq = need - gt;
    if (eq > need_eq) {  // T is a whole key here: more candidates carry it than are taken
      auto inv_idx = [&](int e) -> uint32_t {
        return ckey(e) == T ? 0xfffffu - static_cast<uint32_t>(cidx(e)) : kSkipKey;
      };
      int gt2, eq2;
      X = radix_select20<kFinWaves>(nC, need_eq, inv_idx, rh, &sh_rb, &sh_ra, &xmask, &gt2, &eq2);
    }
  }
  for (int e0 = 0; e0 < nC; e0 += NT) {
    const int e = e0 + tid;
    bool take = false;
    int32_t id = 0;
    if (e < nC) {
      const uint32_t kk = ckey(e) & tmask;
      id = cidx(e);
      take = need >= nC || kk > T ||
             (kk == T && ((0xfffffu - static_cast<uint32_t>(id)) & xmask) >= X);
    }
    const uint64_t mt = __ballot(take);
    int bs = 0;
    if (lane == 0 && mt) bs = atomicAdd(&sh_nsel, __popcll(mt));
    bs = __shfl(bs, 0, kWave);
    if (take) {
      const int q = bs + lanes_below(mt);
      if (q < k) {
        sel[q] = id;
        mark(id);
      }
    }
  }
  __syncthreads();
  const int n_sel = min(sh_nsel, k);
  // ascending output through a bitmap over the visible entries (2^19 per pass)
  // and a count per 128-entry block: a selected entry's position is its
  // block's exclusive prefix plus the set bits below it in its block's four
  // words.  One pass (inl): bits and counts were set as entries were
  // selected; more passes (rows over 2^19 entries) set them pass by pass.
  int done = 0;
  uint32_t* bm = obm;
  for (int base = 0; base < vis; base += 32 * kFinBitmapWords) {
    const int nbits = min(32 * kFinBitmapWords, vis - base);
    const int nw = (nbits + 31) >> 5;
    const int nw4 = (nw + 3) & ~3;  // (<= kFinBitmapWords, a multiple of 4)
    const int nb = (nbits + 127) >> 7;
    if (!inl) {  // (the same for every thread)
      for (int w = 4 * tid; w < nw4; w += 4 * NT) *reinterpret_cast<uint4*>(bm + w) = make_uint4(0u, 0u, 0u, 0u);
      for (int i = tid; i < nb; i += NT) bcnt[i] = 0u;
      __syncthreads();
      for (int i = tid; i < n_sel; i += NT) {
        const int x = sel[i] - base;
        if (x >= 0 && x < nbits) {
          atomicOr(&bm[x >> 5], 1u << (x & 31));
          atomicAdd(&bcnt[x >> 7], 1u);
        }
      }
      __syncthreads();
    }
    // thread t: blocks [bpt t, bpt t + bpt), turned into exclusive prefixes
    const int bpt = (nb + NT - 1) / NT;
    int c = 0;
    for (int j = 0; j < bpt; ++j) {
      const int bb = bpt * tid + j;
      if (bb < nb) c += static_cast<int>(bcnt[bb]);
    }
    int tot;
    int at = done + block_excl_scan<kFinWaves>(c, &tot, scan_sh);
    for (int j = 0; j < bpt; ++j) {
      const int bb = bpt * tid + j;
      if (bb < nb) {
        const int v = static_cast<int>(bcnt[bb]);
        bcnt[bb] = static_cast<uint32_t>(at);
        at += v;
      }
    }
    __syncthreads();
    for (int i = tid; i < n_sel; i += NT) {
      const int x = sel[i] - base;
      if (x >= 0 && x < nbits) {
        const int wx = x >> 5;
        int pos = static_cast<int>(bcnt[x >> 7]) + __popc(bm[wx] & ((1u << (x & 31)) - 1u));
        for (int wy = wx & ~3; wy < wx; ++wy) pos += __popc(bm[wy]);
        if (pos < k) out[pos] = base + x;
      }
    }
    done += tot;
    if (base + 32 * kFinBitmapWords < vis) __syncthreads();  // the next pass clears the bitmap
  }
  for (int i = done + tid; i < k; i += NT) out[i] = -1;  // (none when the data is consistent)
}

struct SelectLayout {
  size_t hist, emit_cnt, emit, cand_key, cand_idx, total;
};

inline SelectLayout select_layout(long long rows, int N_cap) {
  SelectLayout L;
  const size_t r = static_cast<size_t>(rows), n = static_cast<size_t>(N_cap);
  const size_t nb = (n + kSelBlock - 1) / kSelBlock;
  size_t off = 0;
  L.hist = off;     off += align256(r * kHistBins * 4);
  L.emit_cnt = off; off += align256(r * nb * 4);
  L.emit = off;     off += align256(r * nb * kSelBlock * 8);
  L.cand_key = off; off += align256(r * n * 4);
  L.cand_idx = off; off += align256(r * n * 4);
  L.total = off;
  return L;
}
// Device checks of a finished selection (debug build): row r of idx holds
// min(k, vis) ascending visible entries, then -1.  One thread per element.
__global__ void dbg_selection_kernel(long long rows, int n_q, int N_cap, const int32_t* __restrict__ q_pos,
                                     int m, const int32_t* __restrict__ n_entries, int k,
                                     const int32_t* __restrict__ idx) {
  const long long gid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= rows * k) return;
  const long long row = gid / k;
  const int i = static_cast<int>(gid % k);
  const int vis = visible_entries(q_pos[row], m, n_entries[row / n_q], N_cap);
  const int v = idx[gid];
  if (i < (vis < k ? vis : k))
    dbg_check(v >= 0 && v < vis && (i == 0 || idx[gid - 1] < v));
  else
    dbg_check(v == -1);
}

hipError_t dbg_selection(long long rows, int n_q, int N_cap, const int32_t* q_pos, int m,
                         const int32_t* n_entries, int k, const int32_t* idx, hipStream_t s) {
  if constexpr (LCA_DEVICE_CHECKS) {
    const long long n = rows * k;
    if (n > 0)
      hipLaunchKernelGGL(dbg_selection_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                         rows, n_q, N_cap, q_pos, m, n_entries, k, idx);
  }
  return hipGetLastError();
}

}  // namespace

static int n_segments(int N_cap) { return (N_cap + kSeg - 1) / kSeg; }

long long topk_hist_words(long long rows) { return rows * kHistBins; }

uint32_t* topk_hist_in_workspace(void* ws, int B, int n_q, int N_cap, int k) {
  if (N_cap <= kLdsMaxRow || ws == nullptr) return nullptr;
  return wide_ws(ws, static_cast<long long>(B) * n_q, n_segments(N_cap), k).hist;
}

template <typename ST>
static hipError_t launch_collect_finish(long long rows, int N_cap, const ST* scores, int n_q,
                                        const int32_t* q_pos, int m, const int32_t* n_entries, int k,
                                        int32_t* idx, const WideWs& w, int n_seg, hipStream_t s) {
  const dim3 g2(static_cast<unsigned>(rows * n_seg));
  hipLaunchKernelGGL(topk_collect_kernel<ST>, g2, dim3(kSegThreads), 0, s, scores, N_cap, n_q, q_pos,
                     m, n_entries, k, n_seg, w);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(static_cast<unsigned>(rows)), dim3(kRowThreads), 0, s,
                     N_cap, n_q, q_pos, m, n_entries, k, n_seg, w, idx);
  return dbg_selection(rows, n_q, N_cap, q_pos, m, n_entries, k, idx, s);
}

hipError_t launch_topk_from_hist(int B, int n_q, int N_cap, const float* scores,
                                 const int32_t* q_pos, int m, const int32_t* n_entries, int k,
                                 int32_t* idx, void* ws, hipStream_t s) {
  const long long rows = static_cast<long long>(B) * n_q;
  if (rows == 0) return hipSuccess;
  if (N_cap <= kLdsMaxRow) return launch_topk(B, n_q, N_cap, scores, q_pos, m, n_entries, k, idx, ws, s);
  const int n_seg = n_segments(N_cap);
  if (n_seg > kMaxSeg || k > kMaxK) return hipErrorInvalidValue;
  return launch_collect_finish<float>(rows, N_cap, scores, n_q, q_pos, m, n_entries, k, idx,
                                      wide_ws(ws, rows, n_seg, k), n_seg, s);
}

size_t topk_workspace_bytes(int B, int n_q, int N_cap, int k) {
  if (N_cap <= kLdsMaxRow) return 0;
  return wide_layout(static_cast<long long>(B) * n_q, n_segments(N_cap), k).total;
}

template <typename ST>
static hipError_t launch_topk_t(int B, int n_q, int N_cap, const ST* scores, const int32_t* q_pos,
                                int m, const int32_t* n_entries, int k, int32_t* idx, void* ws,
                                hipStream_t s) {
  const long long rows = static_cast<long long>(B) * n_q;
  if (rows == 0) return hipSuccess;
  if (N_cap <= kLdsMaxRow) {
    const size_t lds = sizeof(uint32_t) * static_cast<size_t>(N_cap > 0 ? N_cap : 1);
    hipLaunchKernelGGL(topk_lds_kernel<ST>, dim3(static_cast<unsigned>(rows)), dim3(kRowThreads), lds,
                       s, scores, N_cap, n_q, q_pos, m, n_entries, k, idx);
    return dbg_selection(rows, n_q, N_cap, q_pos, m, n_entries, k, idx, s);
  }
  const int n_seg = n_segments(N_cap);
  if (n_seg > kMaxSeg || k > kMaxK) return hipErrorInvalidValue;
  WideWs w = wide_ws(ws, rows, n_seg, k);
  const long long nh = topk_hist_words(rows);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(static_cast<unsigned>((nh + 255) / 256)), dim3(256), 0, s,
                     w.hist, nh);
  const dim3 g2(static_cast<unsigned>(rows * n_seg));
  hipLaunchKernelGGL(topk_hist_kernel<ST>, g2, dim3(kSegThreads), 0, s, scores, N_cap, n_q, q_pos, m,
                     n_entries, k, n_seg, w.hist);
  return launch_collect_finish<ST>(rows, N_cap, scores, n_q, q_pos, m, n_entries, k, idx, w, n_seg, s);
}

hipError_t launch_topk(int B, int n_q, int N_cap, const void* scores, const int32_t* q_pos, int m,
                       const int32_t* n_entries, int k, int32_t* idx, void* ws, hipStream_t s,
                       int score_fmt) {
  if (score_fmt == LCA_BF16)
    return launch_topk_t<uint16_t>(B, n_q, N_cap, static_cast<const uint16_t*>(scores), q_pos, m,
                                   n_entries, k, idx, ws, s);
  if (score_fmt != LCA_F32) return hipErrorInvalidValue;
  return launch_topk_t<float>(B, n_q, N_cap, static_cast<const float*>(scores), q_pos, m, n_entries,
                              k, idx, ws, s);
}

bool select_supported(int N_cap, int k) {
  return N_cap > kLdsMaxRow && (N_cap + kSelBlock - 1) / kSelBlock <= kMaxBlk && k >= 1 && k <= kMaxK;
}

size_t select_workspace_bytes(long long rows, int N_cap) { return select_layout(rows, N_cap).total; }

long long select_zero_words(long long rows) { return rows * kHistBins; }

SelectWs select_ws_in(void* ws, long long rows, int N_cap) {
  const SelectLayout L = select_layout(rows, N_cap);
  char* p = static_cast<char*>(ws);
  SelectWs w{};
  w.hist = reinterpret_cast<uint32_t*>(p + L.hist);
  w.emit_cnt = reinterpret_cast<int32_t*>(p + L.emit_cnt);
  w.emit = reinterpret_cast<uint2*>(p + L.emit);
  w.cand_key = reinterpret_cast<uint32_t*>(p + L.cand_key);
  w.cand_idx = reinterpret_cast<int32_t*>(p + L.cand_idx);
  w.n_blk = (N_cap + kSelBlock - 1) / kSelBlock;
  return w;
}

hipError_t launch_select_finish(long long rows, int n_q, int N_cap, int wpr, const int32_t* q_pos, int m,
                                const int32_t* n_entries, int k, const SelectWs& w, int32_t* idx,
                                hipStream_t s, const StateAppend* app) {
  if (rows == 0) return hipSuccess;
  if (wpr < 1 || wpr > kSelMaxWpr || !select_supported(N_cap, k)) return hipErrorInvalidValue;
  if (app && (n_q != 1 || app->B != rows || app->tokC == nullptr)) return hipErrorInvalidValue;
  const StateAppend a = app ? *app : StateAppend{};
  const long long grid = rows + (app ? app->B : 0);
  hipLaunchKernelGGL(select_finish_kernel, dim3(static_cast<unsigned>(grid)), dim3(kFinThreads), 0, s,
                     n_q, N_cap, wpr, q_pos, m, n_entries, k, w, idx, rows, a);
  return dbg_selection(rows, n_q, N_cap, q_pos, m, n_entries, k, idx, s);
}

LCA_DBG_ACCESSOR(dbg_violations_topk)

}  // namespace lca
