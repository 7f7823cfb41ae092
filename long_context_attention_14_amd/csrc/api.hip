// C ABI of the CSA/HCA attention library: host-side validation, workspace
// sizing and dispatch to the kernels.  Validation runs before any HIP call, so
// a rejected call enqueues nothing; no entry point throws, aborts or prints.
#include <cmath>
#include <cstdio>
#include <cstdarg>
#include <mutex>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return LCA_OK;
  return fail(LCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool io_fmt_ok(int f) { return f == LCA_F32 || f == LCA_BF16; }
bool kv_fmt_ok(int f) { return f == LCA_F32 || f == LCA_BF16 || f == LCA_KV_FP8_BF16ROPE; }
// Partial RoPE base: 0 (off) or a finite base above 1; the kernels take
// base^(-2/64), the ratio of neighbouring pairs' frequencies.
bool rope_ok(float base) { return base == 0.f || (std::isfinite(base) && base > 1.f); }
double rope_step(float base) {
  return base == 0.f ? 0.0 : std::pow(static_cast<double>(base), -2.0 / lca::kRopeDims);
}

bool c_ok(int c) { return c >= 128 && c <= 1024 && c % 64 == 0 && (c / 64 == 2 || c / 64 == 4 || c / 64 == 8 || c / 64 == 16); }

#define REQUIRE(cond, ...)                                         \
  do {                                                             \
    if (!(cond)) return fail(LCA_ERR_INVALID_ARG, __VA_ARGS__);    \
  } while (0)

#define SUPPORT(cond, ...)                                         \
  do {                                                             \
    if (!(cond)) return fail(LCA_ERR_UNSUPPORTED, __VA_ARGS__);    \
  } while (0)

// The device view of an optional paged layout (NULL or no table: contiguous),
// checked against the entries per sequence it must hold.
int kv_pages(const lca_kv_pages* in, int m, int N_cap, lca::KvPages* out) {
  *out = lca::KvPages{nullptr, 0, 1, 0};
  if (in == nullptr || in->block_table == nullptr) return LCA_OK;
  REQUIRE(in->page_tokens >= 1 && m >= 1 && in->page_tokens % m == 0,
          "page_tokens = %d is not a positive multiple of m = %d", in->page_tokens, m);
  REQUIRE(in->max_pages >= 1 && in->n_pages >= 1, "max_pages and n_pages must be >= 1");
  const int epp = in->page_tokens / m;
  REQUIRE(static_cast<long long>(in->max_pages) * epp >= N_cap,
          "max_pages * entries per page = %lld < N_cap = %d",
          static_cast<long long>(in->max_pages) * epp, N_cap);
  *out = lca::KvPages{in->block_table, in->max_pages, epp, in->n_pages};
  return LCA_OK;
}

}  // namespace

extern "C" {

int lca_version(void) { return LCA_ABI_VERSION; }

const char* lca_status_string(int status) {
  switch (status) {
    case LCA_OK: return "ok";
    case LCA_ERR_INVALID_ARG: return "invalid argument";
    case LCA_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case LCA_ERR_WORKSPACE: return "workspace missing or too small";
    case LCA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* lca_last_error(void) { return g_last_error.c_str(); }

size_t lca_kv_row_bytes(int kv_dtype, int c) {
  if (!kv_fmt_ok(kv_dtype) || c <= 0) return 0;
  if (kv_dtype == LCA_KV_FP8_BF16ROPE && c < 64) return 0;
  return lca::row_bytes(kv_dtype, c);
}

int lca_compress(int mode, int m, int B, int n_new, int c, const void* C, const void* Z,
                 int io_dtype, const void* prevC, const void* prevZ, const float* P, void* cache,
                 int kv_dtype, int N_cap, int first_entry, float eps, float rope_base,
                 const lca_kv_pages* pages, lca_stream_t stream) {
  g_last_error.clear();
  lca::KvPages pg;
  if (int st = kv_pages(pages, m, N_cap, &pg)) return st;
  REQUIRE(rope_ok(rope_base), "rope_base = %g is neither 0 nor a finite value > 1", rope_base);
  REQUIRE(mode == LCA_CSA || mode == LCA_HCA, "mode %d is not LCA_CSA/LCA_HCA", mode);
  REQUIRE(m >= 1 && m <= 4096, "m = %d out of range [1, 4096]", m);
  REQUIRE(B >= 0 && n_new >= 0, "negative batch or token count");
  REQUIRE(n_new % m == 0, "n_new = %d is not a multiple of m = %d", n_new, m);
  SUPPORT(c_ok(c), "c = %d unsupported (need 128, 256, 512 or 1024)", c);
  SUPPORT(io_fmt_ok(io_dtype), "io_dtype %d unsupported (F32 or BF16)", io_dtype);
  SUPPORT(kv_fmt_ok(kv_dtype), "kv_dtype %d unsupported", kv_dtype);
  REQUIRE((prevC == nullptr) == (prevZ == nullptr), "prevC and prevZ must both be set or both NULL");
  REQUIRE(mode == LCA_CSA || prevC == nullptr, "prevC/prevZ only apply to CSA");
  REQUIRE(first_entry >= 0 && N_cap >= 0 && static_cast<long long>(first_entry) + n_new / m <= N_cap,
          "entries [%d, %d) exceed N_cap = %d", first_entry, first_entry + n_new / m, N_cap);
  if (B == 0 || n_new == 0) return LCA_OK;
  REQUIRE(C && Z && P && cache, "NULL tensor pointer");
  return hip_status(lca::launch_compress(mode, m, B, n_new, c, C, Z, io_dtype, prevC, prevZ, P, cache,
                                         kv_dtype, N_cap, first_entry, eps, rope_step(rope_base), pg,
                                         reinterpret_cast<hipStream_t>(stream)),
                    "lca_compress");
}

int lca_rmsnorm_rows(int B, int n, int c, const void* x, int x_dtype, void* y, int y_dtype,
                     int y_seq_rows, float eps, int64_t pos0, float rope_base,
                     lca_stream_t stream) {
  g_last_error.clear();
  REQUIRE(B >= 0 && n >= 0, "negative sizes");
  REQUIRE(rope_ok(rope_base), "rope_base = %g is neither 0 nor a finite value > 1", rope_base);
  REQUIRE(pos0 >= 0 && pos0 <= (INT64_C(1) << 40), "pos0 = %lld out of range",
          static_cast<long long>(pos0));
  SUPPORT(c_ok(c), "c = %d unsupported", c);
  SUPPORT(io_fmt_ok(x_dtype), "x_dtype %d unsupported", x_dtype);
  SUPPORT(kv_fmt_ok(y_dtype), "y_dtype %d unsupported", y_dtype);
  REQUIRE(y_seq_rows >= n, "y_seq_rows = %d < n = %d", y_seq_rows, n);
  if (B == 0 || n == 0) return LCA_OK;
  REQUIRE(x && y, "NULL tensor pointer");
  return hip_status(lca::launch_rmsnorm_rows(B, n, c, x, x_dtype, y, y_dtype, y_seq_rows, eps,
                                             static_cast<long long>(pos0), rope_step(rope_base),
                                             reinterpret_cast<hipStream_t>(stream)),
                    "lca_rmsnorm_rows");
}

static int indexer_scores(int B, int n_q, int H_I, int d_I, int idx_dtype, const void* qI,
                          const uint8_t* qI_scale, const void* kI, const uint8_t* kI_scale,
                          int N_cap, const float* w, const int32_t* q_pos, int m,
                          const int32_t* n_entries, void* scores, int score_fmt,
                          lca_stream_t stream, const char* name) {
  g_last_error.clear();
  REQUIRE(B >= 0 && n_q >= 0 && N_cap >= 0, "negative sizes");
  REQUIRE(m >= 1, "m = %d < 1", m);
  REQUIRE(H_I >= 1 && d_I >= 1, "H_I and d_I must be positive");
  if (idx_dtype == LCA_F32) {
    SUPPORT(H_I <= 64 && d_I <= 256 && d_I % 4 == 0, "F32 indexer needs H_I <= 64, d_I <= 256");
  } else if (idx_dtype == LCA_FP8_E4M3 || idx_dtype == LCA_MXFP4) {
    SUPPORT(H_I == 64 && d_I == 128, "FP8/MXFP4 indexer needs H_I == 64 and d_I == 128");
  } else {
    return fail(LCA_ERR_UNSUPPORTED, "idx_dtype %d unsupported", idx_dtype);
  }
  if (idx_dtype == LCA_MXFP4)
    REQUIRE(qI_scale && kI_scale, "MXFP4 needs qI_scale and kI_scale");
  if (B == 0 || n_q == 0 || N_cap == 0) return LCA_OK;
  REQUIRE(qI && kI && w && q_pos && n_entries && scores, "NULL tensor pointer");
  return hip_status(lca::launch_indexer(B, n_q, H_I, d_I, idx_dtype, qI, qI_scale, kI, kI_scale,
                                        N_cap, w, q_pos, m, n_entries, scores,
                                        reinterpret_cast<hipStream_t>(stream), nullptr, nullptr,
                                        nullptr, nullptr, 0, score_fmt),
                    name);
}

int lca_indexer_scores(int B, int n_q, int H_I, int d_I, int idx_dtype, const void* qI,
                       const uint8_t* qI_scale, const void* kI, const uint8_t* kI_scale, int N_cap,
                       const float* w, const int32_t* q_pos, int m, const int32_t* n_entries,
                       float* scores, lca_stream_t stream) {
  return indexer_scores(B, n_q, H_I, d_I, idx_dtype, qI, qI_scale, kI, kI_scale, N_cap, w, q_pos, m,
                        n_entries, scores, LCA_F32, stream, "lca_indexer_scores");
}

int lca_indexer_scores_bf16(int B, int n_q, int H_I, int d_I, int idx_dtype, const void* qI,
                            const uint8_t* qI_scale, const void* kI, const uint8_t* kI_scale,
                            int N_cap, const float* w, const int32_t* q_pos, int m,
                            const int32_t* n_entries, uint16_t* scores, lca_stream_t stream) {
  return indexer_scores(B, n_q, H_I, d_I, idx_dtype, qI, qI_scale, kI, kI_scale, N_cap, w, q_pos, m,
                        n_entries, scores, LCA_BF16, stream, "lca_indexer_scores_bf16");
}

size_t lca_topk_workspace_size(int B, int n_q, int N_cap, int k) {
  if (B < 0 || n_q < 0 || N_cap < 0 || k < 1 || k > 4096) return 0;
  return lca::topk_workspace_bytes(B, n_q, N_cap, k);
}

static int topk(int B, int n_q, int N_cap, const void* scores, int score_fmt, const int32_t* q_pos,
                int m, const int32_t* n_entries, int k, int32_t* idx, void* workspace,
                size_t workspace_bytes, lca_stream_t stream, const char* name) {
  g_last_error.clear();
  REQUIRE(B >= 0 && n_q >= 0 && N_cap >= 0, "negative sizes");
  REQUIRE(k >= 1 && k <= 4096, "k = %d out of range [1, 4096]", k);
  REQUIRE(m >= 1, "m = %d < 1", m);
  SUPPORT(N_cap <= (1 << 23), "N_cap = %d too large", N_cap);
  const size_t need = lca::topk_workspace_bytes(B, n_q, N_cap, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", name, need,
                workspace ? workspace_bytes : 0);
  if (B == 0 || n_q == 0) return LCA_OK;
  REQUIRE(scores && q_pos && n_entries && idx, "NULL tensor pointer");
  return hip_status(lca::launch_topk(B, n_q, N_cap, scores, q_pos, m, n_entries, k, idx, workspace,
                                     reinterpret_cast<hipStream_t>(stream), score_fmt),
                    name);
}

int lca_topk(int B, int n_q, int N_cap, const float* scores, const int32_t* q_pos, int m,
             const int32_t* n_entries, int k, int32_t* idx, void* workspace, size_t workspace_bytes,
             lca_stream_t stream) {
  return topk(B, n_q, N_cap, scores, LCA_F32, q_pos, m, n_entries, k, idx, workspace,
              workspace_bytes, stream, "lca_topk");
}

int lca_topk_bf16(int B, int n_q, int N_cap, const uint16_t* scores, const int32_t* q_pos, int m,
                  const int32_t* n_entries, int k, int32_t* idx, void* workspace,
                  size_t workspace_bytes, lca_stream_t stream) {
  return topk(B, n_q, N_cap, scores, LCA_BF16, q_pos, m, n_entries, k, idx, workspace,
              workspace_bytes, stream, "lca_topk_bf16");
}

size_t lca_sparse_mqa_workspace_size(int B, int n_q, int H, int c, int kv_dtype, int k, int N_cap,
                                     int n_win, int dense) {
  if (B < 0 || n_q < 0 || H < 1 || !c_ok(c) || N_cap < 0 || n_win < 0 || k < 0) return 0;
  return lca::mqa_workspace_bytes(B, n_q, H, c, kv_dtype, k, N_cap, n_win, dense);
}

int lca_sparse_mqa(int B, int n_q, int H, int c, const void* q, int q_dtype, const void* cache,
                   int kv_dtype, int N_cap, const int32_t* idx, int k, const int32_t* q_pos, int m,
                   const int32_t* n_entries, const void* win, int W_cap, int64_t win_origin,
                   int n_win, float tau, float eps, const float* sink, float rope_base, void* out,
                   int out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                   const lca_kv_pages* pages, lca_stream_t stream) {
  g_last_error.clear();
  lca::KvPages pg;
  REQUIRE(m >= 1, "m = %d < 1", m);
  if (int st = kv_pages(pages, m, N_cap, &pg)) return st;
  REQUIRE(rope_ok(rope_base), "rope_base = %g is neither 0 nor a finite value > 1", rope_base);
  REQUIRE(B >= 0 && n_q >= 0 && N_cap >= 0, "negative sizes");
  REQUIRE(m >= 1, "m = %d < 1", m);
  SUPPORT(c == 128 || c == 256 || c == 512, "c = %d unsupported (128, 256 or 512)", c);
  SUPPORT(H >= 8 && H % 8 == 0, "H = %d unsupported (multiple of 8)", H);
  SUPPORT(io_fmt_ok(q_dtype) && io_fmt_ok(out_dtype), "q/out dtype unsupported (F32 or BF16)");
  SUPPORT(kv_fmt_ok(kv_dtype), "kv_dtype %d unsupported", kv_dtype);
  REQUIRE(idx == nullptr || (k >= 1 && k <= 4096), "k = %d out of range", k);
  REQUIRE(n_win >= 0 && n_win <= 4096, "n_win = %d out of range", n_win);
  REQUIRE(n_win == 0 || (win != nullptr && W_cap >= 1), "window buffer missing");
  const int dense = idx == nullptr;
  const size_t need = lca::mqa_workspace_bytes(B, n_q, H, c, kv_dtype, k, N_cap, n_win, dense);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "lca_sparse_mqa needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : 0);
  if (B == 0 || n_q == 0) return LCA_OK;
  REQUIRE(q && cache && q_pos && n_entries && out, "NULL tensor pointer");
  return hip_status(lca::launch_mqa(B, n_q, H, c, q, q_dtype, cache, kv_dtype, N_cap, idx, k, q_pos,
                                    m, n_entries, win, W_cap, win_origin, n_win, tau, eps, sink,
                                    rope_step(rope_base), out, out_dtype, lse, workspace, pg,
                                    reinterpret_cast<hipStream_t>(stream)),
                    "lca_sparse_mqa");
}

int lca_state_append(int mode, int m, int B, int c, int n_win, const void* tokC, const void* tokZ,
                     int io_dtype, void* tailC, void* tailZ, void* ring, int kv_dtype,
                     const float* P, void* cache, int N_cap, int32_t* n_tokens, int32_t* q_pos,
                     int32_t* n_entries, float eps, float rope_base, const lca_kv_pages* pages,
                     lca_stream_t stream) {
  g_last_error.clear();
  REQUIRE(mode == LCA_CSA || mode == LCA_HCA, "mode %d is not LCA_CSA/LCA_HCA", mode);
  REQUIRE(m >= 1 && m <= 4096, "m = %d out of range", m);
  lca::KvPages pg;
  if (int st = kv_pages(pages, m, N_cap, &pg)) return st;
  REQUIRE(rope_ok(rope_base), "rope_base = %g is neither 0 nor a finite value > 1", rope_base);
  REQUIRE(B >= 0 && N_cap >= 0, "negative sizes");
  REQUIRE(n_win >= 1, "n_win = %d < 1", n_win);
  SUPPORT(c_ok(c), "c = %d unsupported", c);
  SUPPORT(io_fmt_ok(io_dtype), "io_dtype %d unsupported", io_dtype);
  SUPPORT(kv_fmt_ok(kv_dtype), "kv_dtype %d unsupported", kv_dtype);
  if (B == 0) return LCA_OK;
  REQUIRE(tokC && tokZ && tailC && tailZ && ring && P && cache && n_tokens && q_pos && n_entries,
          "NULL tensor pointer");
  return hip_status(lca::launch_state_append(mode, m, B, c, n_win, tokC, tokZ, io_dtype, tailC,
                                             tailZ, ring, kv_dtype, P, cache, N_cap, n_tokens,
                                             q_pos, n_entries, eps, rope_step(rope_base), pg,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "lca_state_append");
}

// ---------------------------------------------------------------------------
// grouped output projection

namespace {
int out_proj_check(int T, int n_h, int c, int g, int d_g, int d) {
  REQUIRE(T >= 0, "T = %d < 0", T);
  REQUIRE(n_h >= 1 && c >= 1 && g >= 1 && d_g >= 1 && d >= 1, "sizes must be positive");
  REQUIRE(n_h % g == 0, "n_h = %d is not a multiple of g = %d", n_h, g);
  SUPPORT(d_g % 128 == 0 && d % 128 == 0, "d_g = %d and d = %d must be multiples of 128", d_g, d);
  SUPPORT((n_h / g) * c % 64 == 0, "a group's input (n_h/g)*c = %d must be a multiple of 64",
          (n_h / g) * c);
  SUPPORT(static_cast<long long>(T) * n_h * c < (1LL << 31) &&
              static_cast<long long>(d) * g * d_g < (1LL << 31),
          "tensor too large");
  return LCA_OK;
}
}  // namespace

size_t lca_grouped_out_proj_workspace_size(int T, int n_h, int c, int g, int d_g, int d) {
  if (out_proj_check(T, n_h, c, g, d_g, d) != LCA_OK) return 0;
  return lca::out_proj_workspace_bytes(T, n_h, c, g, d_g, d);
}

int lca_grouped_out_proj(int T, int n_h, int c, int g, int d_g, int d, const uint16_t* o,
                         const uint16_t* W_g, const uint16_t* W_o, uint16_t* z, void* out,
                         int out_dtype, void* workspace, size_t workspace_bytes,
                         lca_stream_t stream) {
  g_last_error.clear();
  if (int st = out_proj_check(T, n_h, c, g, d_g, d)) return st;
  SUPPORT(io_fmt_ok(out_dtype), "out_dtype %d unsupported (F32 or BF16)", out_dtype);
  const size_t need = lca::out_proj_workspace_bytes(T, n_h, c, g, d_g, d);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(LCA_ERR_WORKSPACE, "lca_grouped_out_proj needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : 0);
  if (T == 0) return LCA_OK;
  REQUIRE(o && W_g && W_o && z && out, "NULL tensor pointer");
  return hip_status(lca::launch_out_proj(T, n_h, c, g, d_g, d, o, W_g, W_o, z, out, out_dtype,
                                         workspace, reinterpret_cast<hipStream_t>(stream)),
                    "lca_grouped_out_proj");
}

// ---------------------------------------------------------------------------
// composed decode step

namespace {

struct DecodeLayout {
  size_t q_pos, n_entries, scores, idx, topk, mqa, total;
};

size_t al(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// A CSA layer with an MFMA indexer format on rows too long for the LDS top-k
// fuses the top-k into the indexer (no score array): see SelectWs.
bool fused_select(const lca_decode_layer* L) {
  return L->mode == LCA_CSA && L->idx_dtype != LCA_F32 && lca::select_supported(L->N_cap, L->k);
}

DecodeLayout decode_layout(const lca_decode_layer* L) {
  DecodeLayout d;
  const size_t B = static_cast<size_t>(L->B);
  const bool csa = L->mode == LCA_CSA;
  const bool fused = fused_select(L);
  size_t off = 0;
  d.q_pos = off; off += al(B * 4);
  d.n_entries = off; off += al(B * 4);
  d.scores = off; off += csa && !fused ? al(B * static_cast<size_t>(L->N_cap) * 4) : 0;
  d.idx = off; off += csa ? al(B * static_cast<size_t>(L->k) * 4) : 0;
  d.topk = off;
  if (fused) off += al(lca::select_workspace_bytes(L->B, L->N_cap));
  else if (csa) off += al(lca::topk_workspace_bytes(L->B, 1, L->N_cap, L->k));
  d.mqa = off;
  off += al(lca::mqa_workspace_bytes(L->B, 1, L->H, L->c, L->kv_dtype, csa ? L->k : 0, L->N_cap,
                                     L->n_win, csa ? 0 : 1));
  d.total = off;
  return d;
}

int check_layer(const lca_decode_layer* L) {
  REQUIRE(L != nullptr, "NULL layer");
  REQUIRE(L->struct_size == sizeof(lca_decode_layer), "layer struct_size %zu != %zu",
          L->struct_size, sizeof(lca_decode_layer));
  REQUIRE(L->mode == LCA_CSA || L->mode == LCA_HCA, "bad mode");
  REQUIRE(L->B >= 0 && L->N_cap >= 1 && L->m >= 1, "bad sizes");
  if (L->mode == LCA_CSA) REQUIRE(L->k >= 1 && L->k <= 4096, "k = %d out of range", L->k);
  REQUIRE(rope_ok(L->rope_base), "rope_base = %g is neither 0 nor a finite value > 1", L->rope_base);
  lca::KvPages pg;
  return kv_pages(&L->pages, L->m, L->N_cap, &pg);
}

}  // namespace

size_t lca_decode_workspace_size(const lca_decode_layer* layer) {
  if (check_layer(layer) != LCA_OK) return 0;
  return decode_layout(layer).total;
}

}  // extern "C"

namespace {

// The structs of one decode step.
int decode_check_structs(const lca_decode_layer* L, const lca_decode_io* io) {
  const int st = check_layer(L);
  if (st != LCA_OK) return st;
  REQUIRE(io != nullptr && io->struct_size == sizeof(lca_decode_io), "bad io struct");
  return LCA_OK;
}

// The shapes, formats and tensors of one decode step (structs already checked).
int decode_check_args(const lca_decode_layer* L, const lca_decode_io* io) {
  if (L->B == 0) return LCA_OK;
  const bool csa = L->mode == LCA_CSA;
  SUPPORT(c_ok(L->c) && L->c <= 512, "c = %d unsupported", L->c);
  SUPPORT(io_fmt_ok(L->io_dtype) && kv_fmt_ok(L->kv_dtype) && io_fmt_ok(io->out_dtype),
          "dtype unsupported");
  SUPPORT(L->H >= 8 && L->H % 8 == 0, "H = %d unsupported", L->H);
  REQUIRE(L->n_win >= 1, "n_win must be >= 1");
  if (csa) {
    if (L->idx_dtype == LCA_F32)
      SUPPORT(L->H_I <= 64 && L->d_I <= 256 && L->d_I % 4 == 0, "F32 indexer shape unsupported");
    else
      SUPPORT((L->idx_dtype == LCA_FP8_E4M3 || L->idx_dtype == LCA_MXFP4) && L->H_I == 64 &&
                  L->d_I == 128,
              "indexer dtype/shape unsupported");
    REQUIRE(L->kI && io->qI && io->w, "CSA needs kI, qI and w");
    if (L->idx_dtype == LCA_MXFP4) REQUIRE(L->kI_scale && io->qI_scale, "MXFP4 needs scales");
  }
  REQUIRE(io->tokC && io->tokZ && io->q && io->out, "NULL io tensor");
  return LCA_OK;
}

// Every check of one decode step, before anything is enqueued.
int decode_check(const lca_decode_layer* L, const lca_decode_io* io, const void* workspace,
                 size_t workspace_bytes) {
  const int st = decode_check_structs(L, io);
  if (st != LCA_OK) return st;
  const DecodeLayout d = decode_layout(L);
  if (workspace == nullptr || workspace_bytes < d.total)
    return fail(LCA_ERR_WORKSPACE, "lca_decode_step needs %zu workspace bytes, got %zu", d.total,
                workspace ? workspace_bytes : 0);
  return decode_check_args(L, io);
}

// The launches of one decode step (decode_check passed, B > 0).
int decode_enqueue(const lca_decode_layer* L, const lca_decode_io* io, void* workspace,
                   lca_stream_t stream) {
  int st = LCA_OK;
  const DecodeLayout d = decode_layout(L);
  lca::KvPages pg;
  kv_pages(&L->pages, L->m, L->N_cap, &pg);
  char* ws = static_cast<char*>(workspace);
  int32_t* q_pos = reinterpret_cast<int32_t*>(ws + d.q_pos);
  int32_t* n_ent = reinterpret_cast<int32_t*>(ws + d.n_entries);
  const bool csa = L->mode == LCA_CSA;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> int {
    if (io->stage_events[i] == nullptr) return LCA_OK;
    return hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(io->stage_events[i]), s),
                      "lca_decode_step/event");
  };
  // Long CSA rows: either the fused selection (the indexer keeps its scores on
  // chip and emits a superset of the top k; a finish pass selects) or the
  // histogram path (the indexer writes scores and accumulates the top-k's row
  // histogram).  Either way the append clears the histogram as a side job.
  const bool fused = fused_select(L);
  lca::SelectWs sw{};
  uint32_t* hist = nullptr;
  long long zero_words = 0;
  if (fused) {
    sw = lca::select_ws_in(ws + d.topk, L->B, L->N_cap);
    hist = sw.hist;
    zero_words = lca::select_zero_words(L->B);
  } else if (csa && L->idx_dtype != LCA_F32) {
    hist = lca::topk_hist_in_workspace(ws + d.topk, L->B, 1, L->N_cap, L->k);
    zero_words = hist ? lca::topk_hist_words(L->B) : 0;
  }
  if ((st = mark(0)) != LCA_OK) return st;
  st = hip_status(lca::launch_state_append(L->mode, L->m, L->B, L->c, L->n_win, io->tokC, io->tokZ,
                                           L->io_dtype, L->tailC, L->tailZ, L->ring, L->kv_dtype,
                                           L->P, L->cache, L->N_cap, L->n_tokens, q_pos, n_ent,
                                           L->eps, rope_step(L->rope_base), pg, s, hist, zero_words),
                  "lca_decode_step/append");
  if (st != LCA_OK) return st;
  const int32_t* sel = nullptr;
  if (csa) {
    float* scores = fused ? nullptr : reinterpret_cast<float*>(ws + d.scores);
    int32_t* idx = io->idx_out ? io->idx_out : reinterpret_cast<int32_t*>(ws + d.idx);
    // events 1 and 2 are the indexer dispatch's own start and end stamps
    st = hip_status(lca::launch_indexer(L->B, 1, L->H_I, L->d_I, L->idx_dtype, io->qI, io->qI_scale,
                                        L->kI, L->kI_scale, L->N_cap, io->w, q_pos, L->m, n_ent,
                                        scores, s, fused ? nullptr : hist,
                                        reinterpret_cast<hipEvent_t>(io->stage_events[1]),
                                        reinterpret_cast<hipEvent_t>(io->stage_events[2]),
                                        fused ? &sw : nullptr, L->k, LCA_F32,
                                        fused ? idx : nullptr),
                    "lca_decode_step/indexer");
    if (st != LCA_OK) return st;
    if (fused) {
      // the indexer launch includes the finish pass
    } else if (hist)
      st = hip_status(lca::launch_topk_from_hist(L->B, 1, L->N_cap, scores, q_pos, L->m, n_ent, L->k,
                                                 idx, ws + d.topk, s),
                      "lca_decode_step/topk");
    else
      st = hip_status(lca::launch_topk(L->B, 1, L->N_cap, scores, q_pos, L->m, n_ent, L->k, idx,
                                       ws + d.topk, s),
                      "lca_decode_step/topk");
    if (st != LCA_OK) return st;
    if ((st = mark(3)) != LCA_OK) return st;
    sel = idx;
  } else {
    if ((st = mark(1)) != LCA_OK) return st;
    if ((st = mark(2)) != LCA_OK) return st;
    if ((st = mark(3)) != LCA_OK) return st;
  }
  st = hip_status(lca::launch_mqa(L->B, 1, L->H, L->c, io->q, L->io_dtype, L->cache, L->kv_dtype,
                                  L->N_cap, sel, csa ? L->k : 0, q_pos, L->m, n_ent, L->ring,
                                  L->n_win, 0, L->n_win, L->tau, L->eps, L->sink,
                                  rope_step(L->rope_base), io->out, io->out_dtype, io->lse,
                                  ws + d.mqa, pg, s),
                  "lca_decode_step/mqa");
  if (st != LCA_OK) return st;
  return mark(4);
}

}  // namespace

extern "C" {

int lca_decode_step(const lca_decode_layer* L, const lca_decode_io* io, void* workspace,
                    size_t workspace_bytes, lca_stream_t stream) {
  g_last_error.clear();
  const int st = decode_check(L, io, workspace, workspace_bytes);
  if (st != LCA_OK || L->B == 0) return st;
  return decode_enqueue(L, io, workspace, stream);
}

int lca_decode_steps(const lca_decode_layer* L, const lca_decode_io* io, int n_steps,
                     void* workspace, size_t workspace_bytes, lca_stream_t stream) {
  g_last_error.clear();
  REQUIRE(n_steps >= 0, "n_steps = %d < 0", n_steps);
  REQUIRE(n_steps == 0 || io != nullptr, "NULL io array");
  for (int i = 0; i < n_steps; ++i) {
    const int st = decode_check(L, io + i, workspace, workspace_bytes);
    if (st != LCA_OK) {
      g_last_error = "step " + std::to_string(i) + ": " + g_last_error;
      return st;
    }
  }
  if (n_steps == 0 || L->B == 0) return LCA_OK;
  for (int i = 0; i < n_steps; ++i) {
    const int st = decode_enqueue(L, io + i, workspace, stream);
    if (st != LCA_OK) return st;
  }
  return LCA_OK;
}


}  // extern "C"

// ---------------------------------------------------------------------------
// lca_decode_step_static: the decode step's scratch space in a device array the
// library owns, for callers that cannot allocate.  The array is a file-scope
// __device__ variable: the loader gives every device that runs the library its
// own copy, held until the process ends.  In host code its name is only a
// host-side stand-in, so its device address is asked for once per device (with
// that device current) and kept; kernels only ever see that address.

static __device__ __align__(256) unsigned char scratch[LCA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxStaticDevices = 64;

struct StaticScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};

StaticScratch g_static_scratch[kMaxStaticDevices];

// The current device's copy of `scratch` (its address asked for on the first
// call on that device; std::call_once makes concurrent first calls safe).
int static_scratch_ptr(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "lca_decode_step_static/hipGetDevice");
  if (dev < 0 || dev >= kMaxStaticDevices)
    return fail(LCA_ERR_UNSUPPORTED, "lca_decode_step_static: device %d beyond the %d supported",
                dev, kMaxStaticDevices);
  StaticScratch& sc = g_static_scratch[dev];
  std::call_once(sc.once, [&sc] {
    sc.err = hipGetSymbolAddress(&sc.ptr, HIP_SYMBOL(scratch));
    if (sc.err == hipSuccess && sc.ptr == nullptr) sc.err = hipErrorInvalidSymbol;
  });
  if (sc.err != hipSuccess) return hip_status(sc.err, "lca_decode_step_static/hipGetSymbolAddress");
  *out = sc.ptr;
  return LCA_OK;
}

}  // namespace

extern "C" {

int lca_decode_step_static(const lca_decode_layer* L, const lca_decode_io* io, lca_stream_t stream) {
  g_last_error.clear();
  int st = decode_check_structs(L, io);
  if (st != LCA_OK) return st;
  const size_t need = decode_layout(L).total;
  if (need > LCA_STATIC_SCRATCH_BYTES)
    return fail(LCA_ERR_WORKSPACE,
                "lca_decode_step_static: this layer needs %zu scratch bytes, more than the %zu of the "
                "library's static scratch (use lca_decode_step with a workspace)",
                need, static_cast<size_t>(LCA_STATIC_SCRATCH_BYTES));
  if ((st = decode_check_args(L, io)) != LCA_OK) return st;
  if (L->B == 0) return LCA_OK;
  void* ws = nullptr;
  if ((st = static_scratch_ptr(&ws)) != LCA_OK) return st;
  return decode_enqueue(L, io, ws, stream);
}

}  // extern "C"
