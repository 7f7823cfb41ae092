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

// A fixed split length for the attention: 0 (the automatic plan) or a positive
// multiple of 64 that leaves at most 256 splits per query.
int split_rows_ok(int split_rows, int k, int N_cap, int n_win, int dense) {
  if (split_rows == 0) return LCA_OK;
  REQUIRE(split_rows > 0 && split_rows % 64 == 0, "split_rows = %d is not 0 or a positive multiple of 64",
          split_rows);
  SUPPORT(lca::mqa_splits(k, N_cap, n_win, dense, split_rows) <= lca::kMaxSplits,
          "split_rows = %d gives more than %d splits per query", split_rows, lca::kMaxSplits);
  return LCA_OK;
}

// Every args struct starts with its own size: NULL or another layout is rejected.
#define CHECK_ARGS(a, T)                                                              \
  do {                                                                                \
    if ((a) == nullptr) return fail(LCA_ERR_INVALID_ARG, #T ": NULL argument struct"); \
    if ((a)->struct_size != sizeof(T))                                                \
      return fail(LCA_ERR_INVALID_ARG, #T ".struct_size = %zu, this library's is %zu", \
                  (a)->struct_size, sizeof(T));                                       \
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

int lca_compress(const lca_compress_args* a, lca_stream_t stream) {
  g_last_error.clear();
  CHECK_ARGS(a, lca_compress_args);
  lca::KvPages pg;
  if (int st = kv_pages(&a->pages, a->m, a->N_cap, &pg)) return st;
  REQUIRE(rope_ok(a->rope_base), "rope_base = %g is neither 0 nor a finite value > 1", a->rope_base);
  REQUIRE(a->mode == LCA_CSA || a->mode == LCA_HCA, "mode %d is not LCA_CSA/LCA_HCA", a->mode);
  REQUIRE(a->m >= 1 && a->m <= 4096, "m = %d out of range [1, 4096]", a->m);
  REQUIRE(a->B >= 0 && a->n_new >= 0, "negative batch or token count");
  REQUIRE(a->n_new % a->m == 0, "n_new = %d is not a multiple of m = %d", a->n_new, a->m);
  SUPPORT(c_ok(a->c), "c = %d unsupported (need 128, 256, 512 or 1024)", a->c);
  SUPPORT(io_fmt_ok(a->io_dtype), "io_dtype %d unsupported (F32 or BF16)", a->io_dtype);
  SUPPORT(kv_fmt_ok(a->kv_dtype), "kv_dtype %d unsupported", a->kv_dtype);
  REQUIRE((a->prevC == nullptr) == (a->prevZ == nullptr), "prevC and prevZ must both be set or both NULL");
  REQUIRE(a->mode == LCA_CSA || a->prevC == nullptr, "prevC/prevZ only apply to CSA");
  REQUIRE(a->first_entry >= 0 && a->N_cap >= 0 &&
              static_cast<long long>(a->first_entry) + a->n_new / a->m <= a->N_cap,
          "entries [%d, %d) exceed N_cap = %d", a->first_entry, a->first_entry + a->n_new / a->m, a->N_cap);
  REQUIRE(static_cast<long long>(a->B) * (a->n_new / a->m) <= 0x7fffffffLL, "too many entries");
  if (a->B == 0 || a->n_new == 0) return LCA_OK;
  REQUIRE(a->C && a->Z && a->P && a->cache, "NULL tensor pointer");
  return hip_status(lca::launch_compress(a->mode, a->m, a->B, a->n_new, a->c, a->C, a->Z, a->io_dtype,
                                         a->prevC, a->prevZ, a->P, a->cache, a->kv_dtype, a->N_cap,
                                         a->first_entry, a->eps, rope_step(a->rope_base), pg,
                                         reinterpret_cast<hipStream_t>(stream)),
                    "lca_compress");
}

int lca_rmsnorm_rows(const lca_rmsnorm_rows_args* a, lca_stream_t stream) {
  g_last_error.clear();
  CHECK_ARGS(a, lca_rmsnorm_rows_args);
  REQUIRE(a->B >= 0 && a->n >= 0, "negative sizes");
  REQUIRE(rope_ok(a->rope_base), "rope_base = %g is neither 0 nor a finite value > 1", a->rope_base);
  REQUIRE(a->pos0 >= 0 && a->pos0 <= (INT64_C(1) << 40), "pos0 = %lld out of range",
          static_cast<long long>(a->pos0));
  SUPPORT(c_ok(a->c), "c = %d unsupported", a->c);
  SUPPORT(io_fmt_ok(a->x_dtype), "x_dtype %d unsupported", a->x_dtype);
  SUPPORT(kv_fmt_ok(a->y_dtype), "y_dtype %d unsupported", a->y_dtype);
  REQUIRE(a->y_seq_rows >= a->n, "y_seq_rows = %d < n = %d", a->y_seq_rows, a->n);
  if (a->B == 0 || a->n == 0) return LCA_OK;
  REQUIRE(a->x && a->y, "NULL tensor pointer");
  return hip_status(lca::launch_rmsnorm_rows(a->B, a->n, a->c, a->x, a->x_dtype, a->y, a->y_dtype,
                                             a->y_seq_rows, a->eps, static_cast<long long>(a->pos0),
                                             rope_step(a->rope_base),
                                             reinterpret_cast<hipStream_t>(stream)),
                    "lca_rmsnorm_rows");
}

int lca_indexer_scores(const lca_indexer_args* a, lca_stream_t stream) {
  g_last_error.clear();
  CHECK_ARGS(a, lca_indexer_args);
  REQUIRE(a->B >= 0 && a->n_q >= 0 && a->N_cap >= 0, "negative sizes");
  REQUIRE(a->m >= 1, "m = %d < 1", a->m);
  REQUIRE(a->H_I >= 1 && a->d_I >= 1, "H_I and d_I must be positive");
  if (a->idx_dtype == LCA_F32) {
    SUPPORT(a->H_I <= 64 && a->d_I <= 256 && a->d_I % 4 == 0, "F32 indexer needs H_I <= 64, d_I <= 256");
  } else if (a->idx_dtype == LCA_FP8_E4M3 || a->idx_dtype == LCA_MXFP4) {
    SUPPORT(a->H_I == 64 && a->d_I == 128, "FP8/MXFP4 indexer needs H_I == 64 and d_I == 128");
  } else {
    return fail(LCA_ERR_UNSUPPORTED, "idx_dtype %d unsupported", a->idx_dtype);
  }
  SUPPORT(a->score_dtype == LCA_F32 || a->score_dtype == LCA_BF16, "score_dtype %d unsupported (F32 or BF16)",
          a->score_dtype);
  if (a->idx_dtype == LCA_MXFP4) REQUIRE(a->qI_scale && a->kI_scale, "MXFP4 needs qI_scale and kI_scale");
  if (a->B == 0 || a->n_q == 0 || a->N_cap == 0) return LCA_OK;
  REQUIRE(a->qI && a->kI && a->w && a->q_pos && a->n_entries && a->scores, "NULL tensor pointer");
  return hip_status(lca::launch_indexer(a->B, a->n_q, a->H_I, a->d_I, a->idx_dtype, a->qI, a->qI_scale, a->kI,
                                        a->kI_scale, a->N_cap, a->w, a->q_pos, a->m, a->n_entries, a->scores,
                                        reinterpret_cast<hipStream_t>(stream), nullptr, nullptr, nullptr,
                                        nullptr, 0, a->score_dtype),
                    "lca_indexer_scores");
}

}  // extern "C"

namespace {

int topk_check(const lca_topk_args* a) {
  CHECK_ARGS(a, lca_topk_args);
  REQUIRE(a->B >= 0 && a->n_q >= 0 && a->N_cap >= 0, "negative sizes");
  REQUIRE(a->k >= 1 && a->k <= 4096, "k = %d out of range [1, 4096]", a->k);
  REQUIRE(a->m >= 1, "m = %d < 1", a->m);
  SUPPORT(a->N_cap <= (1 << 23), "N_cap = %d too large", a->N_cap);
  SUPPORT(a->score_dtype == LCA_F32 || a->score_dtype == LCA_BF16, "score_dtype %d unsupported (F32 or BF16)",
          a->score_dtype);
  return LCA_OK;
}

int mqa_check(const lca_sparse_mqa_args* a, lca::KvPages* pg) {
  CHECK_ARGS(a, lca_sparse_mqa_args);
  REQUIRE(a->m >= 1, "m = %d < 1", a->m);
  if (int st = kv_pages(&a->pages, a->m, a->N_cap, pg)) return st;
  REQUIRE(rope_ok(a->rope_base), "rope_base = %g is neither 0 nor a finite value > 1", a->rope_base);
  REQUIRE(a->B >= 0 && a->n_q >= 0 && a->N_cap >= 0, "negative sizes");
  SUPPORT(a->c == 128 || a->c == 256 || a->c == 512, "c = %d unsupported (128, 256 or 512)", a->c);
  SUPPORT(a->H >= 8 && a->H % 8 == 0, "H = %d unsupported (multiple of 8)", a->H);
  SUPPORT(io_fmt_ok(a->q_dtype) && io_fmt_ok(a->out_dtype), "q/out dtype unsupported (F32 or BF16)");
  SUPPORT(kv_fmt_ok(a->kv_dtype), "kv_dtype %d unsupported", a->kv_dtype);
  REQUIRE(a->idx == nullptr || (a->k >= 1 && a->k <= 4096), "k = %d out of range", a->k);
  REQUIRE(a->n_win >= 0 && a->n_win <= 4096, "n_win = %d out of range", a->n_win);
  if (int st = split_rows_ok(a->split_rows, a->idx ? a->k : 0, a->N_cap, a->n_win, a->idx == nullptr))
    return st;
  return LCA_OK;
}

size_t mqa_ws(const lca_sparse_mqa_args* a) {
  return lca::mqa_workspace_bytes(a->B, a->n_q, a->H, a->c, a->kv_dtype, a->k, a->N_cap, a->n_win,
                                  a->idx == nullptr, a->split_rows);
}

int out_proj_check(const lca_grouped_out_proj_args* a) {
  CHECK_ARGS(a, lca_grouped_out_proj_args);
  const int T = a->T, n_h = a->n_h, c = a->c, g = a->g, d_g = a->d_g, d = a->d;
  REQUIRE(T >= 0, "T = %d < 0", T);
  REQUIRE(n_h >= 1 && c >= 1 && g >= 1 && d_g >= 1 && d >= 1, "sizes must be positive");
  REQUIRE(n_h % g == 0, "n_h = %d is not a multiple of g = %d", n_h, g);
  SUPPORT(d_g % 128 == 0 && d % 128 == 0, "d_g = %d and d = %d must be multiples of 128", d_g, d);
  SUPPORT((n_h / g) * c % 64 == 0, "a group's input (n_h/g)*c = %d must be a multiple of 64",
          (n_h / g) * c);
  SUPPORT(static_cast<long long>(T) * n_h * c < (1LL << 31) &&
              static_cast<long long>(d) * g * d_g < (1LL << 31),
          "tensor too large");
  SUPPORT(io_fmt_ok(a->out_dtype), "out_dtype %d unsupported (F32 or BF16)", a->out_dtype);
  return LCA_OK;
}

int workspace_ok(const char* name, size_t need, const void* ws, size_t have) {
  if (need > 0 && (ws == nullptr || have < need))
    return fail(LCA_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", name, need, ws ? have : 0);
  return LCA_OK;
}

}  // namespace

extern "C" {

int lca_topk(const lca_topk_args* a, lca_stream_t stream) {
  g_last_error.clear();
  if (int st = topk_check(a)) return st;
  const size_t need = lca::topk_workspace_bytes(a->B, a->n_q, a->N_cap, a->k);
  if (int st = workspace_ok("lca_topk", need, a->workspace, a->workspace_bytes)) return st;
  if (a->B == 0 || a->n_q == 0) return LCA_OK;
  REQUIRE(a->scores && a->q_pos && a->n_entries && a->idx, "NULL tensor pointer");
  return hip_status(lca::launch_topk(a->B, a->n_q, a->N_cap, a->scores, a->q_pos, a->m, a->n_entries, a->k,
                                     a->idx, a->workspace, reinterpret_cast<hipStream_t>(stream),
                                     a->score_dtype),
                    "lca_topk");
}

int lca_sparse_mqa(const lca_sparse_mqa_args* a, lca_stream_t stream) {
  g_last_error.clear();
  lca::KvPages pg;
  if (int st = mqa_check(a, &pg)) return st;
  REQUIRE(a->n_win == 0 || (a->win != nullptr && a->W_cap >= 1), "window buffer missing");
  if (int st = workspace_ok("lca_sparse_mqa", mqa_ws(a), a->workspace, a->workspace_bytes)) return st;
  if (a->B == 0 || a->n_q == 0) return LCA_OK;
  REQUIRE(a->q && a->cache && a->q_pos && a->n_entries && a->out, "NULL tensor pointer");
  return hip_status(lca::launch_mqa(a->B, a->n_q, a->H, a->c, a->q, a->q_dtype, a->cache, a->kv_dtype, a->N_cap,
                                    a->idx, a->k, a->q_pos, a->m, a->n_entries, a->win, a->W_cap,
                                    a->win_origin, a->n_win, a->tau, a->eps, a->sink,
                                    rope_step(a->rope_base), a->out, a->out_dtype, a->lse, a->workspace,
                                    pg, reinterpret_cast<hipStream_t>(stream), a->split_rows),
                    "lca_sparse_mqa");
}

int lca_state_append(const lca_state_append_args* a, lca_stream_t stream) {
  g_last_error.clear();
  CHECK_ARGS(a, lca_state_append_args);
  REQUIRE(a->mode == LCA_CSA || a->mode == LCA_HCA, "mode %d is not LCA_CSA/LCA_HCA", a->mode);
  REQUIRE(a->m >= 1 && a->m <= 4096, "m = %d out of range", a->m);
  lca::KvPages pg;
  if (int st = kv_pages(&a->pages, a->m, a->N_cap, &pg)) return st;
  REQUIRE(rope_ok(a->rope_base), "rope_base = %g is neither 0 nor a finite value > 1", a->rope_base);
  REQUIRE(a->B >= 0 && a->N_cap >= 0, "negative sizes");
  REQUIRE(a->n_win >= 1, "n_win = %d < 1", a->n_win);
  SUPPORT(c_ok(a->c), "c = %d unsupported", a->c);
  SUPPORT(io_fmt_ok(a->io_dtype), "io_dtype %d unsupported", a->io_dtype);
  SUPPORT(kv_fmt_ok(a->kv_dtype), "kv_dtype %d unsupported", a->kv_dtype);
  if (a->B == 0) return LCA_OK;
  REQUIRE(a->tokC && a->tokZ && a->tailC && a->tailZ && a->ring && a->P && a->cache && a->n_tokens &&
              a->q_pos && a->n_entries,
          "NULL tensor pointer");
  return hip_status(lca::launch_state_append(a->mode, a->m, a->B, a->c, a->n_win, a->tokC, a->tokZ, a->io_dtype,
                                             a->tailC, a->tailZ, a->ring, a->kv_dtype, a->P, a->cache,
                                             a->N_cap, a->n_tokens, a->q_pos, a->n_entries, a->eps,
                                             rope_step(a->rope_base), pg,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "lca_state_append");
}

int lca_read_bandwidth_probe(const void* buf, size_t bytes, uint32_t* sink, lca_stream_t stream) {
  g_last_error.clear();
  REQUIRE(bytes % 16 == 0, "bytes = %zu is not a multiple of 16", bytes);
  if (bytes == 0) return LCA_OK;
  REQUIRE(buf && sink, "NULL pointer");
  return hip_status(lca::launch_read_probe(buf, bytes, sink, reinterpret_cast<hipStream_t>(stream)),
                    "lca_read_bandwidth_probe");
}

int lca_device_checks(uint64_t* violations, int reset) {
  g_last_error.clear();
  REQUIRE(violations, "NULL pointer");
  *violations = 0;
  if (!LCA_DEVICE_CHECKS)
    return fail(LCA_ERR_UNSUPPORTED, "lca_device_checks: this build has no device checks "
                                     "(build.py --device-checks)");
  int st = hip_status(hipDeviceSynchronize(), "lca_device_checks/hipDeviceSynchronize");
  if (st != LCA_OK) return st;
  unsigned long long a = 0, c = 0, t = 0;
  const bool rs = reset != 0;
  if ((st = hip_status(lca::dbg_violations_attention(&a, rs), "lca_device_checks/attention")) != LCA_OK ||
      (st = hip_status(lca::dbg_violations_compress(&c, rs), "lca_device_checks/compress")) != LCA_OK ||
      (st = hip_status(lca::dbg_violations_topk(&t, rs), "lca_device_checks/topk")) != LCA_OK)
    return st;
  *violations = a + c + t;
  return LCA_OK;
}

int lca_grouped_out_proj(const lca_grouped_out_proj_args* a, lca_stream_t stream) {
  g_last_error.clear();
  if (int st = out_proj_check(a)) return st;
  const size_t need = lca::out_proj_workspace_bytes(a->T, a->n_h, a->c, a->g, a->d_g, a->d);
  if (int st = workspace_ok("lca_grouped_out_proj", need, a->workspace, a->workspace_bytes)) return st;
  if (a->T == 0) return LCA_OK;
  REQUIRE(a->o && a->W_g && a->W_o && a->z && a->out, "NULL tensor pointer");
  return hip_status(lca::launch_out_proj(a->T, a->n_h, a->c, a->g, a->d_g, a->d, a->o, a->W_g, a->W_o, a->z,
                                         a->out, a->out_dtype, a->workspace,
                                         reinterpret_cast<hipStream_t>(stream)),
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
                                     L->n_win, csa ? 0 : 1, L->split_rows));
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
  const bool csa = L->mode == LCA_CSA;
  if (int st = split_rows_ok(L->split_rows, csa ? L->k : 0, L->N_cap, L->n_win, csa ? 0 : 1)) return st;
  lca::KvPages pg;
  return kv_pages(&L->pages, L->m, L->N_cap, &pg);
}

}  // namespace

int lca_workspace_size(int op, const void* args, size_t* bytes) {
  g_last_error.clear();
  REQUIRE(bytes != nullptr, "NULL bytes pointer");
  *bytes = 0;
  switch (op) {
    case LCA_OP_TOPK: {
      const auto* a = static_cast<const lca_topk_args*>(args);
      if (int st = topk_check(a)) return st;
      *bytes = lca::topk_workspace_bytes(a->B, a->n_q, a->N_cap, a->k);
      return LCA_OK;
    }
    case LCA_OP_SPARSE_MQA: {
      const auto* a = static_cast<const lca_sparse_mqa_args*>(args);
      lca::KvPages pg;
      if (int st = mqa_check(a, &pg)) return st;
      *bytes = mqa_ws(a);
      return LCA_OK;
    }
    case LCA_OP_GROUPED_OUT_PROJ: {
      const auto* a = static_cast<const lca_grouped_out_proj_args*>(args);
      if (int st = out_proj_check(a)) return st;
      *bytes = lca::out_proj_workspace_bytes(a->T, a->n_h, a->c, a->g, a->d_g, a->d);
      return LCA_OK;
    }
    case LCA_OP_DECODE_STEP: {
      const auto* L = static_cast<const lca_decode_layer*>(args);
      if (int st = check_layer(L)) return st;
      *bytes = decode_layout(L).total;
      return LCA_OK;
    }
    default:
      return fail(LCA_ERR_INVALID_ARG, "op %d has no workspace (enum lca_op)", op);
  }
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
  // sel_hist: the histogram kept (zero-filled) with the layer's state instead,
  // which the finish pass leaves cleared, so nothing clears it before the indexer
  const bool state_hist = fused && L->sel_hist != nullptr;
  if (fused) {
    sw = lca::select_ws_in(ws + d.topk, L->B, L->N_cap);
    if (state_hist) {
      sw.hist = L->sel_hist;
      sw.clear_hist = 1;
    } else {
      hist = sw.hist;
      zero_words = lca::select_zero_words(L->B);
    }
  } else if (csa && L->idx_dtype != LCA_F32) {
    hist = lca::topk_hist_in_workspace(ws + d.topk, L->B, 1, L->N_cap, L->k);
    zero_words = hist ? lca::topk_hist_words(L->B) : 0;
  }
  if ((st = mark(0)) != LCA_OK) return st;
  // HCA steps whose attention runs on the few-row decode kernel append the token
  // inside that launch (same rows, entries and counts, one launch fewer)
  const bool fused_append = !csa && L->io_dtype == LCA_BF16 &&
                            lca::mqa_can_append(L->B, L->H, L->c, L->io_dtype, L->kv_dtype, L->N_cap,
                                                L->n_win, L->split_rows);
  // CSA steps with the fused selection run the append as extra workgroups of the
  // selection's finish launch, beside its one workgroup per row; the indexer
  // takes its positions from n_tokens (sel_hist given) or from a light launch
  // that also clears the workspace histogram
  const bool finish_append = fused && L->io_dtype == LCA_BF16 && L->c == 512;
  lca::StateAppend app{};
  lca::DecodeAppend ap{};
  if (finish_append) {
    app.m = L->m;
    app.B = L->B;
    app.n_win = L->n_win;
    app.kv_fmt = L->kv_dtype;
    app.N_cap = L->N_cap;
    app.tokC = static_cast<const uint8_t*>(io->tokC);
    app.tokZ = static_cast<const uint8_t*>(io->tokZ);
    app.tailC = static_cast<uint8_t*>(L->tailC);
    app.tailZ = static_cast<uint8_t*>(L->tailZ);
    app.ring = static_cast<uint8_t*>(L->ring);
    app.P = L->P;
    app.cache = static_cast<uint8_t*>(L->cache);
    app.n_tokens = L->n_tokens;
    app.eps = L->eps;
    app.rope_step = rope_step(L->rope_base);
    app.pg = pg;
    if (state_hist) {  // the indexer takes the positions from n_tokens itself
      sw.n_tokens = L->n_tokens;
      sw.q_pos_out = q_pos;
      sw.n_entries_out = n_ent;
    } else {
      st = hip_status(lca::launch_decode_prep(L->m, L->B, L->N_cap, L->n_tokens, q_pos, n_ent, hist,
                                              zero_words, s),
                      "lca_decode_step/prep");
      if (st != LCA_OK) return st;
    }
  } else if (fused_append) {
    ap.tokC = static_cast<const uint8_t*>(io->tokC);
    ap.tokZ = static_cast<const uint8_t*>(io->tokZ);
    ap.tailC = static_cast<uint8_t*>(L->tailC);
    ap.tailZ = static_cast<uint8_t*>(L->tailZ);
    ap.P = L->P;
    ap.ring = static_cast<uint8_t*>(L->ring);
    ap.cache = static_cast<uint8_t*>(L->cache);
    ap.n_tokens = L->n_tokens;
    ap.q_pos = q_pos;
    ap.n_entries = n_ent;
  } else {
    st = hip_status(lca::launch_state_append(L->mode, L->m, L->B, L->c, L->n_win, io->tokC, io->tokZ,
                                             L->io_dtype, L->tailC, L->tailZ, L->ring, L->kv_dtype,
                                             L->P, L->cache, L->N_cap, L->n_tokens, q_pos, n_ent,
                                             L->eps, rope_step(L->rope_base), pg, s, hist, zero_words),
                    "lca_decode_step/append");
    if (st != LCA_OK) return st;
  }
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
                                        fused ? idx : nullptr, finish_append ? &app : nullptr),
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
                                  ws + d.mqa, pg, s, L->split_rows, fused_append ? &ap : nullptr),
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
