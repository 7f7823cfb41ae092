/*
 * lca.h -- C ABI of the MI355X (gfx950) CSA/HCA long-context attention path.
 *
 * The method (DeepSeek-V4's hybrid attention, as described on the pages
 * "DeepSeek V4 Architecture Tricks" (pinktalk.online), the QbitAI article on
 * DeepSeek-V4 (m.admirer.cn) and "[DeepSeek-5] DeepSeek-V4 Technical Report:
 * Hybrid Attention and Post-Training for Million-Token Contexts"
 * (xutianle.me)):
 *   - every m tokens' KV candidates are pooled into one compressed entry by a
 *     per-channel softmax over gate logits plus a learned positional bias;
 *     CSA (m = 4) also pools the previous block (overlap), HCA (m' = 128)
 *     does not;
 *   - CSA scores each query against every visible entry with the lightning
 *     indexer and keeps the top-k (k = 1024) entries;
 *   - multi-query attention (one KV row is both key and value, head dim
 *     c = 512) runs over the kept entries (CSA) or all visible entries (HCA),
 *     plus a sliding window over the last n_win = 128 tokens' uncompressed
 *     KV; both branches form one softmax, merged by log-sum-exp;
 *   - queries and KV are RMS-normalised before attention.
 *
 * Conventions shared by every call
 *   - Every entry point takes a pointer to a versioned argument struct whose
 *     first field, struct_size, must equal sizeof() of that struct in this
 *     header (a caller built against another layout is rejected with
 *     LCA_ERR_INVALID_ARG, never misread), plus the stream.  Appending fields
 *     in a later version changes sizeof() and so cannot be confused with an
 *     older caller's struct.
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory and keeps no pointer after a
 *     call returns.  Scratch space is a caller-provided device workspace whose
 *     size lca_workspace_size() returns for the same arguments
 *     (lca_decode_step_static is the one exception: see there).
 *   - Tensors are dense and row-major in the shapes given, with no element
 *     strides: the kernels derive every address from the shape, and the
 *     innermost dimension is read in 16-byte pieces.  Every pointer must be
 *     16-byte aligned.  A strided view is made contiguous by the caller.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call synchronises the host.
 *   - Arguments are validated on the host before any HIP call; a call that
 *     returns an error has enqueued nothing.  A HIP launch failure returns
 *     LCA_ERR_HIP.  lca_last_error() gives a per-thread message for the last
 *     failing call.  No call aborts, prints or throws.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs.  A sequence's outputs do not depend on the other sequences'
 *     data; its selection does not depend on the batch at all, while its
 *     attention output can change in the last bits when the batch size moves
 *     the attention into another split plan, unless the caller fixes the
 *     plan with split_rows (see lca_sparse_mqa).
 *   - The library keeps no mutable state of its own besides, per device and
 *     kernel, a once-only record that a kernel's LDS limit was raised and the
 *     address of lca_decode_step_static's scratch array (both set under
 *     std::call_once, so first calls from several host threads are safe).

 * Stored formats (enum lca_dtype)
 *   LCA_F32              IEEE float32.
 *   LCA_BF16             bfloat16 (upper half of float32), round to nearest even.
 *   LCA_FP8_E4M3         OCP fp8 e4m3fn (bias 7, no inf, max 448), one byte.
 *   LCA_MXFP4            OCP MXFP4: e2m1 codes, two per byte (element 2i in the
 *                        low nibble), plus a separate uint8 E8M0 scale
 *                        (2^(s-127)) per 32 consecutive elements of the row.
 *   LCA_KV_FP8_BF16ROPE  a KV row of c dims stored as c-64 e4m3 bytes followed
 *                        by the last 64 dims (the RoPE dims) as bf16: c+64 bytes
 *                        ("DeepSeek V4 Architecture Tricks", section
 *                        "Partial RoPE 和 Attention Sink").
 *
 * Positions and visibility
 *   Tokens of a sequence have positions 0, 1, 2, ...  Compressed entry s covers
 *   tokens [s*m, (s+1)*m).  A query at position t sees entry s iff
 *   (s+1)*m - 1 <= t and s < n_entries[b] (strict causality of compressed
 *   attention: an entry that covers a future token is never visible).  Its
 *   window is positions max(0, t-n_win+1) .. t.
 *
 * Partial RoPE (argument rope_base; 0 = off, otherwise a finite base > 1)
 *   "DeepSeek V4 Architecture Tricks", section "Partial RoPE 和 Attention
 *   Sink"; QbitAI article, hybrid attention section: only the last 64 dims of
 *   queries, KV entries and the attention output carry positions, and the
 *   output is turned back by minus the query position so that only relative
 *   positions remain.  Pair i of the last 64 dims (c-64+2i, c-64+2i+1) turns
 *   by the angle pos * rope_base^(-2i/64): (x, y) -> (x cos - y sin,
 *   x sin + y cos).  A compressed entry is turned at the position of the last
 *   token it covers, (s+1)*m - 1; window KV at its token's position; the
 *   query at t; the output by -t.  Rows that the caller stores directly in a
 *   cache or ring are taken as already turned.  The angle is reduced in
 *   float64 before a float32 sincos.
 */
#ifndef LCA_H
#define LCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCA_ABI_VERSION 5

/* A hipStream_t. */
typedef struct ihipStream_t* lca_stream_t;

enum lca_status {
  LCA_OK = 0,
  LCA_ERR_INVALID_ARG = -1, /* a NULL pointer, bad size, shape, enum value or struct_size */
  LCA_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype/shape combination)        */
  LCA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required                 */
  LCA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed                 */
};

enum lca_dtype {
  LCA_F32 = 0,
  LCA_BF16 = 1,
  LCA_FP8_E4M3 = 2,
  LCA_MXFP4 = 3,
  LCA_KV_FP8_BF16ROPE = 4
};

enum lca_mode {
  LCA_CSA = 0, /* compressed sparse attention: overlapped m-token blocks, top-k */
  LCA_HCA = 1  /* heavily compressed attention: disjoint m'-token blocks, dense */
};

/* Operations with a workspace, for lca_workspace_size. */
enum lca_op {
  LCA_OP_TOPK = 1,           /* args: const lca_topk_args*            */
  LCA_OP_SPARSE_MQA = 2,     /* args: const lca_sparse_mqa_args*      */
  LCA_OP_GROUPED_OUT_PROJ = 3, /* args: const lca_grouped_out_proj_args* */
  LCA_OP_DECODE_STEP = 4     /* args: const lca_decode_layer*         */
};

/* Paged compressed-KV cache ("DeepSeek V4 Architecture Tricks", section
 * "Heterogeneous KV Cache Layout": the classical cache of compressed entries is
 * kept in blocks of lcm(m, m') = 128 tokens, so that CSA and HCA layers share
 * one block table).  With pages, a cache argument is a pool of n_pages pages of
 * epp = page_tokens / m entries each ([n_pages, epp, row]); entry e of
 * sequence b lives in page block_table[b * max_pages + e / epp], row e % epp.
 * The indexer keys are not paged (they stay [B, N_cap, d_I]).  block_table ==
 * NULL means the contiguous [B, N_cap, row] layout.  Requirements:
 * page_tokens % m == 0, N_cap <= max_pages * epp.  The table is device memory
 * the library cannot inspect on the host: an entry whose page id is outside
 * [0, n_pages) is treated as absent (never read, never written), so a bad
 * table cannot make a kernel touch memory outside the pool. */
typedef struct lca_kv_pages {
  const int32_t* block_table; /* [B, max_pages] int32 device: physical page of logical page j */
  int max_pages;              /* logical pages per sequence (row stride of block_table) */
  int page_tokens;            /* tokens per page (128 = lcm(4, 128) shares a table across layers) */
  int n_pages;                /* pages in the pool */
} lca_kv_pages;

/* ABI version (LCA_ABI_VERSION of the built library). */
int lca_version(void);

/* Static text for a status code. */
const char* lca_status_string(int status);

/* Message of the last failing call on this thread ("" if none). */
const char* lca_last_error(void);

/* Bytes of one stored KV row of c dims in format kv_dtype (F32, BF16 or
 * KV_FP8_BF16ROPE), or 0 if the combination is invalid. */
size_t lca_kv_row_bytes(int kv_dtype, int c);

/* ---------------------------------------------------------------------------
 * lca_workspace_size -- *bytes = the workspace that operation `op` (enum
 * lca_op) needs for these arguments (0: none).  The args struct is validated
 * as by the operation itself, except for its tensor pointers and workspace
 * fields; an invalid one returns its error status and leaves *bytes at 0.
 * Operations not in lca_op need no workspace.
 * ------------------------------------------------------------------------- */
int lca_workspace_size(int op, const void* args, size_t* bytes);

/* ---------------------------------------------------------------------------
 * lca_compress -- the KV compressor on a prefill chunk.
 * "DeepSeek V4 Architecture Tricks", section "压缩 KV 的具体 trick": KV
 * candidates and compression weights come from the hidden states; weights
 * plus a learnable positional bias go through a softmax; the weighted sum is
 * the compressed entry; CSA also looks at the previous block's candidates.
 *
 * For entry s of the chunk (s = 0 .. n_new/m - 1) and channel ch:
 *   E[s,ch] = sum_j softmax_j(Z[j,ch] + P[slot(j),ch]) * C[j,ch]
 * over candidates j: CSA -- the m tokens of the previous block then the m
 * tokens of block s (slots 0 .. 2m-1 in time order; for s = 0 the previous
 * block is prevC/prevZ, or absent (masked) when those are NULL); HCA -- the m
 * tokens of block s (slots 0 .. m-1).  The stored entry is
 * cast(E / sqrt(mean(E^2) + eps)) (unit-gain RMSNorm, QbitAI article, hybrid
 * attention section), written to cache[b, first_entry + s].  Entries have the
 * bits lca_state_append gives an entry it compresses from the same tokens.
 * ------------------------------------------------------------------------- */
typedef struct lca_compress_args {
  size_t struct_size;   /* sizeof(lca_compress_args) */
  int mode;             /* LCA_CSA or LCA_HCA */
  int m;                /* tokens per entry (1 .. 4096); n_new % m == 0 */
  int B, n_new, c;      /* sequences, new tokens per sequence, channels (128, 256, 512 or 1024) */
  const void* C;        /* [B, n_new, c] candidates, io_dtype */
  const void* Z;        /* [B, n_new, c] gate logits, io_dtype */
  int io_dtype;         /* F32 or BF16 */
  const void* prevC;    /* [B, m, c] previous block (CSA only) or NULL ...   */
  const void* prevZ;    /* ... both set or both NULL                         */
  const float* P;       /* [2m, c] (CSA) or [m, c] (HCA) float32 positional bias */
  void* cache;          /* [B, N_cap, row] in kv_dtype (or a page pool); rows first_entry ..
                           first_entry + n_new/m - 1 are written */
  int kv_dtype;         /* F32, BF16 or KV_FP8_BF16ROPE */
  int N_cap;            /* rows per sequence; first_entry + n_new/m <= N_cap */
  int first_entry;
  float eps;            /* RMSNorm epsilon */
  float rope_base;      /* partial RoPE base (0 = off): entry first_entry + s is turned at
                           position (first_entry+s+1)*m - 1 */
  lca_kv_pages pages;   /* block_table NULL: contiguous cache */
} lca_compress_args;
int lca_compress(const lca_compress_args* args, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_rmsnorm_rows -- y[b, i] = cast(x[b, i] / sqrt(mean(x[b, i]^2) + eps)):
 * the window (uncompressed) KV of new tokens, RMSNorm of their KV candidates
 * (QbitAI article, hybrid attention section: Q/KV RMSNorm; sliding-window
 * branch over uncompressed KV).  Rows have the bits lca_state_append writes
 * to the window ring for the same token.
 * ------------------------------------------------------------------------- */
typedef struct lca_rmsnorm_rows_args {
  size_t struct_size;   /* sizeof(lca_rmsnorm_rows_args) */
  int B, n, c;
  const void* x;        /* [B, n, c] in x_dtype (F32 or BF16) */
  int x_dtype;
  void* y;              /* row (b, i) at y + (b*y_seq_rows + i) * row_bytes(y_dtype, c) */
  int y_dtype;          /* F32, BF16 or KV_FP8_BF16ROPE */
  int y_seq_rows;       /* >= n */
  float eps;
  float rope_base;      /* 0 = off, else row i is turned at position pos0 + i */
  int64_t pos0;         /* 0 .. 2^40 */
} lca_rmsnorm_rows_args;
int lca_rmsnorm_rows(const lca_rmsnorm_rows_args* args, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_indexer_scores -- lightning-indexer scores (QbitAI article, hybrid
 * attention section: inherited from V3.2's DSA; "DeepSeek V4 Architecture
 * Tricks", section "CSA": 64 indexer heads of dim 128; section "FP4 / FP8
 * Quantization-Aware Training": the indexer QK path in FP4, and index scores
 * kept in BF16 for an about twice faster selector):
 *   I[b,t,s] = sum_h w[b,t,h] * max(0, sum_d qI[b,t,h,d] * kI[b,s,d])
 * for s < vis(b,t) = min((q_pos[b,t]+1)/m, n_entries[b]).  Entries s >=
 * vis(b,t) are not written.  Products accumulate in float32; with score_dtype
 * BF16 each visible score is stored as the round-to-nearest-even of that
 * float32 score.  FP8/MXFP4 need H_I == 64 and d_I == 128; F32 needs
 * d_I <= 256, d_I % 4 == 0, H_I <= 64.
 * ------------------------------------------------------------------------- */
typedef struct lca_indexer_args {
  size_t struct_size;   /* sizeof(lca_indexer_args) */
  int B, n_q, H_I, d_I;
  int idx_dtype;        /* F32, FP8_E4M3 or MXFP4 (for both qI and kI) */
  const void* qI;       /* [B, n_q, H_I, d_I] (MXFP4: [B, n_q, H_I, d_I/2] bytes) */
  const uint8_t* qI_scale; /* MXFP4: [B, n_q, H_I, d_I/32] E8M0; NULL otherwise */
  const void* kI;       /* [B, N_cap, d_I] (MXFP4: bytes) */
  const uint8_t* kI_scale; /* MXFP4: [B, N_cap, d_I/32]; NULL otherwise */
  int N_cap;
  const float* w;       /* [B, n_q, H_I] float32 head weights */
  const int32_t* q_pos; /* [B, n_q] int32 positions (device) */
  int m;
  const int32_t* n_entries; /* [B] int32 (device) */
  void* scores;         /* [B, n_q, N_cap] in score_dtype */
  int score_dtype;      /* F32 or BF16 */
} lca_indexer_args;
int lca_indexer_scores(const lca_indexer_args* args, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_topk -- per-query top-k selection ("DeepSeek V4 Architecture Tricks",
 * section "CSA": top-k = 1024; QbitAI article: 1M tokens attend 1024
 * compressed blocks).  idx[b,t,:] holds the min(k, vis) indices s < vis(b,t)
 * with the largest scores[b,t,s] (equal scores: lower index first; -0 counts
 * as +0 and NaN as -inf), in ascending order, followed by -1 padding.  A BF16
 * row selects among the bf16 values (its selection can differ from the
 * float32 one only among scores that round to the same bf16 value).
 * ------------------------------------------------------------------------- */
typedef struct lca_topk_args {
  size_t struct_size;   /* sizeof(lca_topk_args) */
  int B, n_q, N_cap;    /* N_cap <= 2^23 */
  const void* scores;   /* [B, n_q, N_cap] in score_dtype */
  int score_dtype;      /* F32 or BF16 */
  const int32_t* q_pos; /* [B, n_q] */
  int m;
  const int32_t* n_entries; /* [B] */
  int k;                /* 1 .. 4096 */
  int32_t* idx;         /* [B, n_q, k] int32 */
  void* workspace;      /* lca_workspace_size(LCA_OP_TOPK, ...) bytes (NULL if 0) */
  size_t workspace_bytes;
} lca_topk_args;
int lca_topk(const lca_topk_args* args, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_sparse_mqa -- core attention of CSA (over idx) or HCA (idx == NULL: all
 * visible entries) plus the sliding-window branch, merged into one softmax
 * (QbitAI article, hybrid attention section: MQA over the selected compressed
 * entries, KV entries act as both key and value; Q/KV RMSNorm; the window
 * branch over the most recent tokens' uncompressed KV; the attention sink as
 * an extra logit in the denominator).  For head h of query (b,t):
 *   qh  = q[b,t,h] / sqrt(mean(q[b,t,h]^2) + eps)
 *   rows = {cache[b,s] : s in S(b,t)} u {win[b, slot(j)] : j in window(t)}
 *   out[b,t,h] = sum_x softmax_x(tau * qh . row_x) * row_x, where the softmax
 *   denominator also holds exp(sink[h]) when sink != NULL;
 *   lse[b,t,h]  = log of that denominator.
 * A query's candidate rows (selected entries in idx order, then the window
 * oldest first) are split into chunks of whole 64-row tiles, one workgroup
 * each, whose partial results are merged by log-sum-exp in chunk order.  With
 * split_rows == 0 the chunk length follows the number of query rows B*n_q
 * (about 256 workgroups in all), so a query's output bits can depend on B*n_q,
 * never on the other queries' data; a fixed split_rows (a multiple of 64)
 * makes every query's bits independent of the batch ("DeepSeek-V4：迈向高效的
 * 百万Token上下文智能", 引言: batch-invariant, deterministic kernels).
 * ------------------------------------------------------------------------- */
typedef struct lca_sparse_mqa_args {
  size_t struct_size;   /* sizeof(lca_sparse_mqa_args) */
  int B, n_q, H, c;     /* c in {128, 256, 512}, H a multiple of 8 */
  const void* q;        /* [B, n_q, H, c] in q_dtype (F32 or BF16), not normalised */
  int q_dtype;
  const void* cache;    /* [B, N_cap, row] in kv_dtype (F32, BF16 or KV_FP8_BF16ROPE), rows
                           already RMS-normalised (or a page pool); the few-row kernel keeps
                           its per-chunk partial outputs, convex combinations of such rows
                           (|value| <= sqrt(c)), in fp16 */
  int kv_dtype;
  int N_cap;
  const int32_t* idx;   /* [B, n_q, k] ascending, -1 padded (lca_topk output), or NULL (dense) */
  int k;                /* 1 .. 4096 when idx != NULL */
  const int32_t* q_pos; /* [B, n_q] */
  int m;
  const int32_t* n_entries; /* [B] */
  const void* win;      /* [B, W_cap, row] window KV in kv_dtype; position j lives in slot
                           (j - win_origin) mod W_cap.  A decode ring is W_cap = n_win,
                           win_origin = 0; a prefill buffer of positions p0 .. p0+W_cap-1 is
                           win_origin = p0.  Every window position must be present. */
  int W_cap;
  int64_t win_origin;
  int n_win;            /* 0 .. 4096 */
  float tau, eps;
  const float* sink;    /* [H] or NULL */
  float rope_base;      /* 0 = off, else qh is turned to q_pos[b,t] and out[b,t,h] back by
                           -q_pos[b,t]; the stored rows are taken as turned */
  void* out;            /* [B, n_q, H, c] in out_dtype (F32 or BF16) */
  int out_dtype;
  float* lse;           /* [B, n_q, H] or NULL */
  void* workspace;      /* lca_workspace_size(LCA_OP_SPARSE_MQA, ...) bytes (split partials) */
  size_t workspace_bytes;
  lca_kv_pages pages;   /* block_table NULL: contiguous cache; else the gather reads entry e
                           through the block table */
  int split_rows;       /* 0: automatic chunk length; else candidate rows per chunk, a multiple
                           of 64 leaving at most 256 chunks per query (batch-invariant bits) */
} lca_sparse_mqa_args;
int lca_sparse_mqa(const lca_sparse_mqa_args* args, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_grouped_out_proj -- the grouped output projection after the attention
 * (QbitAI article on DeepSeek-V4, hybrid attention section, the fourth step of
 * CSA: the n_h heads are split into g groups, each group is projected to an
 * intermediate dim d_g, and the groups' results are projected back to d):
 *   z[t, j*d_g + r] = bf16( sum_i W_g[j, r, i] * o[t, j*(n_h/g)*c + i] )
 *   out[t, n]       = sum_q W_o[n, q] * z[t, q]
 * (group j holds heads j*n_h/g .. (j+1)*n_h/g - 1, concatenated in head order).
 * Products accumulate in float32.  Needs n_h % g == 0, d_g and d multiples of
 * 128, (n_h/g)*c a multiple of 64.
 * ------------------------------------------------------------------------- */
typedef struct lca_grouped_out_proj_args {
  size_t struct_size;   /* sizeof(lca_grouped_out_proj_args) */
  int T, n_h, c, g, d_g, d;
  const uint16_t* o;    /* [T, n_h, c] bf16 (the attention output) */
  const uint16_t* W_g;  /* [g, d_g, (n_h/g)*c] bf16 (each group's matrix, output x input) */
  const uint16_t* W_o;  /* [d, g*d_g] bf16 (output x input) */
  uint16_t* z;          /* [T, g*d_g] bf16, written (the intermediate) */
  void* out;            /* [T, d] in out_dtype (F32 or BF16) */
  int out_dtype;
  void* workspace;      /* lca_workspace_size(LCA_OP_GROUPED_OUT_PROJ, ...) bytes
                           (K-split partials for small T; 0 for large T) */
  size_t workspace_bytes;
} lca_grouped_out_proj_args;
int lca_grouped_out_proj(const lca_grouped_out_proj_args* args, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_state_append -- decode-time state of uncompressed tokens ("DeepSeek V4
 * Architecture Tricks", section "Heterogeneous KV Cache Layout": the state
 * cache keeps the window KV and the tail tokens of the block not yet
 * compressed; the classical cache keeps compressed entries).  For each
 * sequence b with L = n_tokens[b] tokens so far, the new token gets position
 * p = L:
 *   - tokC/tokZ go to tail row  ((p/m)%2)*m + p%m  (CSA: two-block ring that
 *     also keeps the previous block for the overlap) or p%m (HCA);
 *   - ring[b, p % n_win] = cast(RMSNorm(tokC[b]));
 *   - if (p+1) % m == 0 the block is compressed (as lca_compress, same bits)
 *     into cache[b, (p+1)/m - 1] (skipped if that row is >= N_cap);
 *   - n_tokens[b] = p+1, q_pos[b] = p, n_entries[b] = (p+1)/m.
 *   rope_base (0 = off): the ring row and a new entry are turned at position p
 *   (the new entry's last token).
 * ------------------------------------------------------------------------- */
typedef struct lca_state_append_args {
  size_t struct_size;   /* sizeof(lca_state_append_args) */
  int mode, m, B, c, n_win;
  const void* tokC;     /* [B, c] io_dtype */
  const void* tokZ;
  int io_dtype;         /* F32 or BF16 */
  void* tailC;          /* [B, 2m (CSA) or m (HCA), c] io_dtype */
  void* tailZ;
  void* ring;           /* [B, n_win, row] kv_dtype */
  int kv_dtype;
  const float* P;       /* [2m or m, c] */
  void* cache;          /* [B, N_cap, row] (or a page pool) */
  int N_cap;
  int32_t* n_tokens;    /* [B] int32 device, advanced by one */
  int32_t* q_pos;       /* [B] written */
  int32_t* n_entries;   /* [B] written */
  float eps, rope_base;
  lca_kv_pages pages;   /* block_table NULL: contiguous cache */
} lca_state_append_args;
int lca_state_append(const lca_state_append_args* args, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_read_bandwidth_probe -- measurement only, not a step of the method: reads
 * `bytes` (a multiple of 16) of device memory at buf once, with the launch
 * shape that read fastest on MI355X (grid-stride 16-byte loads, two per lane in
 * flight, 256 workgroups of 768 threads), and writes nothing (sink, one
 * uint32 of device memory, is written only if the buffer's XOR equals a fixed
 * constant).  Timing it gives the achievable HBM read bandwidth that the
 * decode kernels' roofline fractions are set beside.
 * ------------------------------------------------------------------------- */
int lca_read_bandwidth_probe(const void* buf, size_t bytes, uint32_t* sink, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_device_checks -- debug builds only (the library built with device checks,
 * build.py --device-checks), not a step of the method: the number of violated
 * invariants the kernels have counted on the current device since the library
 * was loaded or last reset, over the index data they gather through -- a
 * selected entry that is neither -1 nor visible to its query, a page id outside
 * the pool -- and the selections they produce (min(k, vis) ascending visible
 * entries, then -1).  The kernels treat such data as the release build does (an
 * absent row, a skipped write); only the counting differs.  reset != 0 sets
 * the counters to 0.  Synchronises the device.  A release build returns
 * LCA_ERR_UNSUPPORTED with *violations = 0; NULL violations -> INVALID_ARG.
 * ------------------------------------------------------------------------- */
int lca_device_checks(uint64_t* violations, int reset);

/* ---------------------------------------------------------------------------
 * lca_decode_step -- one decode step of one CSA or HCA layer for B sequences:
 * lca_state_append, then (CSA) lca_indexer_scores + lca_topk, then
 * lca_sparse_mqa over the ring window (W_cap = n_win, win_origin = 0).  For
 * CSA rows longer than 36864 entries with an FP8/MXFP4 indexer, the indexer and
 * the top-k are fused: the scores stay on chip, each indexer workgroup writes
 * out the entries that can still be among the row's k largest, and a finish
 * pass selects the k largest among them -- the indices lca_topk returns over
 * the scores lca_indexer_scores writes for the same inputs.  Shorter rows go
 * through a score array in the workspace and lca_topk's path.  An HCA step
 * whose attention runs on the few-row decode kernel (bf16 io, H = 64, c = 512,
 * fewer than 512 sequences) does the state append inside the attention launch:
 * the workgroups that hold the new window row and the entry a completed block
 * makes write them, and use them for this step's query, and the split merge
 * advances n_tokens -- the bits of lca_state_append followed by lca_sparse_mqa.
 * A CSA step with the fused selection (bf16 io, c = 512) runs the append as
 * extra workgroups of the selection's finish launch, one per sequence, and a
 * light launch before the indexer writes the query positions and clears the
 * selection's histogram -- again the bits of the separate calls.  With a
 * sel_hist state buffer (below) that light launch goes: the indexer takes the
 * positions from n_tokens itself and the finish pass leaves the histogram
 * cleared for the next step.
 * ------------------------------------------------------------------------- */
typedef struct lca_decode_layer {
  size_t struct_size;   /* sizeof(lca_decode_layer) */
  int mode, m, B, c, H, n_win, N_cap;
  int io_dtype, kv_dtype;
  void* tailC;          /* [B, 2m|m, c]   */
  void* tailZ;
  void* ring;           /* [B, n_win, row] */
  void* cache;          /* [B, N_cap, row] */
  int32_t* n_tokens;    /* [B]            */
  const float* P;       /* [2m|m, c]      */
  const float* sink;    /* [H] or NULL    */
  float tau, eps;
  /* CSA only */
  int k, H_I, d_I, idx_dtype;
  const void* kI;       /* [B, N_cap, d_I] (+ kI_scale for MXFP4) */
  const uint8_t* kI_scale;
  float rope_base;      /* partial RoPE base, 0 = off (as in lca_state_append / lca_sparse_mqa) */
  lca_kv_pages pages;   /* paged cache (pages.block_table == NULL: contiguous [B, N_cap, row]) */
  int split_rows;       /* the attention's chunk length (see lca_sparse_mqa): 0 = automatic,
                           else fixed, which makes every sequence's bits independent of B */
  /* (ABI version 5) */
  uint32_t* sel_hist;   /* CSA: [B, 4096] uint32 device, or NULL.  The fused selection's row
                           histogram kept with the layer's state: zero-filled by the caller
                           before the layer's first step (and after any step that failed to
                           enqueue in full), left zero-filled by every step.  Used only by steps
                           that take the fused selection; with it the step needs no launch to
                           clear a histogram before the indexer.  NULL: the histogram lives in
                           the workspace and every step clears it first. */
} lca_decode_layer;

typedef struct lca_decode_io {
  size_t struct_size;   /* sizeof(lca_decode_io) */
  const void* tokC;     /* [B, c] io_dtype */
  const void* tokZ;
  const void* q;        /* [B, H, c] io_dtype */
  const void* qI;       /* CSA: [B, H_I, d_I] (+ qI_scale) */
  const uint8_t* qI_scale;
  const float* w;       /* CSA: [B, H_I] */
  void* out;            /* [B, H, c] out_dtype */
  float* lse;           /* [B, H] or NULL */
  int out_dtype;
  int32_t* idx_out;     /* CSA: [B, k] selected entries, or NULL (kept in workspace) */
  /* Optional hipEvent_t handles (NULL = skip) on `stream`: [0] is recorded before
   * the state append; in a CSA layer [1] and [2] are the start and end stamps of
   * the indexer's own dispatch (given to its launch, so [2] - [1] is the indexer
   * kernel's duration; stamped dispatches still leave a few microseconds idle on
   * either side, so a timing caller stamps a sample of its steps); [3] is
   * recorded after the top-k and [4] after the attention.  An HCA layer records
   * [1], [2] and [3] right after the append (right after [0] when the append
   * runs inside the attention launch). */
  void* stage_events[5];
} lca_decode_io;

/* Workspace of lca_decode_step: lca_workspace_size(LCA_OP_DECODE_STEP, layer, &bytes). */
int lca_decode_step(const lca_decode_layer* layer, const lca_decode_io* io, void* workspace,
                    size_t workspace_bytes, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_decode_steps -- n_steps decode steps of one layer back to back on
 * `stream` (the serving loop over the state cache: each step appends its token,
 * compresses a completed block and answers its query, so later steps see the
 * entries earlier steps made).  io points to n_steps host structs, one per
 * step (its own token, query, indexer query and outputs); the same workspace
 * serves every step.  Equivalent to n_steps calls of lca_decode_step; all
 * steps are validated before the first is enqueued.
 * ------------------------------------------------------------------------- */
int lca_decode_steps(const lca_decode_layer* layer, const lca_decode_io* io, int n_steps,
                     void* workspace, size_t workspace_bytes, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_decode_step_static -- lca_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It takes no workspace: the step's scratch space is a
 * device array of LCA_STATIC_SCRATCH_BYTES that the library owns, one copy per
 * device, placed when the library's code object is loaded on that device and
 * held until the process ends.  The call allocates nothing.  Same arguments,
 * kernels and results as lca_decode_step; the caller still passes every
 * input and output.
 *   - Returns LCA_ERR_WORKSPACE, having enqueued nothing, when the layer needs
 *     more scratch than that (the LCA_OP_DECODE_STEP workspace size >
 *     LCA_STATIC_SCRATCH_BYTES; 96 MiB holds a CSA layer of 16 sequences at
 *     1M tokens, or any HCA layer of the workloads).
 *   - Every call on a device shares that device's array, which keeps the last
 *     call's contents; the step clears what it needs cleared.  Calls that
 *     overlap on one device (unordered streams or host threads) race on the
 *     array: the caller must order them.
 * ------------------------------------------------------------------------- */
#define LCA_STATIC_SCRATCH_BYTES ((size_t)96 << 20)
int lca_decode_step_static(const lca_decode_layer* layer, const lca_decode_io* io,
                           lca_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LCA_H */
