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
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory and keeps no pointer after a
 *     call returns.  Scratch space is a caller-provided device workspace whose
 *     size the matching *_workspace_size call returns.
 *   - Tensors are dense and row-major in the shapes given; the innermost
 *     dimension is contiguous.  Every pointer must be 16-byte aligned.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call synchronises the host.
 *   - Arguments are validated on the host before any HIP call; a call that
 *     returns an error has enqueued nothing.  A HIP launch failure returns
 *     LCA_ERR_HIP.  lca_last_error() gives a per-thread message for the last
 *     failing call.  No call aborts, prints or throws.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs, independent of the other sequences in the batch.
 *
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

#define LCA_ABI_VERSION 3

/* A hipStream_t. */
typedef struct ihipStream_t* lca_stream_t;

enum lca_status {
  LCA_OK = 0,
  LCA_ERR_INVALID_ARG = -1, /* a NULL pointer, bad size, shape or enum value      */
  LCA_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype/shape combination) */
  LCA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required          */
  LCA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed          */
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

/* Paged compressed-KV cache ("DeepSeek V4 Architecture Tricks", section
 * "Heterogeneous KV Cache Layout": the classical cache of compressed entries is
 * kept in blocks of lcm(m, m') = 128 tokens, so that CSA and HCA layers share
 * one block table).  With pages, a cache argument is a pool of n_pages pages of
 * epp = page_tokens / m entries each ([n_pages, epp, row]); entry e of
 * sequence b lives in page block_table[b * max_pages + e / epp], row e % epp.
 * The indexer keys are not paged (they stay [B, N_cap, d_I]).  A NULL
 * lca_kv_pages pointer (or block_table == NULL in lca_decode_layer) means the
 * contiguous [B, N_cap, row] layout.  Requirements: page_tokens % m == 0,
 * N_cap <= max_pages * epp.  The table is device memory the library cannot
 * inspect on the host: an entry whose page id is outside [0, n_pages) is
 * treated as absent (never read, never written), so a bad table cannot make a
 * kernel touch memory outside the pool. */
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
 * attention section), written to cache[b, first_entry + s].
 *
 *   mode         LCA_CSA or LCA_HCA
 *   m            tokens per entry (>= 1); n_new % m == 0
 *   B, n_new, c  sequences, new tokens per sequence, channels (c % 64 == 0, c <= 1024)
 *   C, Z         [B, n_new, c] candidates / gate logits, format io_dtype (F32|BF16)
 *   prevC,prevZ  [B, m, c] previous block (CSA only) or both NULL
 *   P            [2m, c] (CSA) or [m, c] (HCA) float32 positional bias
 *   cache        [B, N_cap, row] stored entries, format kv_dtype; rows
 *                first_entry .. first_entry + n_new/m - 1 are written
 *   N_cap        rows per sequence in cache; first_entry + n_new/m <= N_cap
 *   eps          RMSNorm epsilon
 *   rope_base    partial RoPE base (0 = off): the normalised entry
 *                first_entry + s is turned at position (first_entry+s+1)*m - 1
 *   pages        NULL, or the paged layout of cache (see lca_kv_pages)
 * ------------------------------------------------------------------------- */
int lca_compress(int mode, int m, int B, int n_new, int c, const void* C, const void* Z,
                 int io_dtype, const void* prevC, const void* prevZ, const float* P,
                 void* cache, int kv_dtype, int N_cap, int first_entry, float eps,
                 float rope_base, const lca_kv_pages* pages, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_rmsnorm_rows -- y[b, i] = cast(x[b, i] / sqrt(mean(x[b, i]^2) + eps)):
 * the window (uncompressed) KV of new tokens, RMSNorm of their KV candidates
 * (QbitAI article, hybrid attention section: Q/KV RMSNorm; sliding-window
 * branch over uncompressed KV).
 *   x  [B, n, c] format x_dtype (F32|BF16)
 *   y  rows (b, i) at y + (b*y_seq_rows + i) * row_bytes(y_dtype, c)
 *   pos0, rope_base  with rope_base != 0, row i is turned at position pos0 + i
 *                    (0 <= pos0 <= 2^40)
 * ------------------------------------------------------------------------- */
int lca_rmsnorm_rows(int B, int n, int c, const void* x, int x_dtype, void* y, int y_dtype,
                     int y_seq_rows, float eps, int64_t pos0, float rope_base,
                     lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_indexer_scores -- lightning-indexer scores (QbitAI article, hybrid
 * attention section: inherited from V3.2's DSA; "DeepSeek V4 Architecture
 * Tricks", section "CSA": 64 indexer heads of dim 128; section "FP4 / FP8
 * Quantization-Aware Training": the indexer QK path in FP4):
 *   I[b,t,s] = sum_h w[b,t,h] * max(0, sum_d qI[b,t,h,d] * kI[b,s,d])
 * for s < vis(b,t) = min((q_pos[b,t]+1)/m, n_entries[b]).  Entries s >=
 * vis(b,t) are not written.  Products accumulate in float32.
 *
 *   idx_dtype  F32, FP8_E4M3 or MXFP4 (for both qI and kI)
 *   qI         [B, n_q, H_I, d_I] (MXFP4: [B, n_q, H_I, d_I/2] bytes + qI_scale
 *              [B, n_q, H_I, d_I/32]); qI_scale NULL otherwise
 *   kI         [B, N_cap, d_I] (MXFP4: bytes + kI_scale [B, N_cap, d_I/32])
 *   w          [B, n_q, H_I] float32 head weights
 *   q_pos      [B, n_q] int32 positions; n_entries [B] int32 (both device)
 *   scores     [B, n_q, N_cap] float32
 * FP8/MXFP4 need H_I == 64 and d_I == 128; F32 needs d_I <= 256, H_I <= 64.
 * ------------------------------------------------------------------------- */
int lca_indexer_scores(int B, int n_q, int H_I, int d_I, int idx_dtype, const void* qI,
                       const uint8_t* qI_scale, const void* kI, const uint8_t* kI_scale,
                       int N_cap, const float* w, const int32_t* q_pos, int m,
                       const int32_t* n_entries, float* scores, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_topk -- per-query top-k selection ("DeepSeek V4 Architecture Tricks",
 * section "CSA": top-k = 1024; QbitAI article: 1M tokens attend 1024
 * compressed blocks).  idx[b,t,:] holds the min(k, vis) indices s < vis(b,t)
 * with the largest scores[b,t,s] (equal scores: lower index first; -0 counts
 * as +0 and NaN as -inf), in ascending order, followed by -1 padding.
 *   scores [B, n_q, N_cap] float32, idx [B, n_q, k] int32, 1 <= k <= 4096.
 * Workspace: lca_topk_workspace_size(B, n_q, N_cap, k) bytes.
 * ------------------------------------------------------------------------- */
size_t lca_topk_workspace_size(int B, int n_q, int N_cap, int k);
int lca_topk(int B, int n_q, int N_cap, const float* scores, const int32_t* q_pos, int m,
             const int32_t* n_entries, int k, int32_t* idx, void* workspace,
             size_t workspace_bytes, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * The BF16-score selector ("DeepSeek V4 Architecture Tricks", section "FP4 /
 * FP8 Quantization-Aware Training": index scores kept in BF16 make the top-k
 * selector about twice as fast).
 * lca_indexer_scores_bf16 -- as lca_indexer_scores, but each visible score is
 *   stored as bf16: the round-to-nearest-even of the float32 score that
 *   lca_indexer_scores writes for the same inputs.  scores [B, n_q, N_cap] bf16.
 * lca_topk_bf16 -- as lca_topk over bf16 scores [B, n_q, N_cap]: the min(k, vis)
 *   largest bf16 values, equal values lower index first (-0 counts as +0, NaN
 *   as -inf), ascending, -1 padded; workspace lca_topk_workspace_size(...).
 * The selection of a bf16 row can differ from the float32 selection only among
 * scores that round to the same bf16 value.
 * ------------------------------------------------------------------------- */
int lca_indexer_scores_bf16(int B, int n_q, int H_I, int d_I, int idx_dtype, const void* qI,
                            const uint8_t* qI_scale, const void* kI, const uint8_t* kI_scale,
                            int N_cap, const float* w, const int32_t* q_pos, int m,
                            const int32_t* n_entries, uint16_t* scores, lca_stream_t stream);
int lca_topk_bf16(int B, int n_q, int N_cap, const uint16_t* scores, const int32_t* q_pos, int m,
                  const int32_t* n_entries, int k, int32_t* idx, void* workspace,
                  size_t workspace_bytes, lca_stream_t stream);

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
 *   q        [B, n_q, H, c] format q_dtype (F32|BF16), not normalised
 *   cache    [B, N_cap, row] format kv_dtype (F32|BF16|KV_FP8_BF16ROPE), rows
 *            already RMS-normalised
 *   idx      [B, n_q, k] int32 ascending, -1 padded (lca_topk output), or NULL
 *   q_pos    [B, n_q], n_entries [B] int32 device
 *   win      [B, W_cap, row] window KV in kv_dtype; position j lives in slot
 *            (j - win_origin) mod W_cap.  A decode ring is W_cap = n_win,
 *            win_origin = 0; a prefill buffer of positions p0 .. p0+W_cap-1 is
 *            win_origin = p0.  Every window position must be present.
 *   out      [B, n_q, H, c] format out_dtype (F32|BF16); lse [B, n_q, H] or NULL
 *   rope_base  partial RoPE (0 = off): qh is turned to q_pos[b,t] and out[b,t,h]
 *            back by -q_pos[b,t]; the stored rows are taken as turned
 *   pages    NULL, or the paged layout of cache (see lca_kv_pages); the gather
 *            reads entry e through the block table
 * Workspace: lca_sparse_mqa_workspace_size(...) bytes (split partials).
 * ------------------------------------------------------------------------- */
size_t lca_sparse_mqa_workspace_size(int B, int n_q, int H, int c, int kv_dtype, int k,
                                     int N_cap, int n_win, int dense);
int lca_sparse_mqa(int B, int n_q, int H, int c, const void* q, int q_dtype, const void* cache,
                   int kv_dtype, int N_cap, const int32_t* idx, int k, const int32_t* q_pos,
                   int m, const int32_t* n_entries, const void* win, int W_cap,
                   int64_t win_origin, int n_win, float tau, float eps, const float* sink,
                   float rope_base, void* out, int out_dtype, float* lse, void* workspace,
                   size_t workspace_bytes, const lca_kv_pages* pages, lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_grouped_out_proj -- the grouped output projection after the attention
 * (QbitAI article on DeepSeek-V4, hybrid attention section, the fourth step of
 * CSA: the n_h heads are split into g groups, each group is projected to an
 * intermediate dim d_g, and the groups' results are projected back to d):
 *   z[t, j*d_g + r] = bf16( sum_i W_g[j, r, i] * o[t, j*(n_h/g)*c + i] )
 *   out[t, n]       = sum_q W_o[n, q] * z[t, q]
 * (group j holds heads j*n_h/g .. (j+1)*n_h/g - 1, concatenated in head order).
 *   o    [T, n_h, c] bf16 (the attention output)
 *   W_g  [g, d_g, (n_h/g)*c] bf16 (each group's matrix, output x input)
 *   W_o  [d, g*d_g] bf16 (output x input)
 *   z    [T, g*d_g] bf16, written (the intermediate; an output of the call)
 *   out  [T, d] out_dtype (F32|BF16)
 * Products accumulate in float32.  Needs n_h % g == 0, d_g and d multiples of
 * 128, (n_h/g)*c a multiple of 64.  Workspace: lca_grouped_out_proj_workspace_size
 * bytes (K-split partials for small T; 0 for large T).
 * ------------------------------------------------------------------------- */
size_t lca_grouped_out_proj_workspace_size(int T, int n_h, int c, int g, int d_g, int d);
int lca_grouped_out_proj(int T, int n_h, int c, int g, int d_g, int d, const uint16_t* o,
                         const uint16_t* W_g, const uint16_t* W_o, uint16_t* z, void* out,
                         int out_dtype, void* workspace, size_t workspace_bytes,
                         lca_stream_t stream);

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
 *   - if (p+1) % m == 0 the block is compressed (as lca_compress) into
 *     cache[b, (p+1)/m - 1] (skipped if that row is >= N_cap);
 *   - n_tokens[b] = p+1, q_pos[b] = p, n_entries[b] = (p+1)/m.
 *   tailC, tailZ [B, 2m or m, c] io_dtype; ring [B, n_win, row] kv_dtype;
 *   cache [B, N_cap, row]; n_tokens, q_pos, n_entries [B] int32 device.
 *   rope_base (0 = off): the ring row and a new entry are turned at position p
 *   (the new entry's last token).
 *   pages (NULL = contiguous cache): the new entry goes through the block table.
 * ------------------------------------------------------------------------- */
int lca_state_append(int mode, int m, int B, int c, int n_win, const void* tokC, const void* tokZ,
                     int io_dtype, void* tailC, void* tailZ, void* ring, int kv_dtype,
                     const float* P, void* cache, int N_cap, int32_t* n_tokens, int32_t* q_pos,
                     int32_t* n_entries, float eps, float rope_base, const lca_kv_pages* pages,
                     lca_stream_t stream);

/* ---------------------------------------------------------------------------
 * lca_decode_step -- one decode step of one CSA or HCA layer for B sequences:
 * lca_state_append, then (CSA) lca_indexer_scores + lca_topk, then
 * lca_sparse_mqa over the ring window (W_cap = n_win, win_origin = 0).  For
 * CSA rows longer than 36864 entries with an FP8/MXFP4 indexer, the indexer
 * also builds the top-k's score histogram (the append clears it), so the
 * top-k skips its own histogram pass; results are identical.
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
   * [1], [2] and [3] right after the append. */
  void* stage_events[5];
} lca_decode_io;

size_t lca_decode_workspace_size(const lca_decode_layer* layer);
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

#ifdef __cplusplus
}
#endif
#endif /* LCA_H */
