"""Plain float64 CPU oracle of the CSA/HCA attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the package smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP path: every decoder, rounding rule and step of
the method below is written here, from the pages' descriptions, in float64.

Sources (all pages discuss the DeepSeek-V4 report):
  [XT]  "[DeepSeek-5] DeepSeek-V4 Technical Report: Hybrid Attention and
        Post-Training for Million-Token Contexts" (xutianle.me), sections
        "3. CSA", "4. HCA", "5. From MLA to CSA/HCA".
  [QB]  QbitAI article on DeepSeek-V4 (m.admirer.cn), section
        "混合注意力机制" (hybrid attention mechanism).
  [PT]  "DeepSeek V4 Architecture Tricks" (pinktalk.online), sections
        "CSA: Compressed Sparse Attention", "HCA: Heavily Compressed
        Attention", "压缩 KV 的具体 trick" (compressed-KV tricks),
        "Sliding Window Branch", "Partial RoPE 和 Attention Sink",
        "FP4 / FP8 Quantization-Aware Training", "Heterogeneous KV Cache Layout".

Readings where the pages are silent (each also listed in the design notes):
  * gate softmax is per channel over the candidate window; bias row i goes with
    the i-th candidate in time order; a CSA entry with no previous block masks
    the missing candidates;
  * entry s is visible to a query at position t iff its last token
    (s+1)*m - 1 <= t;
  * the window is the query's own token and the n_win-1 before it; the window
    KV of token j is RMSNorm(C[j]) stored in the KV format;
  * RMSNorm has unit gain and eps = 1e-6; softmax scale 1/sqrt(c);
  * indexer score I[t,s] = sum_h w[t,h] * relu(q_I[t,h] . k_I[s]);
  * top-k keeps the min(k, visible) largest scores, ties to the lower index,
    -0 counted as +0, NaN counted as -inf, output ascending, padded with -1;
  * the two branches form one softmax, merged by log-sum-exp; an optional
    per-head sink logit joins the denominator only;
  * partial RoPE (off unless a base is given): adjacent pairs of the last 64
    dims turn by pos * base^(-2i/64); a compressed entry sits at the position of
    the last token it covers, (s+1)*m - 1; queries turn at their own position
    and the output turns back by minus that position.
"""
from collections import deque

import numpy as np

# ---------------------------------------------------------------------------
# exact decoders of the stored formats


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact (bf16 is the top half of fp32)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    """All 256 OCP fp8 e4m3fn values: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    exponent 0 is subnormal; S.1111.111 is NaN; no infinities."""
    t = np.empty(256, np.float64)
    for v in range(256):
        s = -1.0 if v & 0x80 else 1.0
        e = (v >> 3) & 0xF
        f = v & 0x7
        if e == 0xF and f == 0x7:
            t[v] = np.nan
        elif e == 0:
            t[v] = s * (f / 8.0) * 2.0 ** -6
        else:
            t[v] = s * (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return t


E4M3 = _e4m3_table()
# e2m1 (fp4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 subnormal.
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                 -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def decode_e4m3(bits) -> np.ndarray:
    return E4M3[np.asarray(bits, dtype=np.uint8)]


def decode_mxfp4(packed, scales, block: int = 32) -> np.ndarray:
    """OCP MXFP4: two e2m1 codes per byte (element 2i in the low nibble), one E8M0
    scale byte 2^(e-127) per `block` elements along the last dim."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = E2M1[packed & 0xF]
    hi = E2M1[packed >> 4]
    x = np.stack([lo, hi], -1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return (x.reshape(*x.shape[:-1], -1, block) * sc[..., None]).reshape(x.shape)


def decode(arr, fmt: str, scales=None) -> np.ndarray:
    """Stored rows -> float64.  fmt: f32 | bf16 | fp8 | fp8_bf16rope | mxfp4."""
    if fmt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return decode_bf16(arr)
    if fmt == "fp8":
        return decode_e4m3(arr)
    if fmt == "mxfp4":
        return decode_mxfp4(arr, scales)
    if fmt == "fp8_bf16rope":
        a = np.asarray(arr, dtype=np.uint8)
        nope = a.shape[-1] - 128          # 64 bf16 rope dims take the last 128 bytes
        lo = decode_e4m3(a[..., :nope])
        hi = decode_bf16(np.ascontiguousarray(a[..., nope:]).view(np.uint16))
        return np.concatenate([lo, hi], -1)
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# rounding to a stored format (round to nearest, ties to even)


def _round_binary(x, mbits: int, emin: int, maxval: float, saturate: bool) -> np.ndarray:
    """Round to the binary format with `mbits` fraction bits, smallest normal exponent
    `emin` (gradual underflow below it) and largest finite value `maxval`."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, E = np.frexp(a)                       # a = f * 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, emin)              # exponent of the leading bit, clamped
    ulp = np.exp2(e - mbits)
    r = np.round(a / ulp) * ulp              # np.round: half to even; a/ulp is exact
    if saturate:
        r = np.minimum(r, maxval)
    else:
        r = np.where(r > maxval, np.inf, r)
    r = np.where(np.isnan(a), np.nan, r)
    return np.copysign(r, x)


def round_to(x, fmt: str, rope_dims: int = 64) -> np.ndarray:
    """Value of x after the storage cast to `fmt` (as float64)."""
    if fmt == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if fmt == "bf16":
        return _round_binary(x, 7, -126, float.fromhex("0x1.fep127"), saturate=False)
    if fmt == "fp8":
        return _round_binary(x, 3, -6, 448.0, saturate=True)
    if fmt == "fp8_bf16rope":
        x = np.asarray(x, dtype=np.float64)
        c = x.shape[-1]
        return np.concatenate([round_to(x[..., : c - rope_dims], "fp8"),
                               round_to(x[..., c - rope_dims:], "bf16")], -1)
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# the method


def rmsnorm(x, eps: float = 1e-6) -> np.ndarray:
    """Unit-gain RMSNorm over the last dim; [QB] applies it to queries and KV
    entries before core attention."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def gate_softmax(logits) -> np.ndarray:
    """Softmax over axis 1 (the candidate axis), independently per channel."""
    mx = np.max(logits, axis=1, keepdims=True)
    e = np.exp(logits - mx)
    return e / e.sum(axis=1, keepdims=True)


def compress(C, Z, P, m: int, overlap: bool, prevC=None, prevZ=None) -> np.ndarray:
    """Softmax-gated pooling of every m tokens into one entry ([PT] compressed-KV
    tricks; [XT] 3/4; [QB]).

    C, Z: [n, c] KV candidates and gate logits of n = nb*m consecutive tokens that
    start on a block boundary.  P: positional bias, one row per candidate slot.
    overlap=True (CSA): entry s pools the 2m tokens of blocks s-1 and s, with
    candidate slot i in time order taking bias row i; block -1 of the first entry
    is prevC/prevZ, or masked out when those are None.  overlap=False (HCA): entry
    s pools its own m tokens.  Returns the pooled, un-normalised entries [nb, c].
    """
    C = np.asarray(C, np.float64)
    Z = np.asarray(Z, np.float64)
    P = np.asarray(P, np.float64)
    n, c = C.shape
    assert n % m == 0
    nb = n // m
    Cb = C.reshape(nb, m, c)
    Zb = Z.reshape(nb, m, c)
    if overlap:
        if prevC is None:
            pC = np.zeros((1, m, c))
            pZ = np.zeros((1, m, c))
        else:
            pC = np.asarray(prevC, np.float64)[None]
            pZ = np.asarray(prevZ, np.float64)[None]
        cand = np.concatenate([np.concatenate([pC, Cb[:-1]], 0), Cb], 1)       # [nb, 2m, c]
        logits = np.concatenate([np.concatenate([pZ, Zb[:-1]], 0), Zb], 1) + P[None, :2 * m]
        if prevC is None:
            logits[0, :m] = -np.inf
    else:
        cand = Cb
        logits = Zb + P[None, :m]
    return (gate_softmax(logits) * cand).sum(axis=1)


def compress_error_bound(C, Z, P, m: int, overlap: bool, prevC=None, prevZ=None,
                         eps: float = 1e-6) -> np.ndarray:
    """Bound on the error of an fp32 evaluation of rmsnorm(compress(...)), before
    the storage cast.  The pooled value sum_j p_j C_j is a sum of W terms whose
    weights carry a few ulps of exp/division error, so its absolute error is at
    most gamma(2W + 32) * sum_j p_j |C_j|; the RMSNorm scale multiplies it.  Near
    zero (cancelling terms) this exceeds an ulp of the stored value."""
    C = np.asarray(C, np.float64)
    E = compress(C, Z, P, m, overlap, prevC, prevZ)
    E_abs = compress(np.abs(C), Z, P, m, overlap,
                     None if prevC is None else np.abs(np.asarray(prevC, np.float64)), prevZ)
    W = 2 * m if overlap else m
    r = 1.0 / np.sqrt(np.mean(E * E, axis=-1, keepdims=True) + eps)
    return gamma(2 * W + 32) * E_abs * r


def visible(q_pos, m: int, n_entries) -> np.ndarray:
    """Number of entries visible at position t: entry s needs (s+1)*m-1 <= t."""
    return np.minimum((np.asarray(q_pos, np.int64) + 1) // m, n_entries)


def index_scores(qI, kI, w, vis) -> np.ndarray:
    """Lightning-indexer scores ([QB]: inherited from V3.2's DSA; [PT] CSA section):
    I[t,s] = sum_h w[t,h] * max(0, qI[t,h] . kI[s]) for s < vis[t], else -inf.

    qI [nq, H_I, d_I], kI [N, d_I] (one key per entry, shared by the heads),
    w [nq, H_I]."""
    qI = np.asarray(qI, np.float64)
    kI = np.asarray(kI, np.float64)
    dots = qI @ kI.T                                          # [nq, H_I, N]
    I = (np.asarray(w, np.float64)[:, None, :] @ np.maximum(dots, 0.0))[:, 0, :]
    cols = np.arange(kI.shape[0])[None, :]
    return np.where(cols < np.asarray(vis)[:, None], I, -np.inf)


def score_error_bound(qI, kI, w, d_terms: int = 0) -> np.ndarray:
    """Bound on |I_fp32 - I_exact| for any fp32 evaluation order: the standard
    gamma_n = n*u/(1-n*u) (u = 2^-24) summation bound with n = d_I + H_I + 2,
    applied to sum_h w_h sum_d |q_hd k_d|."""
    qI = np.abs(np.asarray(qI, np.float64))
    kI = np.abs(np.asarray(kI, np.float64))
    n = qI.shape[-1] + qI.shape[-2] + 2 + d_terms
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    # sum_h w_h sum_d |q_hd| |k_sd| = sum_d (sum_h w_h |q_hd|) |k_sd|
    wq = (np.asarray(w, np.float64)[:, None, :] @ qI)[:, 0, :]  # [nq, d_I]
    return gamma * (wq @ kI.T)


def _select_key(s) -> np.ndarray:
    s = np.asarray(s, np.float64)
    s = np.where(np.isnan(s), -np.inf, s)
    return s + 0.0                       # -0.0 + 0.0 == +0.0


def topk(scores, vis, k: int) -> np.ndarray:
    """Top-k selection ([PT] CSA section: k=1024; [QB]): for each row, the indices of
    the min(k, vis) largest of scores[:vis], larger score first and lower index
    first among equal scores, returned in ascending index order, padded with -1."""
    scores = np.atleast_2d(scores)
    out = np.full((scores.shape[0], k), -1, np.int32)
    for r in range(scores.shape[0]):
        v = int(vis[r])
        key = _select_key(scores[r, :v])
        order = np.lexsort((np.arange(v), -key))          # primary: -key, then index
        sel = np.sort(order[: min(k, v)])
        out[r, : sel.size] = sel
    return out


def attend(qhat, rows, tau: float):
    """Softmax attention of H query heads over R rows that are both key and value
    (MQA, [QB]).  Returns (o [H, c], lse [H]); no rows gives lse = -inf, o = 0."""
    qhat = np.asarray(qhat, np.float64)
    rows = np.asarray(rows, np.float64)
    H, c = qhat.shape
    if rows.shape[0] == 0:
        return np.zeros((H, c)), np.full(H, -np.inf)
    logits = tau * (qhat @ rows.T)
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    l = p.sum(axis=1, keepdims=True)
    return (p @ rows) / l, (mx + np.log(l))[:, 0]


def merge(parts, sink=None):
    """Log-sum-exp merge of branch partials (o_i, lse_i) into one softmax over the
    union of their rows; an optional per-head sink logit only enlarges the
    denominator ([QB] attention sink)."""
    lses = np.stack([p[1] for p in parts])                  # [n_parts, H]
    if sink is not None:
        lses_all = np.concatenate([lses, np.asarray(sink, np.float64)[None]])
    else:
        lses_all = lses
    mx = np.max(lses_all, axis=0)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    tot = mx + np.log(np.exp(lses_all - mx).sum(axis=0))
    o = sum(np.exp(lse - tot)[:, None] * o_i for o_i, lse in parts)
    return o, tot


ROPE_DIMS = 64


def rope(x, pos, base: float, rope_dims: int = ROPE_DIMS) -> np.ndarray:
    """Rotary position embedding of the last `rope_dims` dims ([PT] Partial RoPE and
    attention sink: only the last 64 dims of queries, KV entries and the attention
    output carry positions; [QB] hybrid attention).  The pages give no frequencies
    or pairing, so this is the original rotary embedding: pair i of the rotary part
    (dims c-rope_dims+2i and c-rope_dims+2i+1) turns by the angle
    pos * base^(-2i/rope_dims), the pair (x, y) becoming
    (x cos a - y sin a, x sin a + y cos a).  `pos` broadcasts against x.shape[:-1];
    base == 0 returns x unchanged."""
    x = np.array(x, dtype=np.float64, copy=True)
    if not base:
        return x
    c = x.shape[-1]
    i = np.arange(rope_dims // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / rope_dims)
    a = np.asarray(pos, np.float64)[..., None] * theta
    cs, sn = np.cos(a), np.sin(a)
    xe = x[..., c - rope_dims::2].copy()
    xo = x[..., c - rope_dims + 1::2].copy()
    x[..., c - rope_dims::2] = xe * cs - xo * sn
    x[..., c - rope_dims + 1::2] = xe * sn + xo * cs
    return x


def entry_position(s, m: int):
    """Position of compressed entry s for RoPE: the last token it covers (the pages
    leave it open; this is also the first position that sees the entry)."""
    return (np.asarray(s, np.int64) + 1) * m - 1


def core_attention(q, parts, tau: float, eps: float, t: int, sink=None, rope_base: float = 0.0):
    """One query token's output over the branches' stored rows (each a [R, c] array:
    the selected or visible entries, then the window): RMSNorm of the query per
    head, the query turned to its position t, one softmax over all branches (their
    partials merged by log-sum-exp, with the optional sink), and the output turned
    back by -t so that only relative positions remain ([PT] Partial RoPE).  Returns
    the unrounded (o [H, c], lse [H])."""
    qhat = rope(rmsnorm(np.asarray(q, np.float64), eps), t, rope_base)
    o, lse = merge([attend(qhat, rows, tau) for rows in parts], sink)
    return rope(o, -t, rope_base), lse


def window_positions(t: int, n_win: int) -> np.ndarray:
    """The query's own position and the n_win-1 before it ([PT] Sliding Window
    Branch, n_win = 128), clipped at 0."""
    return np.arange(max(0, t - n_win + 1), t + 1)


# ---------------------------------------------------------------------------
# a whole layer: prefill of new tokens after an optional prefix


def prefill_layer(*, mode, m, k, n_win, tau, eps, kv_fmt, out_fmt, pos0,
                  C, Z, P, q, cache_prefix, prevC=None, prevZ=None, win_prefix=None,
                  qI=None, kI=None, w=None, queries=None, sink=None, idx_given=None,
                  rope_base=0.0):
    """One sequence of CSA ("csa") or HCA ("hca") prefill.

    New tokens occupy positions pos0 .. pos0+n-1 (pos0 % m == 0).  cache_prefix
    [pos0/m, c] holds the stored entries of the prefix, win_prefix the stored
    window KV of the n_win-1 prefix positions before pos0.  `queries` selects which
    new tokens to evaluate (default all); q, qI and w are indexed per query, so
    they may be lazy row accessors.  idx_given ([len(queries), k]) makes the
    attention use those selections instead of the oracle's own (the oracle's
    scores and selections are still returned).  rope_base != 0 turns the new
    entries (at their entry positions), the new window KV (at their tokens'
    positions), the queries and the outputs; the prefix rows are taken as stored.
    Returns float64 results.
    """
    C = np.asarray(C, np.float64)
    n, c = C.shape
    E = compress(C, Z, P, m, overlap=(mode == "csa"), prevC=prevC, prevZ=prevZ)
    n_pre = np.asarray(cache_prefix).reshape(-1, c).shape[0]
    e_pos = entry_position(n_pre + np.arange(E.shape[0]), m)
    entries_exact = rope(rmsnorm(E, eps), e_pos, rope_base)
    entries_new = round_to(entries_exact, kv_fmt)
    Khat = np.concatenate([np.asarray(cache_prefix, np.float64).reshape(-1, c), entries_new], 0)
    U_exact = rope(rmsnorm(C, eps), pos0 + np.arange(n), rope_base)
    U_new = round_to(U_exact, kv_fmt)
    n_pre_win = 0 if win_prefix is None else len(win_prefix)
    bound = compress_error_bound(C, Z, P, m, mode == "csa", prevC, prevZ, eps)
    if rope_base:
        bound = rope_error_bound(entries_exact, bound)
    U = U_new if win_prefix is None else np.concatenate([np.asarray(win_prefix, np.float64), U_new], 0)
    win_origin = pos0 - n_pre_win
    queries = np.arange(n) if queries is None else np.asarray(queries)
    H = np.asarray(q[int(queries[0])]).shape[0] if len(queries) else 0
    res = {"entries": entries_new, "entries_bound": bound, "window": U_new,
           "window_bound": rope_error_bound(U_exact, 0.0) if rope_base else None,
           "out": np.zeros((len(queries), H, c)),
           "lse": np.zeros((len(queries), H)), "idx": None, "scores": None}
    if mode == "csa":
        res["idx"] = np.full((len(queries), k), -1, np.int32)
        res["scores"] = []
    for r, i in enumerate(queries):
        t = pos0 + int(i)
        vis = int(visible([t], m, len(Khat))[0])
        if mode == "csa":
            I = index_scores(np.asarray(qI[i], np.float64)[None], kI[:vis],
                             np.asarray(w[i], np.float64)[None], [vis])
            sel = topk(I, [vis], k)[0]
            res["idx"][r] = sel
            res["scores"].append(I[0])
            use = sel if idx_given is None else np.asarray(idx_given[r])
            S = use[use >= 0]
        else:
            S = np.arange(vis)
        W = window_positions(t, n_win) - win_origin
        assert W.min() >= 0, "window reaches before the provided window KV"
        o, lse = core_attention(q[i], [Khat[S], U[W]], tau, eps, t, sink, rope_base)
        res["out"][r] = round_to(o, out_fmt)
        res["lse"][r] = lse
    return res


# ---------------------------------------------------------------------------
# decode: state of uncompressed tokens, one token per step


class DecodeState:
    """Per-sequence decode state ([PT] Heterogeneous KV Cache Layout: a state cache
    holds the window KV and the tail tokens of the block not yet compressed; the
    classical cache holds compressed entries).

    L: tokens seen.  cur: (C, Z) rows of the incomplete block (L % m rows).
    prev: (C, Z) rows of the last complete block (CSA overlap) or None.
    window: the stored window KV of the last n_win-1 or fewer tokens.
    entries: stored compressed entries present before the first step -- any
    object with len() whose [index array] gives float64 rows; entries that
    decode steps create are kept in `new`.
    """

    def __init__(self, *, mode, m, n_win, c, L=0, cur=None, prev=None, window=None, entries=None):
        self.mode, self.m, self.n_win, self.c = mode, m, n_win, c
        self.L = L
        self.cur = cur if cur is not None else (np.zeros((0, c)), np.zeros((0, c)))
        self.prev = prev
        self.window = deque(list(window) if window is not None else [],
                            maxlen=n_win - 1 if n_win > 1 else 0)
        self.base = np.zeros((0, c)) if entries is None else entries
        self.new = []

    @property
    def n_entries(self) -> int:
        return len(self.base) + len(self.new)

    def rows(self, S) -> np.ndarray:
        """Stored entries at the indices S, float64 [len(S), c]."""
        S = np.asarray(S, np.int64)
        nb = len(self.base)
        out = np.zeros((len(S), self.c))
        old = S < nb
        if old.any():
            out[old] = np.asarray(self.base[S[old]], np.float64).reshape(-1, self.c)
        for r in np.nonzero(~old)[0]:
            out[r] = self.new[S[r] - nb]
        return out


def decode_step(st: DecodeState, *, tokC, tokZ, P, q, tau, eps, kv_fmt, out_fmt, k=0,
                qI=None, kI=None, w=None, sink=None, idx_given=None, rope_base=0.0):
    """Append one token and answer its query (the step of a decode loop).

    The token goes to the incomplete block and its normalised KV to the window;
    when its block completes, the block is compressed into a new entry (with the
    previous block as overlap for CSA).  The query at the token's position then
    attends top-k (CSA) or all (HCA) visible entries plus the window.
    kI holds the indexer keys of all entries including a new one.  idx_given makes
    the attention use that selection instead of the oracle's own.  rope_base != 0
    turns the token's window KV and a new entry (both at the token's position t,
    the last token of the entry's block), the query and the output."""
    m, c = st.m, st.c
    t = st.L
    tokC = np.asarray(tokC, np.float64).reshape(c)
    tokZ = np.asarray(tokZ, np.float64).reshape(c)
    curC = np.concatenate([st.cur[0], tokC[None]], 0)
    curZ = np.concatenate([st.cur[1], tokZ[None]], 0)
    u_exact = rope(rmsnorm(tokC, eps), t, rope_base)
    u_t = round_to(u_exact, kv_fmt)
    win_rows = np.array(list(st.window) + [u_t]).reshape(-1, c)
    new_entry = new_bound = None
    if (t + 1) % m == 0:
        if st.mode == "csa":
            pc, pz = (None, None) if st.prev is None else st.prev
            E = compress(curC, curZ, P, m, True, pc, pz)
        else:
            E = compress(curC, curZ, P, m, False)
        e_exact = rope(rmsnorm(E, eps), entry_position(st.n_entries, m), rope_base)
        new_entry = round_to(e_exact, kv_fmt)[0]
        if st.mode == "csa":
            new_bound = compress_error_bound(curC, curZ, P, m, True, pc, pz, eps)[0]
        else:
            new_bound = compress_error_bound(curC, curZ, P, m, False, eps=eps)[0]
        if rope_base:
            new_bound = rope_error_bound(e_exact[0], new_bound)
        st.new.append(new_entry)
        st.prev = (curC, curZ)
        st.cur = (np.zeros((0, c)), np.zeros((0, c)))
    else:
        st.cur = (curC, curZ)
    if st.window.maxlen:
        st.window.append(u_t)
    st.L = t + 1
    vis = int(visible([t], m, st.n_entries)[0])
    res = {"new_entry": new_entry, "new_entry_bound": new_bound, "window_row": u_t, "idx": None,
           "scores": None,
           "window_row_bound": rope_error_bound(u_exact, 0.0) if rope_base else None}
    if st.mode == "csa":
        I = index_scores(np.asarray(qI, np.float64)[None], np.asarray(kI, np.float64)[:vis],
                         np.asarray(w, np.float64)[None], [vis])
        sel = topk(I, [vis], k)[0]
        res["idx"], res["scores"] = sel, I[0]
        use = sel if idx_given is None else np.asarray(idx_given)
        S = use[use >= 0]
    else:
        S = np.arange(vis)
    o, lse = core_attention(q, [st.rows(S), win_rows], tau, eps, t, sink, rope_base)
    res["out"] = round_to(o, out_fmt)
    res["out_exact"] = o
    res["lse"] = lse
    return res


def grouped_output_projection(o, W_g, W_o, z_fmt=None):
    """Grouped output projection ([QB] hybrid attention, the fourth step of CSA:
    with c = 512 a direct projection of all heads back to d is expensive, so the
    n_h heads are split into g groups, each group is projected to an intermediate
    dim d_g, and the groups' results are projected together back to d).

    o [T, n_h, c]; W_g [g, d_g, (n_h/g)*c] (group j's matrix, output x input);
    W_o [d, g*d_g].  Group j takes heads j*n_h/g .. (j+1)*n_h/g - 1, their outputs
    concatenated in head order.  z_fmt: the storage format of the intermediate
    (the GPU keeps it as bf16 between its two products); None keeps it exact.
    Returns (out [T, d], z [T, g*d_g])."""
    o = np.asarray(o, np.float64)
    W_g = np.asarray(W_g, np.float64)
    T, n_h, c = o.shape
    g, d_g, din = W_g.shape
    assert n_h % g == 0 and din == (n_h // g) * c
    x = o.reshape(T, g, din)
    z = np.stack([x[:, j] @ W_g[j].T for j in range(g)], axis=1).reshape(T, g * d_g)
    if z_fmt is not None:
        z = round_to(z, z_fmt)
    return z @ np.asarray(W_o, np.float64).T, z


def matmul_error_bound(a_abs, b_abs_t, n_terms: int) -> np.ndarray:
    """Bound on |fl32(A B^T) - A B^T| for float32 accumulation in any order of
    n_terms products of exact (bf16) operands: gamma(n_terms) * |A| |B|^T."""
    return gamma(n_terms) * (np.asarray(a_abs, np.float64) @ np.asarray(b_abs_t, np.float64).T)


def rope_error_bound(y, bound, rope_dims: int = ROPE_DIMS) -> np.ndarray:
    """Bound on the error of an fp32 rotation of values y (exact: the rotated values;
    the rotation preserves |pair|) whose inputs carry the error bound `bound`: a
    rotated dim mixes both dims of its pair, so it takes both bounds, plus
    2^-20 |pair| for the float32 cos/sin (of an angle reduced in float64) and the
    float32 products.  Dims outside the rotary part keep their bound."""
    y = np.asarray(y, np.float64)
    b = np.array(np.broadcast_to(np.asarray(bound, np.float64), y.shape), copy=True)
    c = y.shape[-1]
    ye, yo = y[..., c - rope_dims::2], y[..., c - rope_dims + 1::2]
    pair = np.sqrt(ye * ye + yo * yo)
    be, bo = b[..., c - rope_dims::2].copy(), b[..., c - rope_dims + 1::2].copy()
    extra = be + bo + 2.0 ** -20 * pair
    b[..., c - rope_dims::2] = extra
    b[..., c - rope_dims + 1::2] = extra
    return b


def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1 - n * u)
