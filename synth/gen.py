"""Seeded synthetic inputs, in the byte formats the path stores.

Every random tensor is drawn from numpy's PCG64 with a SeedSequence keyed by
(seed, tensor name, sequence, 4096-row block), so any slice can be drawn again
without drawing the rest.  Distributions (from the workload descriptions):

* "normal":  N(0,1) per element (KV candidates C, gate logits Z, queries,
  indexer queries and keys);
* "bias":    N(0, 0.1^2) per element (the learnable positional bias P);
* "uniform": U(0,1) per element (indexer head weights w);
* "sphere":  rows uniform on the sphere of radius sqrt(c).  A Gaussian row
  divided by its root-mean-square lies exactly there, so this is the
  distribution of a stored, already RMS-normalised KV row.

Decode state conventions (shared with the library header): a sequence whose
step appends the token at position p = L-1 holds, before the step, the tail
rows of the uncompressed tokens (CSA: the previous complete block plus the
current partial block, two-block ring, row ((p // m) % 2) * m + p % m; HCA:
the current partial block, row p % m), the window ring of normalised KV
(slot p % n_win) and the count of tokens L-1.
"""
from concurrent.futures import ThreadPoolExecutor
import os
import zlib

import numpy as np

from . import encode as enc
from .configs import LayerConfig

BLOCK_ROWS = 4096
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        n = max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = ThreadPoolExecutor(n)
    return _POOL


def _key(seed: int, name: str, b: int, blk: int):
    return np.random.SeedSequence([seed, zlib.crc32(name.encode()), b, blk])


def _draw_block(seed, name, b, blk, rows, c, dist):
    rng = np.random.Generator(np.random.PCG64(_key(seed, name, b, blk)))
    if dist == "uniform":
        return rng.random((rows, c), dtype=np.float32)
    x = rng.standard_normal((rows, c), dtype=np.float32)
    if dist == "bias":
        x *= np.float32(0.1)
    elif dist == "sphere":
        nrm = np.sqrt(np.einsum("ij,ij->i", x.astype(np.float64), x.astype(np.float64)))
        x = (x.astype(np.float64) * (np.sqrt(c) / nrm)[:, None]).astype(np.float32)
    return x


def draw_rows(seed: int, name: str, b: int, n_rows: int, c: int, dist: str,
              row0: int = 0) -> np.ndarray:
    """Rows [row0, row0+n_rows) of tensor `name` for sequence b, float32."""
    if n_rows == 0:
        return np.zeros((0, c), np.float32)
    first, last = row0 // BLOCK_ROWS, (row0 + n_rows - 1) // BLOCK_ROWS
    blocks = [_draw_block(seed, name, b, blk, BLOCK_ROWS, c, dist) for blk in range(first, last + 1)]
    allr = np.concatenate(blocks, 0) if len(blocks) > 1 else blocks[0]
    off = row0 - first * BLOCK_ROWS
    return allr[off: off + n_rows]


def draw_encoded(seed, name, B, n_rows, c, dist, fmt, n_valid=None):
    """[B, n_rows, ...] encoded rows; rows >= n_valid[b] are zero bytes.

    fmt "mxfp4" returns (packed, scales)."""
    n_valid = [n_rows] * B if n_valid is None else list(n_valid)

    def one(args):
        b, blk = args
        r0 = blk * BLOCK_ROWS
        rows = min(BLOCK_ROWS, n_rows - r0)
        x = _draw_block(seed, name, b, blk, BLOCK_ROWS, c, dist)[:rows]
        nv = max(0, min(rows, n_valid[b] - r0))
        if nv < rows:
            x = x.copy()
            x[nv:] = 0
        return b, r0, rows, (enc.to_mxfp4(x) if fmt == "mxfp4" else enc.encode(x, fmt))

    nblk = (n_rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    jobs = [(b, blk) for b in range(B) for blk in range(nblk)]
    outs = list(_pool().map(one, jobs))
    if fmt == "mxfp4":
        packed = np.zeros((B, n_rows, c // 2), np.uint8)
        scales = np.zeros((B, n_rows, c // 32), np.uint8)
        for b, r0, rows, (p, s) in outs:
            packed[b, r0:r0 + rows] = p
            scales[b, r0:r0 + rows] = s
        return packed, scales
    sample = outs[0][3]
    out = np.zeros((B, n_rows) + sample.shape[1:], sample.dtype)
    for b, r0, rows, e in outs:
        out[b, r0:r0 + rows] = e
    return out


def draw_small(seed, name, shape, dist, fmt):
    """A small tensor of any shape whose last dim is the feature dim."""
    shape = tuple(shape)
    lead = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    x = draw_rows(seed, name, 0, lead, shape[-1], dist).reshape(shape)
    if fmt == "mxfp4":
        return enc.to_mxfp4(x)
    return enc.encode(x, fmt)


# ---------------------------------------------------------------------------
# workloads

def tails(cfg: LayerConfig, m: int, tag: str = "tail") -> np.ndarray:
    """Per-sequence tail length T_b in [0, m-1] (tokens after the last full block)."""
    rng = np.random.Generator(np.random.PCG64(_key(cfg.seed, tag, 0, 0)))
    return rng.integers(0, m, size=cfg.B).astype(np.int64)


def decode_layer(cfg: LayerConfig, kind: str, m: int, lengths: np.ndarray, layer: int = 0,
                 extra_entries: int = 0) -> dict:
    """Inputs of one decode step of one layer.  kind "C" (CSA) or "H" (HCA).

    lengths[b] = L_b, the token count after the step (query at position L_b-1).
    extra_entries leaves room in the cache for further steps.
    """
    B, c, s = cfg.B, cfg.c, cfg.seed
    pre = lengths - 1
    n_pre = pre // m
    n_cap = int((lengths.max() + (extra_entries + 1) * m) // m)
    p = f"L{layer}{kind}."
    kvf = cfg.kv_dtype
    d = {
        "kind": kind, "m": m, "lengths": lengths.astype(np.int64), "n_cap": n_cap,
        "n_tokens": pre.astype(np.int32),
        "cache": draw_encoded(s, p + "cache", B, n_cap, c, "sphere", kvf, n_valid=n_pre),
        "ring": draw_encoded(s, p + "ring", B, cfg.n_win, c, "sphere", kvf),
        "tailC": draw_encoded(s, p + "tailC", B, 2 * m if kind == "C" else m, c, "normal", cfg.io_dtype),
        "tailZ": draw_encoded(s, p + "tailZ", B, 2 * m if kind == "C" else m, c, "normal", cfg.io_dtype),
        "P": draw_small(s, p + "P", (2 * m if kind == "C" else m, c), "bias", "f32"),
        "tokC": draw_small(s, p + "tokC", (B, c), "normal", cfg.io_dtype),
        "tokZ": draw_small(s, p + "tokZ", (B, c), "normal", cfg.io_dtype),
        "q": draw_small(s, p + "q", (B, cfg.H, c), "normal", cfg.io_dtype),
    }
    if kind == "C":
        if cfg.idx_dtype == "mxfp4":
            d["kI"], d["kI_scale"] = draw_encoded(s, p + "kI", B, n_cap, cfg.d_I, "normal", "mxfp4")
            d["qI"], d["qI_scale"] = draw_small(s, p + "qI", (B, cfg.H_I, cfg.d_I), "normal", "mxfp4")
        else:
            d["kI"] = draw_encoded(s, p + "kI", B, n_cap, cfg.d_I, "normal", cfg.idx_dtype)
            d["qI"] = draw_small(s, p + "qI", (B, cfg.H_I, cfg.d_I), "normal", cfg.idx_dtype)
        d["w"] = draw_small(s, p + "w", (B, cfg.H_I), "uniform", "f32")
    return d


def decode_inputs(cfg: LayerConfig, extra_entries: int = 0) -> dict:
    """One decode step for a single-kind config (csa_decode / hca_decode)."""
    T = tails(cfg, cfg.m)
    lengths = cfg.ctx + T
    kind = "C" if cfg.kind == "csa_decode" else "H"
    return decode_layer(cfg, kind, cfg.m, lengths, 0, extra_entries)


def hybrid_lengths(cfg: LayerConfig) -> np.ndarray:
    """One L_b = ctx + U{0..m'-1} per sequence, shared by every layer."""
    return cfg.ctx + tails(cfg, cfg.m_hca, "hybrid_len")


def hybrid_inputs(cfg: LayerConfig, extra_entries: int = 0):
    lengths = hybrid_lengths(cfg)
    return [decode_layer(cfg, kind, cfg.m if kind == "C" else cfg.m_hca, lengths, i, extra_entries)
            for i, kind in enumerate(cfg.layers)]


def prefill_inputs(cfg: LayerConfig) -> dict:
    """CSA prefill of n_new tokens after a prefix of ctx tokens (ctx % m == 0)."""
    B, c, m, s, n = cfg.B, cfg.c, cfg.m, cfg.seed, cfg.n_new
    assert cfg.ctx % m == 0 and n % m == 0
    n_prefix = cfg.ctx // m
    n_cap = (cfg.ctx + n) // m
    io, kvf = cfg.io_dtype, cfg.kv_dtype
    d = {
        "n_prefix": n_prefix, "n_cap": n_cap, "pos0": cfg.ctx,
        "C": draw_encoded(s, "C", B, n, c, "normal", io),
        "Z": draw_encoded(s, "Z", B, n, c, "normal", io),
        "P": draw_small(s, "P", (2 * m, c), "bias", "f32"),
        "cache": draw_encoded(s, "cache", B, n_cap, c, "sphere", kvf, n_valid=[n_prefix] * B),
        "q": draw_encoded(s, "q", B, n, cfg.H * c, "normal", io).reshape(B, n, cfg.H, -1),
        "w": draw_encoded(s, "w", B, n, cfg.H_I, "uniform", "f32"),
    }
    if cfg.ctx > 0:
        d["prevC"] = draw_encoded(s, "prevC", B, m, c, "normal", io)
        d["prevZ"] = draw_encoded(s, "prevZ", B, m, c, "normal", io)
        d["win_prefix"] = draw_encoded(s, "win_prefix", B, cfg.n_win - 1, c, "sphere", kvf)
    if cfg.idx_dtype == "mxfp4":
        d["kI"], d["kI_scale"] = draw_encoded(s, "kI", B, n_cap, cfg.d_I, "normal", "mxfp4")
        qp, qs = draw_encoded(s, "qI", B, n, cfg.H_I * cfg.d_I, "normal", "mxfp4")
        d["qI"] = qp.reshape(B, n, cfg.H_I, -1)
        d["qI_scale"] = qs.reshape(B, n, cfg.H_I, -1)
    else:
        d["kI"] = draw_encoded(s, "kI", B, n_cap, cfg.d_I, "normal", cfg.idx_dtype)
        d["qI"] = draw_encoded(s, "qI", B, n, cfg.H_I * cfg.d_I, "normal",
                               cfg.idx_dtype).reshape(B, n, cfg.H_I, -1)
    return d


def page_table(B: int, max_pages: int, n_pages: int, seed: int = 0) -> np.ndarray:
    """A block table for a paged cache: [B, max_pages] int32 of distinct physical
    pages drawn at random from a pool of n_pages >= B * max_pages (so that
    sequences interleave in the pool and logical order never matches physical
    order)."""
    assert n_pages >= B * max_pages
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x9A6E])))
    return rng.permutation(n_pages)[: B * max_pages].reshape(B, max_pages).astype(np.int32)
