"""Drivers that run whole layers of the path on the GPU through the C ABI.

`PrefillLayer` runs a CSA prefill chunk: compressor -> window KV -> indexer ->
top-k -> sparse MQA with the window branch.  `DecodeLayer` runs decode steps of
a CSA or HCA layer with lca_decode_step.  Inputs are the byte arrays of the
seeded synthetic workloads (numpy), uploaded once; every computation happens in
the library's kernels.
"""
import numpy as np
import torch

from . import ops


def _dev(a, device):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def _empty_bytes(n, device):
    return torch.empty(max(1, int(n)), dtype=torch.uint8, device=device)


# paged compressed-KV cache: host-side layout helpers (setup and read-back only)

def to_pool(cache, epp, block_table, n_pages):
    """cache [B, N_cap, row] bytes -> pool [n_pages, epp, row] with logical page j
    of sequence b at physical page block_table[b, j] (unused pool rows zero)."""
    B, N_cap, rb = cache.shape
    max_pages = block_table.shape[1]
    padded = np.zeros((B, max_pages * epp, rb), cache.dtype)
    padded[:, :N_cap] = cache
    pool = np.zeros((n_pages, epp, rb), cache.dtype)
    pool[block_table.reshape(-1)] = padded.reshape(B * max_pages, epp, rb)
    return pool


def from_pool(pool, block_table, N_cap):
    """The logical [B, N_cap, row] view of a pool."""
    B, max_pages = block_table.shape
    epp, rb = pool.shape[1], pool.shape[2]
    return pool[block_table.reshape(-1)].reshape(B, max_pages * epp, rb)[:, :N_cap]


class Paged:
    """A block table over 128-token pages (lcm of the CSA and HCA rates) and its pool
    size: n_pages = B * max_pages + extra unused pages."""

    def __init__(self, B, N_cap, m, page_tokens=128, extra=3, seed=0):
        from synth import gen
        self.page_tokens, self.epp = page_tokens, page_tokens // m
        self.max_pages = -(-N_cap // self.epp)
        self.n_pages = B * self.max_pages + extra
        self.table = gen.page_table(B, self.max_pages, self.n_pages, seed)

    def struct(self, device):
        self.table_dev = torch.from_numpy(self.table).to(device)
        return ops.kv_pages(self.table_dev, self.page_tokens, self.n_pages, self.table.shape[0])


class PrefillLayer:
    """CSA prefill of n_new tokens after a prefix of ctx tokens (one chunk)."""

    def __init__(self, cfg, d, device="cuda", paged=None):
        self.cfg, self.device = cfg, device
        B, c, m, n = cfg.B, cfg.c, cfg.m, cfg.n_new
        self.B, self.c, self.m, self.n = B, c, m, n
        self.N_cap = d["n_cap"]
        self.n_prefix = d["n_prefix"]
        self.pos0 = d["pos0"]
        g = lambda name: _dev(d[name], device) if name in d else None  # noqa: E731
        self.C, self.Z, self.P, self.q, self.w = g("C"), g("Z"), g("P"), g("q"), g("w")
        self.prevC, self.prevZ = g("prevC"), g("prevZ")
        self.cache0 = d["cache"]
        self.paged, self.pages = None, None
        if paged is not None:     # the compressed cache as a pool of pages (paged: dict(seed=...))
            rb0 = ops.row_bytes(cfg.kv_dtype, c)
            self.paged = Paged(B, self.N_cap, m, seed=paged.get("seed", 0))
            pool = to_pool(np.ascontiguousarray(d["cache"]).view(np.uint8).reshape(B, self.N_cap, rb0),
                           self.paged.epp, self.paged.table, self.paged.n_pages)
            self.cache = _dev(pool, device)
            self.pages = self.paged.struct(device)
        else:
            self.cache = g("cache")
        self.kI, self.qI = g("kI"), g("qI")
        self.kI_scale, self.qI_scale = g("kI_scale"), g("qI_scale")
        self.n_pre_win = 0 if "win_prefix" not in d else d["win_prefix"].shape[1]
        self.W_cap = self.n_pre_win + n
        rb = ops.row_bytes(cfg.kv_dtype, c)
        self.win = torch.zeros(B * self.W_cap * rb, dtype=torch.uint8, device=device)
        if self.n_pre_win:
            wp = d["win_prefix"].view(np.uint8).reshape(B, self.n_pre_win, rb)
            full = np.zeros((B, self.W_cap, rb), np.uint8)
            full[:, : self.n_pre_win] = wp
            self.win.copy_(torch.from_numpy(full.reshape(-1)).to(device))
        self.q_pos = (self.pos0 + torch.arange(n, dtype=torch.int32, device=device)).repeat(B, 1).contiguous()
        self.n_entries = torch.full((B,), self.N_cap, dtype=torch.int32, device=device)
        self.scores = torch.empty((B, n, self.N_cap), dtype=torch.float32, device=device)
        self.idx = torch.empty((B, n, cfg.k), dtype=torch.int32, device=device)
        out_t = torch.float32 if cfg.io_dtype == "f32" else torch.bfloat16
        self.out = torch.empty((B, n, cfg.H, c), dtype=out_t, device=device)
        self.lse = torch.empty((B, n, cfg.H), dtype=torch.float32, device=device)
        self.ws_topk = _empty_bytes(ops.topk_workspace_size(B, n, self.N_cap, cfg.k), device)
        self.ws_mqa = _empty_bytes(ops.sparse_mqa_workspace_size(
            B, n, cfg.H, c, cfg.kv_dtype, cfg.k, self.N_cap, cfg.n_win, False), device)

    def compress(self):
        cfg = self.cfg
        ops.lca_compress("csa", self.m, self.B, self.n, self.c, self.C, self.Z, cfg.io_dtype,
                         self.prevC, self.prevZ, self.P, self.cache, cfg.kv_dtype, self.N_cap,
                         self.n_prefix, cfg.eps, cfg.rope_base, pages=self.pages)

    def window_kv(self):
        cfg = self.cfg
        rb = ops.row_bytes(cfg.kv_dtype, self.c)
        y = self.win[self.n_pre_win * rb:]
        ops.lca_rmsnorm_rows(self.B, self.n, self.c, self.C, cfg.io_dtype, y, cfg.kv_dtype, self.W_cap,
                             cfg.eps, self.pos0, cfg.rope_base)

    def indexer(self):
        cfg = self.cfg
        ops.lca_indexer_scores(self.B, self.n, cfg.H_I, cfg.d_I, cfg.idx_dtype, self.qI, self.qI_scale,
                               self.kI, self.kI_scale, self.N_cap, self.w, self.q_pos, self.m,
                               self.n_entries, self.scores)

    def topk(self):
        ops.lca_topk(self.B, self.n, self.N_cap, self.scores, self.q_pos, self.m, self.n_entries,
                     self.cfg.k, self.idx, self.ws_topk)

    # the BF16-score selector: bf16 scores and a top-k over them (own buffers)
    def indexer_bf16(self):
        cfg = self.cfg
        if not hasattr(self, "scores16"):
            self.scores16 = torch.empty((self.B, self.n, self.N_cap), dtype=torch.int16,
                                        device=self.device)
            self.idx16 = torch.empty_like(self.idx)
        ops.lca_indexer_scores(self.B, self.n, cfg.H_I, cfg.d_I, cfg.idx_dtype, self.qI,
                               self.qI_scale, self.kI, self.kI_scale, self.N_cap, self.w,
                               self.q_pos, self.m, self.n_entries, self.scores16, score_fmt="bf16")

    def topk_bf16(self):
        ops.lca_topk(self.B, self.n, self.N_cap, self.scores16, self.q_pos, self.m,
                     self.n_entries, self.cfg.k, self.idx16, self.ws_topk, score_fmt="bf16")

    def attention(self):
        cfg = self.cfg
        ops.lca_sparse_mqa(self.B, self.n, cfg.H, self.c, self.q, cfg.io_dtype, self.cache,
                           cfg.kv_dtype, self.N_cap, self.idx, cfg.k, self.q_pos, self.m,
                           self.n_entries, self.win, self.W_cap, self.pos0 - self.n_pre_win,
                           cfg.n_win, cfg.tau, cfg.eps, None, cfg.rope_base, self.out, cfg.io_dtype,
                           self.lse, self.ws_mqa, pages=self.pages)

    def run(self):
        self.compress()
        self.window_kv()
        self.indexer()
        self.topk()
        self.attention()

    def logical_cache(self):
        """The compressed cache as [B, N_cap, row] bytes on the host."""
        rb = ops.row_bytes(self.cfg.kv_dtype, self.c)
        raw = self.cache.cpu().numpy().view(np.uint8)
        if self.paged is None:
            return raw.reshape(self.B, self.N_cap, rb)
        return from_pool(raw.reshape(self.paged.n_pages, self.paged.epp, rb), self.paged.table, self.N_cap)


class DecodeLayer:
    """One CSA ("C") or HCA ("H") layer's decode state on the GPU."""

    def __init__(self, cfg, d, device="cuda", sink=None, paged=None, split_rows=0, sel_hist=True):
        self.cfg, self.device, self.d = cfg, device, d
        kind = d["kind"]
        self.mode = "csa" if kind == "C" else "hca"
        B, c, m = cfg.B, cfg.c, d["m"]
        self.B, self.c, self.m = B, c, m
        self.N_cap = d["n_cap"]
        g = lambda name: _dev(d[name], device) if name in d else None  # noqa: E731
        self.ring = g("ring")
        self.paged, pages = None, None
        if paged is not None:     # the compressed cache as a pool of pages (paged: dict(seed=...))
            rb0 = ops.row_bytes(cfg.kv_dtype, c)
            self.paged = Paged(B, self.N_cap, m, seed=paged.get("seed", 0))
            pool = to_pool(np.ascontiguousarray(d["cache"]).view(np.uint8).reshape(B, self.N_cap, rb0),
                           self.paged.epp, self.paged.table, self.paged.n_pages)
            self.cache = _dev(pool, device)
            pages = self.paged.struct(device)
        else:
            self.cache = g("cache")
        self.tailC, self.tailZ = g("tailC"), g("tailZ")
        self.n_tokens = g("n_tokens")
        self.P = g("P")
        self.tokC, self.tokZ, self.q = g("tokC"), g("tokZ"), g("q")
        self.kI, self.kI_scale = g("kI"), g("kI_scale")
        self.qI, self.qI_scale, self.w = g("qI"), g("qI_scale"), g("w")
        self.sink = None if sink is None else torch.as_tensor(sink, dtype=torch.float32, device=device)
        out_t = torch.float32 if cfg.io_dtype == "f32" else torch.bfloat16
        self.out = torch.empty((B, cfg.H, c), dtype=out_t, device=device)
        self.lse = torch.empty((B, cfg.H), dtype=torch.float32, device=device)
        self.idx = torch.empty((B, max(1, cfg.k)), dtype=torch.int32, device=device)
        # CSA: the fused selection's histogram kept zero-filled with the state
        # (sel_hist=False: the step clears one in its workspace instead)
        self.sel_hist = (torch.zeros(B * ops.SEL_HIST_BINS, dtype=torch.int32, device=device)
                         if sel_hist and self.mode == "csa" else None)
        self.state = ops.DecodeLayerState(
            mode=self.mode, m=m, B=B, c=c, H=cfg.H, n_win=cfg.n_win, N_cap=self.N_cap,
            io_fmt=cfg.io_dtype, kv_fmt=cfg.kv_dtype, tailC=self.tailC, tailZ=self.tailZ,
            ring=self.ring, cache=self.cache, n_tokens=self.n_tokens, P=self.P, sink=self.sink,
            tau=cfg.tau, eps=cfg.eps, k=cfg.k, H_I=cfg.H_I, d_I=cfg.d_I, idx_fmt=cfg.idx_dtype,
            kI=self.kI, kI_scale=self.kI_scale, rope_base=cfg.rope_base, pages=pages,
            split_rows=split_rows, sel_hist=self.sel_hist)
        self.workspace = _empty_bytes(self.state.workspace_size(), device)

    def logical_cache(self):
        """The compressed cache as [B, N_cap, row] bytes on the host."""
        rb = ops.row_bytes(self.cfg.kv_dtype, self.c)
        raw = self.cache.cpu().numpy().view(np.uint8)
        if self.paged is None:
            return raw.reshape(self.B, self.N_cap, rb)
        return from_pool(raw.reshape(self.paged.n_pages, self.paged.epp, rb), self.paged.table, self.N_cap)

    def step(self, stream=None):
        csa = self.mode == "csa"
        ops.lca_decode_step(self.state, self.tokC, self.tokZ, self.q, self.out, self.cfg.io_dtype,
                            qI=self.qI if csa else None, qI_scale=self.qI_scale if csa else None,
                            w=self.w if csa else None, lse=self.lse,
                            idx_out=self.idx if csa else None, workspace=self.workspace,
                            stream=stream)
