"""Python binding of liblca.so over torch tensors.

Each function has the name and argument order of its C entry point in
include/lca.h, with torch tensors in place of device pointers and format names
("f32", "bf16", "fp8", "mxfp4", "fp8_bf16rope") in place of lca_dtype values.
The binding only marshals arguments: it checks that every tensor is a
contiguous GPU tensor holding at least the bytes the call will touch, passes
its address and the current torch stream, and raises LcaError on a failed
status.  All computation happens in the library's HIP kernels.
"""
import ctypes

import torch

from . import _lib
from ._lib import FMT, MODE, DecodeIO, DecodeLayer, KvPages, check, lib

_ROW_BYTES = {"f32": lambda c: 4 * c, "bf16": lambda c: 2 * c, "fp8": lambda c: c,
              "fp8_bf16rope": lambda c: c + 64, "mxfp4": lambda c: c // 2}


def row_bytes(fmt: str, c: int) -> int:
    return _ROW_BYTES[fmt](c)


def _ptr(t, need_bytes, name, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < need_bytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {need_bytes}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} is not 16-byte aligned")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def kv_pages(block_table, page_tokens, n_pages, B):
    """A paged layout of the compressed-KV cache: block_table [B, max_pages] int32
    (physical page of each logical page), page_tokens tokens per page, n_pages
    pages in the pool (the cache tensor is then [n_pages, page_tokens / m, row])."""
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be an int32 [B, max_pages] tensor")
    pg = KvPages()
    pg.block_table = _ptr(block_table, block_table.numel() * 4, "block_table")
    pg.max_pages = block_table.shape[1]
    pg.page_tokens = page_tokens
    pg.n_pages = n_pages
    return pg


def _cache_rows(N_cap, B, pages, m):
    """Rows the cache tensor must hold: B * N_cap, or the pool's pages x entries."""
    if pages is None:
        return B * N_cap
    return pages.n_pages * (pages.page_tokens // m)


def _pages_ref(pages):
    return None if pages is None else ctypes.byref(pages)


def lca_version() -> int:
    return lib().lca_version()


def lca_kv_row_bytes(kv_fmt: str, c: int) -> int:
    return lib().lca_kv_row_bytes(FMT[kv_fmt], c)


def lca_compress(mode, m, B, n_new, c, C, Z, io_fmt, prevC, prevZ, P, cache, kv_fmt, N_cap,
                 first_entry, eps=1e-6, rope_base=0.0, pages=None, stream=None):
    io_b = row_bytes(io_fmt, c) * B * n_new
    W = 2 * m if mode == "csa" else m
    args = (MODE[mode], m, B, n_new, c, _ptr(C, io_b, "C"), _ptr(Z, io_b, "Z"), FMT[io_fmt],
            _ptr(prevC, row_bytes(io_fmt, c) * B * m, "prevC", True),
            _ptr(prevZ, row_bytes(io_fmt, c) * B * m, "prevZ", True),
            _ptr(P, 4 * W * c, "P"), _ptr(cache, row_bytes(kv_fmt, c) * _cache_rows(N_cap, B, pages, m), "cache"),
            FMT[kv_fmt], N_cap, first_entry, eps, rope_base, _pages_ref(pages), _stream(stream))
    return check("lca_compress", lib().lca_compress(*args))


def lca_rmsnorm_rows(B, n, c, x, x_fmt, y, y_fmt, y_seq_rows, eps=1e-6, pos0=0, rope_base=0.0,
                     stream=None):
    need_y = row_bytes(y_fmt, c) * ((B - 1) * y_seq_rows + n) if B and n else 0
    return check("lca_rmsnorm_rows", lib().lca_rmsnorm_rows(
        B, n, c, _ptr(x, row_bytes(x_fmt, c) * B * n, "x"), FMT[x_fmt], _ptr(y, need_y, "y"),
        FMT[y_fmt], y_seq_rows, eps, pos0, rope_base, _stream(stream)))


def lca_indexer_scores(B, n_q, H_I, d_I, idx_fmt, qI, qI_scale, kI, kI_scale, N_cap, w, q_pos, m,
                       n_entries, scores, stream=None):
    vb = row_bytes(idx_fmt, d_I)
    mx = idx_fmt == "mxfp4"
    return check("lca_indexer_scores", lib().lca_indexer_scores(
        B, n_q, H_I, d_I, FMT[idx_fmt], _ptr(qI, vb * B * n_q * H_I, "qI"),
        _ptr(qI_scale, B * n_q * H_I * d_I // 32, "qI_scale", not mx),
        _ptr(kI, vb * B * N_cap, "kI"), _ptr(kI_scale, B * N_cap * d_I // 32, "kI_scale", not mx),
        N_cap, _ptr(w, 4 * B * n_q * H_I, "w"), _ptr(q_pos, 4 * B * n_q, "q_pos"), m,
        _ptr(n_entries, 4 * B, "n_entries"), _ptr(scores, 4 * B * n_q * N_cap, "scores"),
        _stream(stream)))


def lca_indexer_scores_bf16(B, n_q, H_I, d_I, idx_fmt, qI, qI_scale, kI, kI_scale, N_cap, w, q_pos,
                            m, n_entries, scores, stream=None):
    vb = row_bytes(idx_fmt, d_I)
    mx = idx_fmt == "mxfp4"
    return check("lca_indexer_scores_bf16", lib().lca_indexer_scores_bf16(
        B, n_q, H_I, d_I, FMT[idx_fmt], _ptr(qI, vb * B * n_q * H_I, "qI"),
        _ptr(qI_scale, B * n_q * H_I * d_I // 32, "qI_scale", not mx),
        _ptr(kI, vb * B * N_cap, "kI"), _ptr(kI_scale, B * N_cap * d_I // 32, "kI_scale", not mx),
        N_cap, _ptr(w, 4 * B * n_q * H_I, "w"), _ptr(q_pos, 4 * B * n_q, "q_pos"), m,
        _ptr(n_entries, 4 * B, "n_entries"), _ptr(scores, 2 * B * n_q * N_cap, "scores"),
        _stream(stream)))


def lca_topk_workspace_size(B, n_q, N_cap, k) -> int:
    return lib().lca_topk_workspace_size(B, n_q, N_cap, k)


def lca_topk(B, n_q, N_cap, scores, q_pos, m, n_entries, k, idx, workspace=None, stream=None):
    need = lca_topk_workspace_size(B, n_q, N_cap, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    return check("lca_topk", lib().lca_topk(
        B, n_q, N_cap, _ptr(scores, 4 * B * n_q * N_cap, "scores"), _ptr(q_pos, 4 * B * n_q, "q_pos"),
        m, _ptr(n_entries, 4 * B, "n_entries"), k, _ptr(idx, 4 * B * n_q * k, "idx"),
        _ptr(workspace, need, "workspace", need == 0), need, _stream(stream)))


def lca_topk_bf16(B, n_q, N_cap, scores, q_pos, m, n_entries, k, idx, workspace=None, stream=None):
    need = lca_topk_workspace_size(B, n_q, N_cap, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    return check("lca_topk_bf16", lib().lca_topk_bf16(
        B, n_q, N_cap, _ptr(scores, 2 * B * n_q * N_cap, "scores"), _ptr(q_pos, 4 * B * n_q, "q_pos"),
        m, _ptr(n_entries, 4 * B, "n_entries"), k, _ptr(idx, 4 * B * n_q * k, "idx"),
        _ptr(workspace, need, "workspace", need == 0), need, _stream(stream)))


def lca_sparse_mqa_workspace_size(B, n_q, H, c, kv_fmt, k, N_cap, n_win, dense) -> int:
    return lib().lca_sparse_mqa_workspace_size(B, n_q, H, c, FMT[kv_fmt], k, N_cap, n_win, int(dense))


def lca_sparse_mqa(B, n_q, H, c, q, q_fmt, cache, kv_fmt, N_cap, idx, k, q_pos, m, n_entries, win,
                   W_cap, win_origin, n_win, tau, eps, sink, rope_base, out, out_fmt, lse=None,
                   workspace=None, pages=None, stream=None):
    dense = idx is None
    need = lca_sparse_mqa_workspace_size(B, n_q, H, c, kv_fmt, k, N_cap, n_win, dense)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    kvb = row_bytes(kv_fmt, c)
    return check("lca_sparse_mqa", lib().lca_sparse_mqa(
        B, n_q, H, c, _ptr(q, row_bytes(q_fmt, c) * B * n_q * H, "q"), FMT[q_fmt],
        _ptr(cache, kvb * _cache_rows(N_cap, B, pages, m), "cache"), FMT[kv_fmt], N_cap,
        _ptr(idx, 4 * B * n_q * k, "idx", True), k, _ptr(q_pos, 4 * B * n_q, "q_pos"), m,
        _ptr(n_entries, 4 * B, "n_entries"), _ptr(win, kvb * B * W_cap, "win", n_win == 0), W_cap,
        win_origin, n_win, tau, eps, _ptr(sink, 4 * H, "sink", True), rope_base,
        _ptr(out, row_bytes(out_fmt, c) * B * n_q * H, "out"), FMT[out_fmt],
        _ptr(lse, 4 * B * n_q * H, "lse", True), _ptr(workspace, need, "workspace", need == 0), need,
        _pages_ref(pages), _stream(stream)))


def lca_state_append(mode, m, B, c, n_win, tokC, tokZ, io_fmt, tailC, tailZ, ring, kv_fmt, P, cache,
                     N_cap, n_tokens, q_pos, n_entries, eps=1e-6, rope_base=0.0, pages=None,
                     stream=None):
    iob = row_bytes(io_fmt, c)
    T = 2 * m if mode == "csa" else m
    kvb = row_bytes(kv_fmt, c)
    return check("lca_state_append", lib().lca_state_append(
        MODE[mode], m, B, c, n_win, _ptr(tokC, iob * B, "tokC"), _ptr(tokZ, iob * B, "tokZ"),
        FMT[io_fmt], _ptr(tailC, iob * B * T, "tailC"), _ptr(tailZ, iob * B * T, "tailZ"),
        _ptr(ring, kvb * B * n_win, "ring"), FMT[kv_fmt], _ptr(P, 4 * T * c, "P"),
        _ptr(cache, kvb * _cache_rows(N_cap, B, pages, m), "cache"), N_cap,
        _ptr(n_tokens, 4 * B, "n_tokens"), _ptr(q_pos, 4 * B, "q_pos"),
        _ptr(n_entries, 4 * B, "n_entries"), eps, rope_base, _pages_ref(pages), _stream(stream)))


def lca_grouped_out_proj_workspace_size(T, n_h, c, g, d_g, d) -> int:
    return lib().lca_grouped_out_proj_workspace_size(T, n_h, c, g, d_g, d)


def lca_grouped_out_proj(T, n_h, c, g, d_g, d, o, W_g, W_o, z, out, out_fmt, workspace=None,
                         stream=None):
    need = lca_grouped_out_proj_workspace_size(T, n_h, c, g, d_g, d)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=o.device)
    return check("lca_grouped_out_proj", lib().lca_grouped_out_proj(
        T, n_h, c, g, d_g, d, _ptr(o, 2 * T * n_h * c, "o"),
        _ptr(W_g, 2 * g * d_g * (n_h // g) * c, "W_g"), _ptr(W_o, 2 * d * g * d_g, "W_o"),
        _ptr(z, 2 * T * g * d_g, "z"), _ptr(out, row_bytes(out_fmt, d) * T, "out"), FMT[out_fmt],
        _ptr(workspace, need, "workspace", need == 0), need, _stream(stream)))


class DecodeLayerState:
    """Device buffers of one layer's decode state plus its lca_decode_layer struct."""

    def __init__(self, *, mode, m, B, c, H, n_win, N_cap, io_fmt, kv_fmt, tailC, tailZ, ring, cache,
                 n_tokens, P, sink=None, tau=None, eps=1e-6, k=0, H_I=0, d_I=0, idx_fmt="fp8",
                 kI=None, kI_scale=None, rope_base=0.0, pages=None):
        T = 2 * m if mode == "csa" else m
        iob, kvb = row_bytes(io_fmt, c), row_bytes(kv_fmt, c)
        self.keep = [tailC, tailZ, ring, cache, n_tokens, P, sink, kI, kI_scale, pages]
        s = DecodeLayer()
        s.struct_size = ctypes.sizeof(DecodeLayer)
        s.mode, s.m, s.B, s.c, s.H, s.n_win, s.N_cap = MODE[mode], m, B, c, H, n_win, N_cap
        s.io_dtype, s.kv_dtype = FMT[io_fmt], FMT[kv_fmt]
        s.tailC = _ptr(tailC, iob * B * T, "tailC")
        s.tailZ = _ptr(tailZ, iob * B * T, "tailZ")
        s.ring = _ptr(ring, kvb * B * n_win, "ring")
        s.cache = _ptr(cache, kvb * _cache_rows(N_cap, B, pages, m), "cache")
        s.n_tokens = _ptr(n_tokens, 4 * B, "n_tokens")
        s.P = _ptr(P, 4 * T * c, "P")
        s.sink = _ptr(sink, 4 * H, "sink", True)
        s.tau = c ** -0.5 if tau is None else tau
        s.eps = eps
        s.rope_base = rope_base
        if pages is not None:
            s.pages = pages
        if mode == "csa":
            mx = idx_fmt == "mxfp4"
            s.k, s.H_I, s.d_I, s.idx_dtype = k, H_I, d_I, FMT[idx_fmt]
            s.kI = _ptr(kI, row_bytes(idx_fmt, d_I) * B * N_cap, "kI")
            s.kI_scale = _ptr(kI_scale, B * N_cap * d_I // 32, "kI_scale", not mx)
        self.struct = s
        self.mode, self.B, self.c, self.H, self.k, self.H_I, self.d_I = mode, B, c, H, k, H_I, d_I
        self.io_fmt, self.idx_fmt = io_fmt, idx_fmt
        self.workspace = None

    def workspace_size(self) -> int:
        return lib().lca_decode_workspace_size(ctypes.byref(self.struct))


def _decode_io(layer, tokC, tokZ, q, out, out_fmt, qI=None, qI_scale=None, w=None, lse=None,
               idx_out=None, stage_events=None):
    B, c, H = layer.B, layer.c, layer.H
    iob = row_bytes(layer.io_fmt, c)
    io = DecodeIO()
    io.struct_size = ctypes.sizeof(DecodeIO)
    io.tokC = _ptr(tokC, iob * B, "tokC")
    io.tokZ = _ptr(tokZ, iob * B, "tokZ")
    io.q = _ptr(q, iob * B * H, "q")
    if layer.mode == "csa":
        mx = layer.idx_fmt == "mxfp4"
        io.qI = _ptr(qI, row_bytes(layer.idx_fmt, layer.d_I) * B * layer.H_I, "qI")
        io.qI_scale = _ptr(qI_scale, B * layer.H_I * layer.d_I // 32, "qI_scale", not mx)
        io.w = _ptr(w, 4 * B * layer.H_I, "w")
        io.idx_out = _ptr(idx_out, 4 * B * layer.k, "idx_out", True)
    io.out = _ptr(out, row_bytes(out_fmt, c) * B * H, "out")
    io.lse = _ptr(lse, 4 * B * H, "lse", True)
    io.out_dtype = FMT[out_fmt]
    if stage_events is not None:
        for i, e in enumerate(stage_events):
            io.stage_events[i] = e
    return io


def _decode_workspace(layer, workspace, device):
    need = layer.workspace_size()
    if workspace is None:
        if layer.workspace is None or layer.workspace.numel() < need:
            layer.workspace = torch.empty(need, dtype=torch.uint8, device=device)
        workspace = layer.workspace
    return workspace, need


def lca_decode_step(layer: DecodeLayerState, tokC, tokZ, q, out, out_fmt, qI=None, qI_scale=None,
                    w=None, lse=None, idx_out=None, workspace=None, stream=None, stage_events=None):
    """stage_events: optional sequence of 5 raw hipEvent_t handles (ints or None)."""
    workspace, need = _decode_workspace(layer, workspace, q.device)
    io = _decode_io(layer, tokC, tokZ, q, out, out_fmt, qI, qI_scale, w, lse, idx_out, stage_events)
    return check("lca_decode_step", lib().lca_decode_step(
        ctypes.byref(layer.struct), ctypes.byref(io), _ptr(workspace, need, "workspace"), need,
        _stream(stream)))


def lca_decode_steps(layer: DecodeLayerState, steps, out_fmt, workspace=None, stream=None):
    """n decode steps back to back: steps is a list of dicts with the per-step
    tensors of lca_decode_step (tokC, tokZ, q, out, and qI, qI_scale, w, lse,
    idx_out as the layer needs)."""
    if not steps:
        return check("lca_decode_steps", lib().lca_decode_steps(
            ctypes.byref(layer.struct), None, 0, None, 0, _stream(stream)))
    workspace, need = _decode_workspace(layer, workspace, steps[0]["q"].device)
    arr = (DecodeIO * len(steps))()
    for i, st in enumerate(steps):
        arr[i] = _decode_io(layer, st["tokC"], st["tokZ"], st["q"], st["out"], out_fmt, st.get("qI"),
                            st.get("qI_scale"), st.get("w"), st.get("lse"), st.get("idx_out"))
    return check("lca_decode_steps", lib().lca_decode_steps(
        ctypes.byref(layer.struct), arr, len(steps), _ptr(workspace, need, "workspace"), need,
        _stream(stream)))
