"""ctypes loader of liblca.so and the C declarations of include/lca.h.

The library is loaded from this package directory (built in-tree by
build.py).  A missing library is an error: there is no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# LCA_LIB names another build of the same library (the CPU-only host-sanitizer
# build used by the tests); by default the in-tree liblca.so.
LIB_PATH = os.environ.get("LCA_LIB") or os.path.join(HERE, "liblca.so")

LCA_OK, LCA_ERR_INVALID_ARG, LCA_ERR_UNSUPPORTED, LCA_ERR_WORKSPACE, LCA_ERR_HIP = 0, -1, -2, -3, -4
FMT = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp4": 3, "fp8_bf16rope": 4}
MODE = {"csa": 0, "hca": 1}

c_int, c_float, c_void_p, c_size_t, c_int64 = (ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                               ctypes.c_size_t, ctypes.c_int64)
P = c_void_p  # every tensor pointer is passed as an address


class KvPages(ctypes.Structure):
    _fields_ = [("block_table", P), ("max_pages", c_int), ("page_tokens", c_int), ("n_pages", c_int)]


class _Args(ctypes.Structure):
    """An lca_*_args struct: struct_size is filled in on construction."""

    def __init__(self, **kw):
        super().__init__(**kw)
        self.struct_size = ctypes.sizeof(self)


class CompressArgs(_Args):
    _fields_ = [("struct_size", c_size_t), ("mode", c_int), ("m", c_int), ("B", c_int),
                ("n_new", c_int), ("c", c_int), ("C", P), ("Z", P), ("io_dtype", c_int),
                ("prevC", P), ("prevZ", P), ("P", P), ("cache", P), ("kv_dtype", c_int),
                ("N_cap", c_int), ("first_entry", c_int), ("eps", c_float), ("rope_base", c_float),
                ("pages", KvPages)]


class RmsnormRowsArgs(_Args):
    _fields_ = [("struct_size", c_size_t), ("B", c_int), ("n", c_int), ("c", c_int), ("x", P),
                ("x_dtype", c_int), ("y", P), ("y_dtype", c_int), ("y_seq_rows", c_int),
                ("eps", c_float), ("rope_base", c_float), ("pos0", c_int64)]


class IndexerArgs(_Args):
    _fields_ = [("struct_size", c_size_t), ("B", c_int), ("n_q", c_int), ("H_I", c_int),
                ("d_I", c_int), ("idx_dtype", c_int), ("qI", P), ("qI_scale", P), ("kI", P),
                ("kI_scale", P), ("N_cap", c_int), ("w", P), ("q_pos", P), ("m", c_int),
                ("n_entries", P), ("scores", P), ("score_dtype", c_int)]


class TopkArgs(_Args):
    _fields_ = [("struct_size", c_size_t), ("B", c_int), ("n_q", c_int), ("N_cap", c_int),
                ("scores", P), ("score_dtype", c_int), ("q_pos", P), ("m", c_int),
                ("n_entries", P), ("k", c_int), ("idx", P), ("workspace", P),
                ("workspace_bytes", c_size_t)]


class SparseMqaArgs(_Args):
    _fields_ = [("struct_size", c_size_t), ("B", c_int), ("n_q", c_int), ("H", c_int), ("c", c_int),
                ("q", P), ("q_dtype", c_int), ("cache", P), ("kv_dtype", c_int), ("N_cap", c_int),
                ("idx", P), ("k", c_int), ("q_pos", P), ("m", c_int), ("n_entries", P),
                ("win", P), ("W_cap", c_int), ("win_origin", c_int64), ("n_win", c_int),
                ("tau", c_float), ("eps", c_float), ("sink", P), ("rope_base", c_float),
                ("out", P), ("out_dtype", c_int), ("lse", P), ("workspace", P),
                ("workspace_bytes", c_size_t), ("pages", KvPages), ("split_rows", c_int)]


class GroupedOutProjArgs(_Args):
    _fields_ = [("struct_size", c_size_t), ("T", c_int), ("n_h", c_int), ("c", c_int), ("g", c_int),
                ("d_g", c_int), ("d", c_int), ("o", P), ("W_g", P), ("W_o", P), ("z", P),
                ("out", P), ("out_dtype", c_int), ("workspace", P), ("workspace_bytes", c_size_t)]


class StateAppendArgs(_Args):
    _fields_ = [("struct_size", c_size_t), ("mode", c_int), ("m", c_int), ("B", c_int), ("c", c_int),
                ("n_win", c_int), ("tokC", P), ("tokZ", P), ("io_dtype", c_int), ("tailC", P),
                ("tailZ", P), ("ring", P), ("kv_dtype", c_int), ("P", P), ("cache", P),
                ("N_cap", c_int), ("n_tokens", P), ("q_pos", P), ("n_entries", P),
                ("eps", c_float), ("rope_base", c_float), ("pages", KvPages)]


class DecodeLayer(ctypes.Structure):
    _fields_ = [("struct_size", c_size_t),
                ("mode", c_int), ("m", c_int), ("B", c_int), ("c", c_int), ("H", c_int),
                ("n_win", c_int), ("N_cap", c_int), ("io_dtype", c_int), ("kv_dtype", c_int),
                ("tailC", P), ("tailZ", P), ("ring", P), ("cache", P), ("n_tokens", P), ("P", P),
                ("sink", P), ("tau", c_float), ("eps", c_float),
                ("k", c_int), ("H_I", c_int), ("d_I", c_int), ("idx_dtype", c_int),
                ("kI", P), ("kI_scale", P), ("rope_base", c_float), ("pages", KvPages),
                ("split_rows", c_int), ("sel_hist", P)]


class DecodeIO(ctypes.Structure):
    _fields_ = [("struct_size", c_size_t), ("tokC", P), ("tokZ", P), ("q", P), ("qI", P),
                ("qI_scale", P), ("w", P), ("out", P), ("lse", P), ("out_dtype", c_int),
                ("idx_out", P), ("stage_events", P * 5)]


OP = {"topk": 1, "sparse_mqa": 2, "grouped_out_proj": 3, "decode_step": 4}
_ptr = ctypes.POINTER
SIGNATURES = {
    "lca_version": (c_int, []),
    "lca_status_string": (ctypes.c_char_p, [c_int]),
    "lca_last_error": (ctypes.c_char_p, []),
    "lca_kv_row_bytes": (c_size_t, [c_int, c_int]),
    "lca_workspace_size": (c_int, [c_int, c_void_p, _ptr(c_size_t)]),
    "lca_compress": (c_int, [_ptr(CompressArgs), P]),
    "lca_rmsnorm_rows": (c_int, [_ptr(RmsnormRowsArgs), P]),
    "lca_indexer_scores": (c_int, [_ptr(IndexerArgs), P]),
    "lca_topk": (c_int, [_ptr(TopkArgs), P]),
    "lca_sparse_mqa": (c_int, [_ptr(SparseMqaArgs), P]),
    "lca_grouped_out_proj": (c_int, [_ptr(GroupedOutProjArgs), P]),
    "lca_state_append": (c_int, [_ptr(StateAppendArgs), P]),
    "lca_read_bandwidth_probe": (c_int, [P, c_size_t, P, P]),
    "lca_device_checks": (c_int, [P, c_int]),
    "lca_decode_step": (c_int, [_ptr(DecodeLayer), _ptr(DecodeIO), P, c_size_t, P]),
    "lca_decode_steps": (c_int, [_ptr(DecodeLayer), _ptr(DecodeIO), c_int, P, c_size_t, P]),
    "lca_decode_step_static": (c_int, [_ptr(DecodeLayer), _ptr(DecodeIO), P]),
}
LCA_STATIC_SCRATCH_BYTES = 96 << 20  # include/lca.h

_LIB = None


class LcaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """The loaded liblca.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_attention_14_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def check(fn_name, status):
    if status != LCA_OK:
        raise LcaError(fn_name, status, lib().lca_last_error().decode())
    return status
