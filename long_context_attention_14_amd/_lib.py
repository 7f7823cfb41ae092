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


class DecodeLayer(ctypes.Structure):
    _fields_ = [("struct_size", c_size_t),
                ("mode", c_int), ("m", c_int), ("B", c_int), ("c", c_int), ("H", c_int),
                ("n_win", c_int), ("N_cap", c_int), ("io_dtype", c_int), ("kv_dtype", c_int),
                ("tailC", P), ("tailZ", P), ("ring", P), ("cache", P), ("n_tokens", P), ("P", P),
                ("sink", P), ("tau", c_float), ("eps", c_float),
                ("k", c_int), ("H_I", c_int), ("d_I", c_int), ("idx_dtype", c_int),
                ("kI", P), ("kI_scale", P), ("rope_base", c_float), ("pages", KvPages)]


class DecodeIO(ctypes.Structure):
    _fields_ = [("struct_size", c_size_t), ("tokC", P), ("tokZ", P), ("q", P), ("qI", P),
                ("qI_scale", P), ("w", P), ("out", P), ("lse", P), ("out_dtype", c_int),
                ("idx_out", P), ("stage_events", P * 5)]


SIGNATURES = {
    "lca_version": (c_int, []),
    "lca_status_string": (ctypes.c_char_p, [c_int]),
    "lca_last_error": (ctypes.c_char_p, []),
    "lca_kv_row_bytes": (c_size_t, [c_int, c_int]),
    "lca_compress": (c_int, [c_int, c_int, c_int, c_int, c_int, P, P, c_int, P, P, P, P, c_int,
                             c_int, c_int, c_float, c_float, ctypes.POINTER(KvPages), P]),
    "lca_rmsnorm_rows": (c_int, [c_int, c_int, c_int, P, c_int, P, c_int, c_int, c_float, c_int64,
                                 c_float, P]),
    "lca_indexer_scores": (c_int, [c_int, c_int, c_int, c_int, c_int, P, P, P, P, c_int, P, P,
                                   c_int, P, P, P]),
    "lca_indexer_scores_bf16": (c_int, [c_int, c_int, c_int, c_int, c_int, P, P, P, P, c_int, P, P,
                                        c_int, P, P, P]),
    "lca_topk_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "lca_topk": (c_int, [c_int, c_int, c_int, P, P, c_int, P, c_int, P, P, c_size_t, P]),
    "lca_topk_bf16": (c_int, [c_int, c_int, c_int, P, P, c_int, P, c_int, P, P, c_size_t, P]),
    "lca_sparse_mqa_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                                 c_int, c_int]),
    "lca_sparse_mqa": (c_int, [c_int, c_int, c_int, c_int, P, c_int, P, c_int, c_int, P, c_int, P,
                               c_int, P, P, c_int, c_int64, c_int, c_float, c_float, P, c_float, P,
                               c_int, P, P, c_size_t, ctypes.POINTER(KvPages), P]),
    "lca_state_append": (c_int, [c_int, c_int, c_int, c_int, c_int, P, P, c_int, P, P, P, c_int, P,
                                 P, c_int, P, P, P, c_float, c_float, ctypes.POINTER(KvPages), P]),
    "lca_grouped_out_proj_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "lca_grouped_out_proj": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, P, P, P, P, P, c_int,
                                     P, c_size_t, P]),
    "lca_decode_workspace_size": (c_size_t, [ctypes.POINTER(DecodeLayer)]),
    "lca_decode_step": (c_int, [ctypes.POINTER(DecodeLayer), ctypes.POINTER(DecodeIO), P, c_size_t,
                                P]),
    "lca_decode_steps": (c_int, [ctypes.POINTER(DecodeLayer), ctypes.POINTER(DecodeIO), c_int, P,
                                 c_size_t, P]),
    "lca_decode_step_static": (c_int, [ctypes.POINTER(DecodeLayer), ctypes.POINTER(DecodeIO), P]),
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
