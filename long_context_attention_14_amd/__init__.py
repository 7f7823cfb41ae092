"""MI355X-native (gfx950) CSA/HCA long-context attention: the compressor,
lightning indexer, top-k selection, sparse/dense multi-query attention with a
sliding-window branch, and decode-time state handling, as hand-written HIP
kernels behind a C ABI (include/lca.h, liblca.so).  `ops` is the torch-tensor
binding of that ABI.
"""
from ._lib import LIB_PATH, LcaError, lib  # noqa: F401

__all__ = ["LIB_PATH", "LcaError", "lib"]
