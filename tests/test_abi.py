"""The C ABI library: it loads without a GPU, exports every function that
include/lca.h declares, and rejects bad arguments with a status code before any
HIP call (so these run on a CPU-only machine)."""
import ctypes
import os
import re

import pytest

from long_context_attention_14_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lca.h")
FAKE = 0x1000  # never dereferenced: every call below fails validation first
F = _lib.FMT


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lca_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("liblca.so is not built; run __graft_entry__.build()")
    return _lib.lib()


def ref(x):
    return ctypes.byref(x)


def ws_size(L, op, args):
    n = ctypes.c_size_t(12345)
    st = L.lca_workspace_size(_lib.OP[op], ref(args), ref(n))
    return st, n.value


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), f"{n} declared in lca.h but not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_version_and_strings(L):
    assert L.lca_version() == 5
    for st in (0, -1, -2, -3, -4):
        assert L.lca_status_string(st)
    assert L.lca_status_string(7) == b"unknown status"
    assert L.lca_kv_row_bytes(F["bf16"], 512) == 1024
    assert L.lca_kv_row_bytes(F["fp8_bf16rope"], 512) == 576
    assert L.lca_kv_row_bytes(F["f32"], 128) == 512
    assert L.lca_kv_row_bytes(99, 128) == 0


def _valid_args():
    """One valid argument struct per struct-taking entry point (tensor pointers
    fake; each call is made invalid before use)."""
    return {
        "lca_compress": _lib.CompressArgs(mode=0, m=4, B=1, n_new=8, c=128, C=FAKE, Z=FAKE, io_dtype=0,
                                          P=FAKE, cache=FAKE, kv_dtype=0, N_cap=2, eps=1e-6),
        "lca_rmsnorm_rows": _lib.RmsnormRowsArgs(B=1, n=4, c=128, x=FAKE, x_dtype=0, y=FAKE, y_dtype=0,
                                                 y_seq_rows=4, eps=1e-6),
        "lca_indexer_scores": _lib.IndexerArgs(B=1, n_q=1, H_I=64, d_I=128, idx_dtype=F["fp8"], qI=FAKE,
                                               kI=FAKE, N_cap=8, w=FAKE, q_pos=FAKE, m=4, n_entries=FAKE,
                                               scores=FAKE, score_dtype=F["f32"]),
        "lca_topk": _lib.TopkArgs(B=1, n_q=1, N_cap=100, scores=FAKE, score_dtype=F["f32"], q_pos=FAKE, m=4,
                                  n_entries=FAKE, k=32, idx=FAKE),
        "lca_sparse_mqa": _lib.SparseMqaArgs(B=1, n_q=1, H=64, c=512, q=FAKE, q_dtype=F["bf16"], cache=FAKE,
                                             kv_dtype=F["bf16"], N_cap=1024, idx=FAKE, k=1024, q_pos=FAKE,
                                             m=4, n_entries=FAKE, win=FAKE, W_cap=128, n_win=128, tau=0.04,
                                             eps=1e-6, out=FAKE, out_dtype=F["bf16"]),
        "lca_grouped_out_proj": _lib.GroupedOutProjArgs(T=16, n_h=64, c=512, g=8, d_g=1024, d=7168, o=FAKE,
                                                        W_g=FAKE, W_o=FAKE, z=FAKE, out=FAKE,
                                                        out_dtype=F["bf16"]),
        "lca_state_append": _lib.StateAppendArgs(mode=0, m=4, B=1, c=512, n_win=128, tokC=FAKE, tokZ=FAKE,
                                                 io_dtype=F["bf16"], tailC=FAKE, tailZ=FAKE, ring=FAKE,
                                                 kv_dtype=F["bf16"], P=FAKE, cache=FAKE, N_cap=8,
                                                 n_tokens=FAKE, q_pos=FAKE, n_entries=FAKE, eps=1e-6),
    }


def test_every_struct_call_rejects_a_wrong_struct_size(L):
    """A caller built against another layout is rejected, never misread; a NULL
    argument struct too."""
    for name, a in _valid_args().items():
        good = a.struct_size
        assert good == ctypes.sizeof(a)
        for bad in (0, good - 8, good + 8):
            a.struct_size = bad
            assert getattr(L, name)(ref(a), None) == _lib.LCA_ERR_INVALID_ARG, (name, bad)
            assert b"struct_size" in L.lca_last_error(), name
        a.struct_size = good
        assert getattr(L, name)(None, None) == _lib.LCA_ERR_INVALID_ARG, name
    lay = _decode_layer()
    io = _lib.DecodeIO()
    io.struct_size = ctypes.sizeof(_lib.DecodeIO) - 8
    st, need = ws_size(L, "decode_step", lay)
    assert st == _lib.LCA_OK
    assert L.lca_decode_step(ref(lay), ref(io), FAKE, need, None) == _lib.LCA_ERR_INVALID_ARG
    assert L.lca_decode_step_static(ref(lay), ref(io), None) == _lib.LCA_ERR_INVALID_ARG
    lay.struct_size += 8
    assert ws_size(L, "decode_step", lay) == (_lib.LCA_ERR_INVALID_ARG, 0)


def test_compress_validation(L):
    def call(**kw):
        a = _valid_args()["lca_compress"]
        for k_, v in kw.items():
            setattr(a, k_, v)
        return L.lca_compress(ref(a), None)

    assert call(mode=5) == _lib.LCA_ERR_INVALID_ARG
    assert call(n_new=6) == _lib.LCA_ERR_INVALID_ARG
    assert b"multiple" in L.lca_last_error()
    assert call(c=100) == _lib.LCA_ERR_UNSUPPORTED
    assert call(io_dtype=2) == _lib.LCA_ERR_UNSUPPORTED
    assert call(prevC=FAKE) == _lib.LCA_ERR_INVALID_ARG
    assert call(N_cap=1) == _lib.LCA_ERR_INVALID_ARG
    assert call(C=None) == _lib.LCA_ERR_INVALID_ARG
    assert call(B=0) == _lib.LCA_OK            # nothing to do: no launch
    assert call(mode=1, prevC=FAKE, prevZ=FAKE) == _lib.LCA_ERR_INVALID_ARG
    # partial RoPE base: 0 (off) or a finite value above 1
    assert call(rope_base=0.5) == _lib.LCA_ERR_INVALID_ARG
    assert b"rope_base" in L.lca_last_error()
    assert call(rope_base=float("inf")) == _lib.LCA_ERR_INVALID_ARG
    assert call(rope_base=-10000.0) == _lib.LCA_ERR_INVALID_ARG
    assert call(B=0, rope_base=10000.0) == _lib.LCA_OK
    # paged cache: page_tokens a multiple of m, the table covering N_cap entries
    assert call(pages=_lib.KvPages(FAKE, 1, 6, 4)) == _lib.LCA_ERR_INVALID_ARG   # 6 tokens, m = 4
    assert b"page_tokens" in L.lca_last_error()
    assert call(pages=_lib.KvPages(FAKE, 1, 4, 4)) == _lib.LCA_ERR_INVALID_ARG   # 1 page < N_cap = 2
    assert b"N_cap" in L.lca_last_error()
    assert call(pages=_lib.KvPages(FAKE, 2, 4, 0)) == _lib.LCA_ERR_INVALID_ARG   # empty pool
    assert call(B=0, pages=_lib.KvPages(FAKE, 2, 4, 4)) == _lib.LCA_OK
    assert call(B=0, pages=_lib.KvPages(None, 0, 0, 0)) == _lib.LCA_OK            # no table: contiguous

    def rows(**kw):
        a = _valid_args()["lca_rmsnorm_rows"]
        for k_, v in kw.items():
            setattr(a, k_, v)
        return L.lca_rmsnorm_rows(ref(a), None)

    assert rows(pos0=-1, rope_base=10000.0) == _lib.LCA_ERR_INVALID_ARG      # negative pos0
    assert rows(rope_base=1.0) == _lib.LCA_ERR_INVALID_ARG                   # base 1
    assert rows(y_seq_rows=3) == _lib.LCA_ERR_INVALID_ARG
    assert rows(B=0) == _lib.LCA_OK


def test_indexer_topk_mqa_validation(L):
    def idx(**kw):
        a = _valid_args()["lca_indexer_scores"]
        for k_, v in kw.items():
            setattr(a, k_, v)
        return L.lca_indexer_scores(ref(a), None)

    assert idx(H_I=32) == _lib.LCA_ERR_UNSUPPORTED                      # fp8 only for 64 x 128
    assert idx(idx_dtype=F["mxfp4"]) == _lib.LCA_ERR_INVALID_ARG         # MXFP4 without scales
    assert idx(idx_dtype=7) == _lib.LCA_ERR_UNSUPPORTED
    assert idx(score_dtype=F["fp8"]) == _lib.LCA_ERR_UNSUPPORTED         # scores are f32 or bf16
    assert idx(B=0, score_dtype=F["bf16"]) == _lib.LCA_OK

    def topk(**kw):
        a = _valid_args()["lca_topk"]
        for k_, v in kw.items():
            setattr(a, k_, v)
        return a

    assert L.lca_topk(ref(topk(k=0)), None) == _lib.LCA_ERR_INVALID_ARG
    assert L.lca_topk(ref(topk(k=5000)), None) == _lib.LCA_ERR_INVALID_ARG
    assert ws_size(L, "topk", topk(k=0)) == (_lib.LCA_ERR_INVALID_ARG, 0)
    big = topk(B=16, N_cap=262148, k=1024)
    st, need = ws_size(L, "topk", big)
    assert st == _lib.LCA_OK and need > 0
    assert ws_size(L, "topk", topk(B=1, n_q=8, N_cap=30000, k=1024)) == (_lib.LCA_OK, 0)
    big.workspace, big.workspace_bytes = FAKE, need - 1
    assert L.lca_topk(ref(big), None) == _lib.LCA_ERR_WORKSPACE
    assert ws_size(L, "topk", topk(score_dtype=F["mxfp4"]))[0] == _lib.LCA_ERR_UNSUPPORTED

    def mqa(**kw):
        a = _valid_args()["lca_sparse_mqa"]
        for k_, v in kw.items():
            setattr(a, k_, v)
        return a

    st, need = ws_size(L, "sparse_mqa", mqa())
    assert st == _lib.LCA_OK and need > 0
    assert L.lca_sparse_mqa(ref(mqa()), None) == _lib.LCA_ERR_WORKSPACE
    assert L.lca_sparse_mqa(ref(mqa(H=12, workspace=FAKE, workspace_bytes=need)), None) == _lib.LCA_ERR_UNSUPPORTED
    assert L.lca_sparse_mqa(ref(mqa(c=384, workspace=FAKE, workspace_bytes=need)), None) == _lib.LCA_ERR_UNSUPPORTED
    assert L.lca_sparse_mqa(ref(mqa(win=None, workspace=FAKE, workspace_bytes=need)),
                            None) == _lib.LCA_ERR_INVALID_ARG        # window buffer missing, n_win > 0
    assert L.lca_sparse_mqa(ref(mqa(rope_base=float("nan"), workspace=FAKE, workspace_bytes=need)),
                            None) == _lib.LCA_ERR_INVALID_ARG
    # dense HCA (idx NULL) needs its own workspace size
    st, need_dense = ws_size(L, "sparse_mqa", mqa(idx=None, k=0))
    assert st == _lib.LCA_OK and need_dense > 0
    # a fixed split length: a positive multiple of 64, at most 256 splits per query
    assert ws_size(L, "sparse_mqa", mqa(split_rows=100))[0] == _lib.LCA_ERR_INVALID_ARG
    assert ws_size(L, "sparse_mqa", mqa(split_rows=-64))[0] == _lib.LCA_ERR_INVALID_ARG
    assert ws_size(L, "sparse_mqa", mqa(idx=None, k=0, N_cap=20000, split_rows=64))[0] == \
        _lib.LCA_ERR_UNSUPPORTED                                    # 315 splits
    st, need_fixed = ws_size(L, "sparse_mqa", mqa(split_rows=128))  # 1152 rows: 9 splits
    assert st == _lib.LCA_OK and need_fixed > 0
    assert ws_size(L, "sparse_mqa", mqa(split_rows=2048)) == (_lib.LCA_OK, 0)   # one split: no partials
    # out projection
    a = _valid_args()["lca_grouped_out_proj"]
    st, need = ws_size(L, "grouped_out_proj", a)
    assert st == _lib.LCA_OK
    a.g = 7
    assert L.lca_grouped_out_proj(ref(a), None) == _lib.LCA_ERR_INVALID_ARG
    assert ws_size(L, "grouped_out_proj", a) == (_lib.LCA_ERR_INVALID_ARG, 0)
    # an op without a workspace, a NULL size pointer
    n = ctypes.c_size_t(0)
    assert L.lca_workspace_size(99, ref(a), ref(n)) == _lib.LCA_ERR_INVALID_ARG
    assert L.lca_workspace_size(_lib.OP["topk"], ref(topk()), None) == _lib.LCA_ERR_INVALID_ARG


def _decode_layer():
    lay = _lib.DecodeLayer()
    lay.struct_size = ctypes.sizeof(_lib.DecodeLayer)
    lay.mode, lay.m, lay.B, lay.c, lay.H, lay.n_win, lay.N_cap = 0, 4, 2, 512, 64, 128, 70000
    lay.io_dtype, lay.kv_dtype, lay.k, lay.H_I, lay.d_I, lay.idx_dtype = 1, 1, 1024, 64, 128, 2
    return lay


def test_state_and_decode_validation(L):
    a = _valid_args()["lca_state_append"]
    a.n_win = 0
    assert L.lca_state_append(ref(a), None) == _lib.LCA_ERR_INVALID_ARG
    lay = _decode_layer()
    st, need = ws_size(L, "decode_step", lay)
    assert st == _lib.LCA_OK and need > 2 * 70000 * 4
    io = _lib.DecodeIO()
    io.struct_size = ctypes.sizeof(_lib.DecodeIO)
    assert L.lca_decode_step(ref(lay), ref(io), FAKE, need - 1, None) == _lib.LCA_ERR_WORKSPACE
    assert L.lca_decode_step(ref(lay), ref(io), FAKE, need,
                             None) == _lib.LCA_ERR_INVALID_ARG       # CSA without kI/qI/w
    lay.rope_base = 0.9
    assert ws_size(L, "decode_step", lay)[0] == _lib.LCA_ERR_INVALID_ARG   # bad RoPE base
    lay.rope_base = 10000.0
    assert ws_size(L, "decode_step", lay) == (_lib.LCA_OK, need)
    lay.pages = _lib.KvPages(FAKE, 100, 128, 10)          # 100 pages x 32 entries < N_cap
    assert ws_size(L, "decode_step", lay)[0] == _lib.LCA_ERR_INVALID_ARG
    lay.pages = _lib.KvPages(FAKE, 2188, 128, 10)         # 2188 x 32 >= 70000
    assert ws_size(L, "decode_step", lay) == (_lib.LCA_OK, need)
    # several steps: every step validated before any is enqueued
    ios = (_lib.DecodeIO * 2)()
    for i in range(2):
        ios[i].struct_size = ctypes.sizeof(_lib.DecodeIO)
    assert L.lca_decode_steps(ref(lay), ios, 2, FAKE, need, None) == _lib.LCA_ERR_INVALID_ARG
    assert L.lca_last_error().startswith(b"step 0")
    assert L.lca_decode_steps(ref(lay), None, 0, None, 0, None) == _lib.LCA_OK
    assert L.lca_decode_steps(ref(lay), None, -1, None, 0, None) == _lib.LCA_ERR_INVALID_ARG
    lay.pages = _lib.KvPages(None, 0, 0, 0)
    lay.split_rows = 96
    assert ws_size(L, "decode_step", lay)[0] == _lib.LCA_ERR_INVALID_ARG
    lay.split_rows = 128
    assert ws_size(L, "decode_step", lay)[0] == _lib.LCA_OK
    lay.split_rows = 0
    lay.k = 0
    assert ws_size(L, "decode_step", lay)[0] == _lib.LCA_ERR_INVALID_ARG


def test_no_cpu_fallback_in_binding():
    """The binding must raise when the library is missing, never compute on the CPU."""
    src = open(os.path.join(ROOT, "long_context_attention_14_amd", "ops.py")).read()
    for name in ("oracle", "numpy", "np."):
        assert name not in src
    src = open(os.path.join(ROOT, "long_context_attention_14_amd", "_lib.py")).read()
    assert "no fallback" in src


def test_device_checks_entry_point_is_debug_only():
    """The release library exports lca_device_checks but has no device checks: it
    returns LCA_ERR_UNSUPPORTED with the count set to 0, and rejects NULL."""
    import ctypes
    from long_context_attention_14_amd import _lib
    L = _lib.lib()
    v = ctypes.c_uint64(123)
    assert L.lca_device_checks(ctypes.addressof(v), 0) == _lib.LCA_ERR_UNSUPPORTED
    assert v.value == 0
    assert L.lca_device_checks(None, 0) == _lib.LCA_ERR_INVALID_ARG
