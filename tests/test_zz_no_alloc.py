"""lca_decode_step_static, the decode step that allocates nothing (its scratch
space is the library's own per-device array): results bit-identical to
lca_decode_step with a caller workspace, on two calls in a row whose second
is smaller (the array then holds the first call's contents), and a layer too
large for the array is rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from long_context_attention_14_amd import _lib, ops, pipeline
from synth import gen
from synth.configs import CSA_DECODE_1M, HCA_DECODE, HYBRID_DECODE_1M

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _bits(layer):
    torch.cuda.synchronize()
    r = {"out": layer.out.view(torch.int16).cpu().numpy(), "lse": layer.lse.cpu().numpy(),
         "cache": layer.logical_cache(), "ring": layer.ring.cpu().numpy().view(np.uint8),
         "n_tokens": layer.n_tokens.cpu().numpy(), "tail": layer.tailC.cpu().numpy().view(np.uint8)}
    if layer.mode == "csa":
        r["idx"] = layer.idx.cpu().numpy()
    return r


def _static_step(layer):
    csa = layer.mode == "csa"
    ops.lca_decode_step_static(layer.state, layer.tokC, layer.tokZ, layer.q, layer.out,
                               layer.cfg.io_dtype, qI=layer.qI if csa else None,
                               qI_scale=layer.qI_scale if csa else None, w=layer.w if csa else None,
                               lse=layer.lse, idx_out=layer.idx if csa else None)


def _case(name):
    if name == "csa_fused_b4_2e18":          # fused indexer + selection, 24 MiB of scratch
        cfg = CSA_DECODE_1M.with_(B=4, ctx=1 << 18)
        return cfg, gen.decode_inputs(cfg)
    if name == "csa_b2_2e14":                # score array + LDS top-k
        cfg = CSA_DECODE_1M.with_(B=2, ctx=1 << 14)
        return cfg, gen.decode_inputs(cfg)
    if name == "hybrid_csa_b2_2e18":         # MXFP4 keys, fp8+bf16 KV
        cfg = HYBRID_DECODE_1M.with_(B=2, ctx=1 << 18)
        return cfg, gen.decode_layer(cfg, "C", cfg.m, gen.hybrid_lengths(cfg), layer=2)
    if name == "hca_b3_2e14":
        cfg = HCA_DECODE.with_(B=3, ctx=1 << 14)
        return cfg, gen.decode_inputs(cfg)
    raise ValueError(name)


@pytest.mark.gpu
@pytest.mark.parametrize("first,second,sel_hist", [("csa_fused_b4_2e18", "csa_b2_2e14", True),
                                                   ("csa_fused_b4_2e18", "csa_b2_2e14", False),
                                                   ("hybrid_csa_b2_2e18", "hca_b3_2e14", True)])
def test_static_scratch_step_equals_workspace_step(first, second, sel_hist):
    """sel_hist=False: the fused selection's histogram lives in the scratch array
    (cleared by each step's first launch) rather than in the layer's state."""
    for name in (first, second):           # the second call is smaller than the first
        cfg, d = _case(name)
        ref = pipeline.DecodeLayer(cfg, d, DEV, sel_hist=sel_hist)
        sta = pipeline.DecodeLayer(cfg, d, DEV, sel_hist=sel_hist)
        need = ref.state.workspace_size()
        assert 0 < need <= _lib.LCA_STATIC_SCRATCH_BYTES
        say(f"no-alloc decode step {name}: B={cfg.B} N_cap={d['n_cap']} scratch {need >> 20} MiB, "
            f"sel_hist {sel_hist}")
        for step in range(2):             # two steps each: the second sees the first's entries
            ref.step()
            _static_step(sta)
            a, b = _bits(ref), _bits(sta)
            for key in a:
                assert np.array_equal(a[key], b[key]), f"{name} step {step}: {key} differs"


def test_static_scratch_rejects_a_layer_too_large():
    """Validation only (no GPU work): a CSA layer of 64 sequences at 1M tokens needs
    more scratch than the library's array holds."""
    L = _lib.lib()
    lay = _lib.DecodeLayer()
    lay.struct_size = ctypes.sizeof(_lib.DecodeLayer)
    lay.mode, lay.m, lay.B, lay.c, lay.H, lay.n_win, lay.N_cap = 0, 4, 64, 512, 64, 128, 262150
    lay.io_dtype, lay.kv_dtype, lay.k, lay.H_I, lay.d_I, lay.idx_dtype = 1, 1, 1024, 64, 128, 2
    need = ctypes.c_size_t(0)
    assert L.lca_workspace_size(_lib.OP["decode_step"], ctypes.byref(lay), ctypes.byref(need)) == _lib.LCA_OK
    assert need.value > _lib.LCA_STATIC_SCRATCH_BYTES
    io = _lib.DecodeIO()
    io.struct_size = ctypes.sizeof(_lib.DecodeIO)
    FAKE = 0x1000
    io.tokC = io.tokZ = io.q = io.qI = io.w = io.out = FAKE
    lay.tailC = lay.tailZ = lay.ring = lay.cache = lay.n_tokens = lay.P = lay.kI = FAKE
    assert L.lca_decode_step_static(ctypes.byref(lay), ctypes.byref(io), None) == _lib.LCA_ERR_WORKSPACE
    assert b"static scratch" in L.lca_last_error()
    lay.struct_size = 5
    assert L.lca_decode_step_static(ctypes.byref(lay), ctypes.byref(io), None) == _lib.LCA_ERR_INVALID_ARG
