"""Workload descriptions for the CSA/HCA attention path.

Hyperparameters follow the pages: CSA compression rate m=4, top-k 1024,
indexer 64 heads x 128 dims ("DeepSeek V4 Architecture Tricks", section
"CSA: Compressed Sparse Attention"); HCA rate m'=128 (same page, section
"HCA: Heavily Compressed Attention"); window n_win=128 (same page, section
"Sliding Window Branch"); head dim c=512 (QbitAI article on DeepSeek-V4,
section on the hybrid attention mechanism); RoPE on the last 64 dims, stored
in bf16 while the other KV dims are fp8 (pinktalk page, section "Partial RoPE
和 Attention Sink").
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str
    kind: str              # "csa_prefill" | "csa_decode" | "hca_decode" | "hybrid_decode"
    B: int                 # batch (sequences)
    ctx: int               # decode: base context (L_b = ctx + T_b); prefill: prefix length
    n_new: int             # prefill: new tokens; decode: 1
    c: int                 # KV / query head dim
    H: int                 # query heads
    H_I: int               # indexer heads
    d_I: int               # indexer head dim
    m: int                 # CSA rate (or HCA rate for pure-HCA configs)
    k: int                 # top-k
    n_win: int             # sliding window
    io_dtype: str          # "f32" | "bf16"   (C, Z, q, outputs)
    kv_dtype: str          # "f32" | "bf16" | "fp8_bf16rope"   (compressed cache and window)
    idx_dtype: str         # "f32" | "fp8" | "mxfp4"           (indexer q/k)
    m_hca: int = 128
    layers: Tuple[str, ...] = ()     # hybrid stack: sequence of "C"/"H"
    seed: int = 0
    rope_dims: int = 64
    eps: float = 1e-6
    rope_base: float = 0.0           # partial RoPE frequency base; 0: off (inputs taken as post-RoPE)

    @property
    def tau(self) -> float:
        return 1.0 / (self.c ** 0.5)

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# Tiny CSA prefill, fp32: n=1024, m=4 -> 256 entries, indexer 4x32, k=32,
# 8 query heads of dim 128, window 16.
TINY_CSA_PREFILL = LayerConfig(
    name="tiny_csa_prefill_fp32", kind="csa_prefill", B=1, ctx=0, n_new=1024, c=128, H=8,
    H_I=4, d_I=32, m=4, k=32, n_win=16, io_dtype="f32", kv_dtype="f32", idx_dtype="f32")

# HCA decode: batch 32, context 131072 (+ tail 0..127), m'=128 -> 1024 entries,
# 64 heads x 512, window 128, bf16 in / fp32 accumulate.
HCA_DECODE = LayerConfig(
    name="hca_decode_b32_128k_bf16", kind="hca_decode", B=32, ctx=131072, n_new=1, c=512, H=64,
    H_I=0, d_I=0, m=128, k=0, n_win=128, io_dtype="bf16", kv_dtype="bf16", idx_dtype="f32")

# CSA decode at 1M context: batch 16, m=4 -> 262144 entries, fp8 indexer keys,
# top-1024, 64 heads x 512, window 128.
CSA_DECODE_1M = LayerConfig(
    name="csa_decode_b16_1m_bf16_fp8idx", kind="csa_decode", B=16, ctx=1 << 20, n_new=1, c=512,
    H=64, H_I=64, d_I=128, m=4, k=1024, n_win=128, io_dtype="bf16", kv_dtype="bf16",
    idx_dtype="fp8")

# CSA prefill chunk: 8192 new tokens on a 131072-token prefix (34816 entries).
CSA_PREFILL_CHUNK = LayerConfig(
    name="csa_prefill_8k_on_128k_bf16_fp8idx", kind="csa_prefill", B=1, ctx=131072, n_new=8192,
    c=512, H=64, H_I=64, d_I=128, m=4, k=1024, n_win=128, io_dtype="bf16", kv_dtype="bf16",
    idx_dtype="fp8")

# Hybrid 8-layer decode slice at 1M: H,H,C,H,C,H,C,H; MXFP4 indexer; fp8 KV with
# bf16 rope dims.
HYBRID_DECODE_1M = LayerConfig(
    name="hybrid8_decode_b4_1m_mxfp4idx_fp8kv", kind="hybrid_decode", B=4, ctx=1 << 20, n_new=1,
    c=512, H=64, H_I=64, d_I=128, m=4, k=1024, n_win=128, io_dtype="bf16",
    kv_dtype="fp8_bf16rope", idx_dtype="mxfp4", layers=("H", "H", "C", "H", "C", "H", "C", "H"))

@dataclass(frozen=True)
class OutProjConfig:
    """Grouped output projection after the attention: the n_h heads' outputs in
    g groups, each projected to d_g, then all groups back to the hidden size d
    (QbitAI article, hybrid attention section; d = 7168 is V4-Pro's hidden size,
    same article, section 模型訓練 (model training)).  The pages give neither g nor
    d_g: g = 8 groups of 8 heads and d_g = 1024 are readings."""
    name: str
    T: int                 # query tokens (decode: the batch; prefill: the chunk)
    n_h: int = 64
    c: int = 512
    g: int = 8
    d_g: int = 1024
    d: int = 7168
    seed: int = 0

    def with_(self, **kw) -> "OutProjConfig":
        return replace(self, **kw)


OUT_PROJ_DECODE = OutProjConfig(name="out_proj_decode_b16", T=16)
OUT_PROJ_PREFILL = OutProjConfig(name="out_proj_prefill_8k", T=8192)

CONFIGS = {cfg.name: cfg for cfg in
           (TINY_CSA_PREFILL, HCA_DECODE, CSA_DECODE_1M, CSA_PREFILL_CHUNK, HYBRID_DECODE_1M)}


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]
