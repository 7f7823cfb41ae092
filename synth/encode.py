"""Encoders from float values to the byte formats the path stores.

bf16 and fp8-e4m3fn use torch's CPU casts (round to nearest even); fp8 values
are clamped to the largest finite magnitude (448) first, the "satfinite"
behaviour the OCP fp8 format specifies.  MXFP4 (OCP microscaling: e2m1
elements in blocks of 32 along the last dim, one E8M0 power-of-two scale per
block) is encoded here directly.  The mixed KV row layout stores the first
c-64 dims as e4m3 bytes followed by the last 64 dims as bf16 values, which is
the split the pinktalk page ("DeepSeek V4 Architecture Tricks", section
"Partial RoPE 和 Attention Sink") describes for RoPE vs non-RoPE dims.
"""
import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def to_f32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def to_bf16_bits(x) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bits(x) -> np.ndarray:
    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e2m1_codes(y: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (ties to the even code) for |y| <= 6 after saturation."""
    a = np.minimum(np.abs(y), 6.0)
    d = np.abs(a[..., None] - E2M1_VALUES)            # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equally near magnitudes, take the even code (codes 0..7 index E2M1_VALUES)
    even = cand & ((np.arange(8) % 2) == 0)
    code = np.where(even.any(-1), np.argmax(even, -1), np.argmax(cand, -1)).astype(np.uint8)
    sign = ((y < 0) & (code != 0)).astype(np.uint8)
    return code | (sign << 3)


def to_mxfp4(x, block: int = 32):
    """Returns (packed uint8 [..., d/2], scales uint8 [..., d/block]).

    Scale exponent = floor(log2(amax)) - 2 (the largest e2m1 exponent), stored
    as the biased E8M0 byte; an all-zero block gets scale byte 127 (2^0).
    Element 2i sits in the low nibble of byte i, element 2i+1 in the high one.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % block == 0
    xb = x.reshape(*x.shape[:-1], d // block, block)
    amax = np.abs(xb).max(-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    e = np.clip(e, -127, 127)
    scaled = xb / np.exp2(e)[..., None]
    codes = _e2m1_codes(scaled).reshape(*x.shape[:-1], d)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(scales)


def to_kv_fp8_bf16rope(x, rope_dims: int = 64) -> np.ndarray:
    """[..., c] float -> [..., (c-rope) + 2*rope] uint8 bytes."""
    x = np.asarray(x, dtype=np.float32)
    c = x.shape[-1]
    lo = to_e4m3_bits(x[..., : c - rope_dims])
    hi = to_bf16_bits(x[..., c - rope_dims:]).view(np.uint8).reshape(*x.shape[:-1], 2 * rope_dims)
    return np.ascontiguousarray(np.concatenate([lo, hi], axis=-1))


def encode(x, fmt: str):
    """Encode float rows into the named storage format."""
    if fmt == "f32":
        return to_f32(x)
    if fmt == "bf16":
        return to_bf16_bits(x)
    if fmt == "fp8":
        return to_e4m3_bits(x)
    if fmt == "fp8_bf16rope":
        return to_kv_fp8_bf16rope(x)
    raise ValueError(fmt)


def row_bytes(fmt: str, c: int) -> int:
    return {"f32": 4 * c, "bf16": 2 * c, "fp8": c, "fp8_bf16rope": c + 64}[fmt]
