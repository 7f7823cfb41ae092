"""The seeded input generator: determinism, slicing, formats and distributions."""
import numpy as np

from oracle import lca_oracle as O
from synth import encode as enc
from synth import gen
from synth.configs import CSA_DECODE_1M, TINY_CSA_PREFILL


def test_rows_are_seeded_and_sliceable():
    a = gen.draw_rows(0, "x", 1, 10000, 8, "normal")
    b = gen.draw_rows(0, "x", 1, 10000, 8, "normal")
    assert np.array_equal(a, b)
    part = gen.draw_rows(0, "x", 1, 300, 8, "normal", row0=4000)
    assert np.array_equal(part, a[4000:4300])
    assert not np.array_equal(a, gen.draw_rows(1, "x", 1, 10000, 8, "normal"))
    assert not np.array_equal(a, gen.draw_rows(0, "x", 2, 10000, 8, "normal"))


def test_distributions():
    x = gen.draw_rows(0, "n", 0, 20000, 16, "normal")
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    s = gen.draw_rows(0, "s", 0, 1000, 512, "sphere").astype(np.float64)
    assert np.allclose(np.sqrt((s * s).mean(-1)), 1.0, atol=1e-6)
    u = gen.draw_rows(0, "u", 0, 1000, 64, "uniform")
    assert u.min() >= 0 and u.max() < 1
    p = gen.draw_rows(0, "p", 0, 1000, 64, "bias")
    assert abs(p.std() - 0.1) < 0.005


def test_encoders_roundtrip_through_oracle_decoders():
    x = gen.draw_rows(0, "e", 0, 64, 512, "sphere")
    assert np.array_equal(O.decode(enc.encode(x, "bf16"), "bf16"), O.round_to(x.astype(np.float64), "bf16"))
    assert np.array_equal(O.decode(enc.encode(x, "fp8"), "fp8"), O.round_to(x.astype(np.float64), "fp8"))
    kv = enc.encode(x, "fp8_bf16rope")
    assert kv.shape == (64, 576)
    assert np.array_equal(O.decode(kv, "fp8_bf16rope"), O.round_to(x.astype(np.float64), "fp8_bf16rope"))


def test_decode_inputs_shapes_small():
    cfg = CSA_DECODE_1M.with_(B=3, ctx=4096)
    d = gen.decode_inputs(cfg)
    L = d["lengths"]
    assert np.all((L >= 4096) & (L < 4100))
    assert d["cache"].shape == (3, d["n_cap"], 512) and d["cache"].dtype == np.uint16
    assert d["kI"].shape == (3, d["n_cap"], 128) and d["kI"].dtype == np.uint8
    # cache rows past the pre-step entry count are zero
    for b in range(3):
        npre = (L[b] - 1) // 4
        assert np.all(d["cache"][b, npre:] == 0) and np.any(d["cache"][b, npre - 1] != 0)


def test_prefill_inputs_tiny():
    d = gen.prefill_inputs(TINY_CSA_PREFILL)
    assert d["C"].shape == (1, 1024, 128) and d["C"].dtype == np.float32
    assert d["kI"].shape == (1, 256, 32) and d["q"].shape == (1, 1024, 8, 128)
    assert d["P"].shape == (8, 128)
