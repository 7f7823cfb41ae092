"""Pins of the float64 oracle against things other than itself: closed forms,
library routines, brute force on tiny inputs and the invariants the method must
satisfy.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import lca_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# stored formats


def test_decode_bf16_matches_torch_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_decode_e4m3_matches_torch_all_patterns():
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9      # format limits


def test_e2m1_table_from_format_definition():
    # value = 2^(e-1) * (1 + f/2) for e > 0, f/2 for e = 0 (bias 1, 1 mantissa bit)
    for code in range(16):
        s, e, f = code >> 3, (code >> 1) & 3, code & 1
        v = (2.0 ** (e - 1)) * (1 + f / 2) if e else f / 2
        assert O.E2M1[code] == (-v if s else v)


@pytest.mark.parametrize("fmt,tdt", [("bf16", torch.bfloat16), ("fp8", torch.float8_e4m3fn)])
def test_round_to_matches_torch_cast(fmt, tdt):
    r = rng(1)
    x = np.concatenate([r.standard_normal(20000) * s for s in (1e-3, 1, 30, 300)]).astype(np.float32)
    if fmt == "fp8":
        # exact halfway points between neighbouring e4m3 values (ties to even)
        vals = np.unique(np.abs(O.E4M3[np.isfinite(O.E4M3)]))
        x = np.concatenate([x, ((vals[1:] + vals[:-1]) / 2).astype(np.float32)])
        x = np.clip(x, -448, 448)
    else:
        # bf16 halfway points: fp32 patterns with exactly the 0x8000 low half
        hb = (r.integers(0x3000, 0x4f00, 5000).astype(np.uint32) << 16) | 0x8000
        x = np.concatenate([x, hb.view(np.float32)])
    ref = torch.from_numpy(x).to(tdt).to(torch.float64).numpy()
    assert np.array_equal(O.round_to(x.astype(np.float64), fmt), ref)


def test_fp8_saturates():
    assert O.round_to(np.array([1e6, -500.0]), "fp8").tolist() == [448.0, -448.0]


def test_mxfp4_decode_closed_form():
    # byte 0x21: low nibble code 1 (0.5), high nibble code 2 (1.0); scale 2^(130-127)=8
    packed = np.full((1, 16), 0x21, np.uint8)
    scales = np.array([[130]], np.uint8)
    x = O.decode_mxfp4(packed, scales)
    assert x.shape == (1, 32)
    assert np.all(x[0, 0::2] == 4.0) and np.all(x[0, 1::2] == 8.0)


def test_mxfp4_generator_roundtrip():
    from synth import encode as enc
    r = rng(2)
    x = r.standard_normal((64, 128))
    p, s = enc.to_mxfp4(x)
    y = O.decode_mxfp4(p, s)
    # error per element <= half an e2m1 step at the block scale, i.e. amax/8 ... /4
    blk = np.abs(x.reshape(64, 4, 32)).max(-1)
    err = np.abs(y - x).reshape(64, 4, 32).max(-1)
    assert np.all(err <= blk / 4 + 1e-12)
    # exactly representable inputs come back exactly
    z = O.E2M1[r.integers(0, 16, (8, 64))] * 0.25
    z[:, ::32] = 1.5                       # amax 1.5 in every block -> scale 2^-2
    p, s = enc.to_mxfp4(z)
    assert np.array_equal(O.decode_mxfp4(p, s), z)


# ---------------------------------------------------------------------------
# RMSNorm and the compressor


def test_rmsnorm_closed_form():
    x = rng(3).standard_normal((10, 64)) * 3
    y = O.rmsnorm(x, 1e-6)
    ms = np.mean(x * x, -1)
    assert np.allclose(np.sqrt(np.mean(y * y, -1)), np.sqrt(ms / (ms + 1e-6)), rtol=1e-14)
    assert np.allclose(y / x, (1 / np.sqrt(ms + 1e-6))[:, None])


def test_compress_hand_example():
    # HCA, m=4, c=1: zero gates, bias ln(1..4) -> weights 1:2:3:4, E = (1+4+9+16)/10 = 3
    C = np.array([[1.0], [2.0], [3.0], [4.0]])
    P = np.log(np.array([[1.0], [2.0], [3.0], [4.0]]))
    assert np.isclose(O.compress(C, np.zeros_like(C), P, 4, False)[0, 0], 3.0, rtol=1e-15)
    # CSA entry 1 pools blocks 0 and 1 (8 candidates), uniform gate -> mean of 1..8
    C8 = np.arange(1.0, 9.0)[:, None]
    E = O.compress(C8, np.zeros_like(C8), np.zeros((8, 1)), 4, True)
    assert np.isclose(E[0, 0], 2.5) and np.isclose(E[1, 0], 4.5)


@pytest.mark.parametrize("overlap,m", [(True, 4), (False, 4), (False, 128), (True, 2)])
def test_compress_uniform_gate_is_block_mean(overlap, m):
    r = rng(4)
    n, c = 4 * m, 16
    C = r.standard_normal((n, c))
    const = r.standard_normal(c)
    Z = np.tile(const, (n, 1))
    P = np.zeros((2 * m if overlap else m, c))
    E = O.compress(C, Z, P, m, overlap)
    Cb = C.reshape(-1, m, c)
    if overlap:
        # entry 0 has no previous block: mean of its own m tokens; later: mean of 2m
        want = np.concatenate([Cb[:1].mean(1), np.concatenate([Cb[:-1], Cb[1:]], 1).mean(1)], 0)
    else:
        want = Cb.mean(1)
    assert np.allclose(E, want, rtol=1e-13, atol=1e-14)


def test_compress_one_hot_and_shift_invariance():
    r = rng(5)
    m, c = 4, 8
    C = r.standard_normal((3 * m, c))
    Z = r.standard_normal((3 * m, c))
    P = r.standard_normal((2 * m, c)) * 0.1
    # one-hot: make candidate slot 5 (own block, token 1) dominate channel 3 of entry 2
    Z2 = Z.copy()
    Z2[2 * m + 1, 3] += 60.0
    E = O.compress(C, Z2, P, m, True)
    assert np.isclose(E[2, 3], C[2 * m + 1, 3], rtol=1e-12)
    # adding a per-channel constant to all gate logits changes nothing
    E0 = O.compress(C, Z, P, m, True)
    E1 = O.compress(C, Z + r.standard_normal(c)[None], P, m, True)
    assert np.allclose(E0, E1, rtol=1e-12, atol=1e-14)
    # m=1 without overlap is the identity
    assert np.allclose(O.compress(C, Z, P[:1], 1, False), C)


def test_compress_matches_brute_force():
    r = rng(6)
    for overlap, m in [(True, 4), (False, 8)]:
        n, c = 4 * m, 6
        C, Z = r.standard_normal((n, c)), r.standard_normal((n, c))
        P = r.standard_normal((2 * m if overlap else m, c)) * 0.1
        pc, pz = r.standard_normal((m, c)), r.standard_normal((m, c))
        E = O.compress(C, Z, P, m, overlap, pc if overlap else None, pz if overlap else None)
        for s in range(n // m):
            b = brute.compress_entry(C.tolist(), Z.tolist(), P.tolist(), m, s, overlap,
                                     pc.tolist() if overlap else None, pz.tolist() if overlap else None)
            assert np.allclose(E[s], b, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# indexer scores and top-k


def test_index_scores_single_head_is_relu_matmul():
    r = rng(7)
    q = r.standard_normal((5, 1, 16))
    k = r.standard_normal((40, 16))
    I = O.index_scores(q, k, np.ones((5, 1)), np.full(5, 40))
    assert np.allclose(I, np.maximum(q[:, 0] @ k.T, 0), rtol=1e-13, atol=1e-13)


def test_index_scores_brute_force_and_mask():
    r = rng(8)
    q = r.standard_normal((3, 4, 8))
    k = r.standard_normal((20, 8))
    w = r.random((3, 4))
    vis = np.array([0, 7, 20])
    I = O.index_scores(q, k, w, vis)
    for t in range(3):
        for s in range(20):
            if s < vis[t]:
                assert np.isclose(I[t, s], brute.score(q[t].tolist(), k[s].tolist(), w[t].tolist()),
                                  rtol=1e-12)
            else:
                assert I[t, s] == -np.inf


def test_index_scores_zero_when_all_dots_negative():
    q = -np.abs(rng(9).standard_normal((1, 3, 8)))
    k = np.abs(rng(10).standard_normal((6, 8)))
    assert np.all(O.index_scores(q, k, np.ones((1, 3)), [6]) == 0.0)


def test_topk_matches_brute_force_with_ties():
    r = rng(11)
    for trial in range(30):
        n = int(r.integers(1, 60))
        s = r.integers(-3, 4, n).astype(np.float64)        # heavy ties
        if trial % 3 == 0:
            s[r.integers(0, n)] = -0.0
        k = int(r.integers(1, 70))
        got = O.topk(s[None], [n], k)[0]
        assert got.tolist() == brute.select(list(s + 0.0), k)


def test_topk_edge_cases():
    s = np.array([[1.0, np.nan, -0.0, 0.0, 5.0, 5.0]])
    # NaN counts as -inf; -0 equals +0 so index 2 wins the tie against 3
    assert O.topk(s, [6], 3)[0].tolist() == [0, 4, 5]
    assert O.topk(s, [6], 4)[0].tolist() == [0, 2, 4, 5]
    assert O.topk(s, [6], 10)[0].tolist() == [0, 1, 2, 3, 4, 5, -1, -1, -1, -1]
    assert O.topk(s, [0], 2)[0].tolist() == [-1, -1]
    assert O.topk(s, [2], 1)[0].tolist() == [0]


def test_topk_invariant_under_increasing_transform_and_scaling():
    r = rng(12)
    q = r.standard_normal((4, 4, 16))
    k = r.standard_normal((300, 16))
    w = r.random((4, 4))
    vis = np.array([10, 100, 250, 300])
    a = O.topk(O.index_scores(q, k, w, vis), vis, 32)
    b = O.topk(O.index_scores(q * 3.7, k, w, vis), vis, 32)
    c = O.topk(np.exp(O.index_scores(q, k, w, vis) / 50.0), vis, 32)
    assert np.array_equal(a, b) and np.array_equal(a, c)


# ---------------------------------------------------------------------------
# attention and merge


def test_attention_constant_rows_and_single_row():
    r = rng(13)
    q = r.standard_normal((3, 8))
    v = r.standard_normal(8)
    o, lse = O.attend(q, np.tile(v, (5, 1)), 0.3)
    assert np.allclose(o, v[None], rtol=1e-13)
    assert np.allclose(lse, 0.3 * q @ v + np.log(5))
    o1, _ = O.attend(q, v[None], 0.3)
    assert np.allclose(o1, v[None])
    oe, le = O.attend(q, np.zeros((0, 8)), 0.3)
    assert np.all(le == -np.inf) and np.all(oe == 0)


def test_merge_split_invariance_and_order():
    r = rng(14)
    q = r.standard_normal((4, 16))
    rows = r.standard_normal((23, 16))
    whole = O.attend(q, rows, 0.25)
    for _ in range(5):
        perm = r.permutation(23)
        cuts = np.sort(r.choice(np.arange(1, 23), 3, replace=False))
        parts = [O.attend(q, rows[p], 0.25) for p in np.split(perm, cuts)]
        o, lse = O.merge(parts)
        assert np.allclose(o, whole[0], rtol=1e-12, atol=1e-13)
        assert np.allclose(lse, whole[1], rtol=1e-13)
    # an empty part changes nothing
    o, lse = O.merge([whole, O.attend(q, rows[:0], 0.25)])
    assert np.allclose(o, whole[0]) and np.allclose(lse, whole[1])


def test_merge_sink_closed_form():
    r = rng(15)
    q = r.standard_normal((2, 8))
    rows = r.standard_normal((5, 8))
    sink = np.array([0.5, -1.0])
    o, lse = O.merge([O.attend(q, rows, 0.5)], sink)
    o_ns, lse_ns = O.attend(q, rows, 0.5)
    scale = np.exp(lse_ns) / (np.exp(lse_ns) + np.exp(sink))
    assert np.allclose(o, o_ns * scale[:, None])
    for h in range(2):
        b = brute.attention(q[h].tolist(), rows.tolist(), 0.5, sink[h])
        assert np.allclose(o[h], b, rtol=1e-12)


def _tiny_layer_inputs(seed, n=48, c=16, H=2, HI=3, dI=8, m=4):
    r = rng(seed)
    return dict(C=r.standard_normal((n, c)), Z=r.standard_normal((n, c)),
                P=r.standard_normal((2 * m, c)) * 0.1, q=r.standard_normal((n, H, c)),
                qI=r.standard_normal((n, HI, dI)), kI=r.standard_normal((n // m, dI)),
                w=r.random((n, HI)))


@pytest.mark.parametrize("mode,m,k,n_win,kv,rope_base",
                         [("csa", 4, 5, 6, "f32", 0.0), ("csa", 4, 3, 1, "bf16", 0.0),
                          ("hca", 8, 0, 5, "fp8", 0.0), ("csa", 2, 4, 3, "fp8_bf16rope", 0.0),
                          ("csa", 4, 5, 6, "f32", 10000.0), ("hca", 8, 0, 5, "fp8_bf16rope", 50.0)])
def test_layer_matches_brute_force(mode, m, k, n_win, kv, rope_base):
    c = 80 if kv == "fp8_bf16rope" or rope_base else 16
    d = _tiny_layer_inputs(20 + m + k, n=32, c=c, m=m)
    tau = 1 / math.sqrt(c)
    sink = np.array([0.3, -0.7])
    res = O.prefill_layer(mode=mode, m=m, k=k, n_win=n_win, tau=tau, eps=1e-6, kv_fmt=kv,
                          out_fmt="f32", pos0=0, C=d["C"], Z=d["Z"], P=d["P"][: 2 * m if mode == "csa" else m],
                          q=d["q"], cache_prefix=np.zeros((0, c)), qI=d["qI"], kI=d["kI"], w=d["w"],
                          sink=sink, rope_base=rope_base)
    rk = (lambda row: O.round_to(np.array(row), kv).tolist())
    outs, idxs, entries = brute.layer(mode=mode, m=m, k=k, n_win=n_win, tau=tau, eps=1e-6,
                                      C=d["C"].tolist(), Z=d["Z"].tolist(),
                                      P=d["P"][: 2 * m if mode == "csa" else m].tolist(),
                                      q=d["q"].tolist(), qI=d["qI"].tolist(), kI=d["kI"].tolist(),
                                      w=d["w"].tolist(), round_kv=rk, sink=sink.tolist(),
                                      rope_base=rope_base)
    assert np.allclose(res["entries"], entries, rtol=1e-12, atol=1e-12)
    if mode == "csa":
        assert np.array_equal(res["idx"], np.array(idxs))
    assert np.allclose(res["out"], np.array(outs), rtol=1e-6, atol=1e-6)   # out rounded to f32


def test_dense_limit_equals_sdpa():
    """With k >= number of entries, CSA is dense attention over [entries; window]
    under the causal masks; checked against torch's scaled_dot_product_attention."""
    m, n, c, H, n_win = 4, 64, 16, 2, 5
    d = _tiny_layer_inputs(30, n=n, c=c, H=H, m=m)
    tau = 1 / math.sqrt(c)
    res = O.prefill_layer(mode="csa", m=m, k=10 ** 6 // 10 ** 4, n_win=n_win, tau=tau, eps=1e-6,
                          kv_fmt="f32", out_fmt="f32", pos0=0, C=d["C"], Z=d["Z"], P=d["P"], q=d["q"],
                          cache_prefix=np.zeros((0, c)), qI=d["qI"], kI=d["kI"], w=d["w"])
    K = np.concatenate([res["entries"], O.round_to(O.rmsnorm(d["C"]), "f32")], 0)   # [N + n, c]
    N = n // m
    t = np.arange(n)[:, None]
    mask = np.concatenate([(np.arange(N)[None] + 1) * m - 1 <= t,
                           (np.arange(n)[None] <= t) & (np.arange(n)[None] > t - n_win)], 1)
    qh = torch.from_numpy(O.rmsnorm(d["q"]).transpose(1, 0, 2))              # [H, n, c]
    kv = torch.from_numpy(K)[None].expand(H, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qh, kv, kv, attn_mask=torch.from_numpy(mask)[None], scale=tau).numpy().transpose(1, 0, 2)
    assert np.allclose(res["out"], ref, rtol=1e-6, atol=1e-6)


def test_empty_selection_is_pure_window():
    # queries at t < m-1 see no entry: output is the window alone
    m, c = 4, 16
    d = _tiny_layer_inputs(31, n=16, c=c, m=m)
    res = O.prefill_layer(mode="csa", m=m, k=2, n_win=3, tau=0.25, eps=1e-6, kv_fmt="f32",
                          out_fmt="f32", pos0=0, C=d["C"], Z=d["Z"], P=d["P"], q=d["q"],
                          cache_prefix=np.zeros((0, c)), qI=d["qI"], kI=d["kI"], w=d["w"],
                          queries=[0, 1, 2])
    U = O.round_to(O.rmsnorm(d["C"]), "f32")
    for r, t in enumerate([0, 1, 2]):
        assert np.all(res["idx"][r] == -1)
        o, _ = O.attend(O.rmsnorm(d["q"][t]), U[max(0, t - 2): t + 1], 0.25)
        assert np.allclose(res["out"][r], o, atol=1e-6)


def test_causality_future_perturbation():
    m, n, c = 4, 40, 16
    d = _tiny_layer_inputs(32, n=n, c=c, m=m)
    kw = dict(mode="csa", m=m, k=3, n_win=4, tau=0.25, eps=1e-6, kv_fmt="bf16", out_fmt="f32",
              pos0=0, P=d["P"], cache_prefix=np.zeros((0, c)))
    a = O.prefill_layer(C=d["C"], Z=d["Z"], q=d["q"], qI=d["qI"], kI=d["kI"], w=d["w"], **kw)
    cut = 21                                     # perturb tokens > cut (and their entries)
    e = {key: v.copy() for key, v in d.items()}
    r = rng(33)
    e["C"][cut + 1:] += r.standard_normal(e["C"][cut + 1:].shape)
    e["Z"][cut + 1:] += 5
    e["q"][cut + 1:] *= -1
    e["qI"][cut + 1:] += 1
    e["kI"][(cut + 1) // m:] += r.standard_normal(e["kI"][(cut + 1) // m:].shape)
    b = O.prefill_layer(C=e["C"], Z=e["Z"], q=e["q"], qI=e["qI"], kI=e["kI"], w=e["w"], **kw)
    assert np.array_equal(a["out"][: cut + 1], b["out"][: cut + 1])
    assert np.array_equal(a["idx"][: cut + 1], b["idx"][: cut + 1])


# ---------------------------------------------------------------------------
# decode: incremental steps reproduce the prefill


@pytest.mark.parametrize("mode,m,rope_base", [("csa", 4, 0.0), ("hca", 8, 0.0), ("csa", 4, 10000.0),
                                               ("hca", 8, 300.0)])
def test_incremental_decode_equals_prefill(mode, m, rope_base):
    n, c, H = 40, 80 if rope_base else 16, 2
    d = _tiny_layer_inputs(40 + m, n=n, c=c, H=H, m=m)
    P = d["P"][: 2 * m if mode == "csa" else m]
    kw = dict(tau=0.25, eps=1e-6, kv_fmt="bf16", out_fmt="f32", rope_base=rope_base)
    pre = O.prefill_layer(mode=mode, m=m, k=3, n_win=5, pos0=0, C=d["C"], Z=d["Z"], P=P, q=d["q"],
                          cache_prefix=np.zeros((0, c)), qI=d["qI"], kI=d["kI"], w=d["w"], **kw)
    st = O.DecodeState(mode=mode, m=m, n_win=5, c=c)
    for t in range(n):
        r = O.decode_step(st, tokC=d["C"][t], tokZ=d["Z"][t], P=P, q=d["q"][t], k=3,
                          qI=d["qI"][t], kI=d["kI"], w=d["w"][t], **kw)
        assert np.array_equal(r["out"], pre["out"][t])
        if mode == "csa":
            assert np.array_equal(r["idx"], pre["idx"][t])
    assert np.array_equal(st.rows(np.arange(st.n_entries)), pre["entries"])


# ---------------------------------------------------------------------------
# partial RoPE: the rotation itself, its group law, relative positions only


def test_rope_is_a_complex_rotation_of_the_last_64_dims():
    r = rng(70)
    x = r.standard_normal((5, 3, 160))
    pos = r.integers(0, 1 << 21, (5, 3))
    base = 10000.0
    y = O.rope(x, pos, base)
    assert np.array_equal(y[..., :96], x[..., :96])
    # pair i as the complex number x[2i] + i x[2i+1], multiplied by e^{i pos w_i}
    z = x[..., 96::2] + 1j * x[..., 97::2]
    w = np.exp(-math.log(base) * np.arange(32) / 32.0)
    zr = z * np.exp(1j * (pos[..., None] * w))
    assert np.allclose(y[..., 96::2], zr.real, rtol=0, atol=1e-8)
    assert np.allclose(y[..., 97::2], zr.imag, rtol=0, atol=1e-8)
    assert np.array_equal(O.rope(x, pos, 0.0), x)
    assert np.array_equal(O.rope(x, 0, base), x)
    # the lowest pair turns by pos radians, the highest by pos * base^(-31/32)
    assert np.allclose(O.rope(np.r_[np.zeros(62), 1.0, 0.0], 0.5, base)[62:],
                       [math.cos(0.5 * base ** (-31 / 32)), math.sin(0.5 * base ** (-31 / 32))])
    assert np.allclose(O.rope(np.r_[1.0, 0.0, np.zeros(62)], 0.5, base)[:2], [math.cos(0.5), math.sin(0.5)])


def test_rope_group_law_and_lengths():
    r = rng(71)
    x = r.standard_normal((4, 128))
    base, a, b = 500.0, 123457, -98765
    assert np.allclose(O.rope(O.rope(x, a, base), b, base), O.rope(x, a + b, base), rtol=0, atol=1e-9)
    assert np.allclose(O.rope(O.rope(x, a, base), -a, base), x, rtol=0, atol=1e-9)
    y = O.rope(x, a, base)
    assert np.allclose(y[:, 64::2] ** 2 + y[:, 65::2] ** 2, x[:, 64::2] ** 2 + x[:, 65::2] ** 2)


def test_rope_scores_depend_on_relative_position_only():
    r = rng(72)
    q, k = r.standard_normal(96), r.standard_normal(96)
    base = 10000.0
    for t, s in [(10, 3), (1 << 20, 17), (5, 5)]:
        d0 = O.rope(q, t, base) @ O.rope(k, s, base)
        for shift in (1, 1000, 777777):
            assert abs(O.rope(q, t + shift, base) @ O.rope(k, s + shift, base) - d0) < 1e-9
    # without the turn the score is the plain dot product at equal positions
    assert abs(O.rope(q, 9, base) @ O.rope(k, 9, base) - q @ k) < 1e-12


def test_core_attention_with_rope_keeps_relative_positions_only():
    r = rng(73)
    H, c, base, t = 3, 128, 10000.0, 23
    q = r.standard_normal((H, c))
    raw = [O.rmsnorm(r.standard_normal((6, c))), O.rmsnorm(r.standard_normal((4, c)))]
    pos = [np.array([3, 7, 11, 15, 19, 23]), np.array([20, 21, 22, 23])]

    def run(shift):
        parts = [O.rope(x, p + shift, base) for x, p in zip(raw, pos)]
        return O.core_attention(q, parts, 0.1, 1e-6, t + shift, sink=np.array([0.1, -2.0, 1.0]),
                                rope_base=base)

    o0, l0 = run(0)
    for shift in (5, 4096, 999999):
        o1, l1 = run(shift)
        assert np.allclose(o1, o0, rtol=0, atol=1e-9) and np.allclose(l1, l0, rtol=0, atol=1e-9)
    # a single row stored at position s: the output is that row turned by s - t
    row = O.rmsnorm(r.standard_normal(c))
    o, _ = O.core_attention(q, [O.rope(row, 40, base)[None]], 0.1, 1e-6, 55, rope_base=base)
    assert np.allclose(o, np.broadcast_to(O.rope(row, -15, base), (H, c)), rtol=0, atol=1e-12)
    # base 0 is the attention without positions
    o_off, _ = O.core_attention(q, raw, 0.1, 1e-6, t)
    o_ref, _ = O.merge([O.attend(O.rmsnorm(q), x, 0.1) for x in raw])
    assert np.array_equal(o_off, o_ref)


def test_rope_error_bound_covers_fp32_rotation():
    r = rng(74)
    x = O.rmsnorm(r.standard_normal((200, 128)))
    pos = r.integers(0, 1 << 21, 200)
    exact = O.rope(x, pos, 10000.0)
    # float32 rotation with float32 cos/sin of the float64-reduced angle
    i = np.arange(32)
    a = pos[:, None] * 10000.0 ** (-2.0 * i / 64)
    a = np.remainder(a + np.pi, 2 * np.pi) - np.pi
    cs, sn = np.cos(a.astype(np.float32)).astype(np.float32), np.sin(a.astype(np.float32)).astype(np.float32)
    xf = x.astype(np.float32)
    ye = xf[:, 64::2] * cs - xf[:, 65::2] * sn
    yo = xf[:, 64::2] * sn + xf[:, 65::2] * cs
    got = xf.astype(np.float64).copy()
    got[:, 64::2], got[:, 65::2] = ye, yo
    bnd = O.rope_error_bound(exact, np.abs(xf.astype(np.float64) - x))
    assert np.all(np.abs(got - exact) <= bnd)


# ---------------------------------------------------------------------------
# grouped output projection


def test_grouped_projection_matches_brute_force():
    r = rng(80)
    T, n_h, c, g, d_g, d = 2, 6, 4, 3, 5, 7
    o = r.standard_normal((T, n_h, c))
    W_g = r.standard_normal((g, d_g, (n_h // g) * c))
    W_o = r.standard_normal((d, g * d_g))
    out, z = O.grouped_output_projection(o, W_g, W_o)
    for t in range(T):
        bo, bz = brute.grouped_projection(o[t].tolist(), W_g.tolist(), W_o.tolist())
        assert np.allclose(out[t], bo, rtol=1e-12, atol=1e-12)
        assert np.allclose(z[t], bz, rtol=1e-12, atol=1e-12)


def test_grouped_projection_structure():
    r = rng(81)
    T, n_h, c, g, d_g = 3, 8, 16, 4, 6
    o = r.standard_normal((T, n_h, c))
    W_g = r.standard_normal((g, d_g, (n_h // g) * c))
    # one group: two plain matrix products of the flattened heads
    W_o1 = r.standard_normal((9, d_g))
    Wg1 = r.standard_normal((1, d_g, n_h * c))
    out1, z1 = O.grouped_output_projection(o, Wg1, W_o1)
    assert np.allclose(out1, (o.reshape(T, -1) @ Wg1[0].T) @ W_o1.T)
    # with W_o the identity, perturbing the heads of group j moves only z's block j
    I = np.eye(g * d_g)
    base, zb = O.grouped_output_projection(o, W_g, I)
    assert np.array_equal(base, zb)
    for j in range(g):
        o2 = o.copy()
        o2[:, j * (n_h // g):(j + 1) * (n_h // g)] += 1.0
        moved, _ = O.grouped_output_projection(o2, W_g, I)
        diff = np.abs(moved - base).reshape(T, g, d_g).max(axis=(0, 2))
        assert diff[j] > 0 and np.all(np.delete(diff, j) == 0)
    # linear in the attention output
    W_o = r.standard_normal((5, g * d_g))
    a, _ = O.grouped_output_projection(o, W_g, W_o)
    b, _ = O.grouped_output_projection(2.5 * o, W_g, W_o)
    assert np.allclose(b, 2.5 * a)
    # the bf16 intermediate is the round-to-nearest-even of the exact one
    _, zx = O.grouped_output_projection(o, W_g, W_o)
    _, zr = O.grouped_output_projection(o, W_g, W_o, z_fmt="bf16")
    assert np.array_equal(zr, O.round_to(zx, "bf16"))


def test_matmul_error_bound_covers_fp32_accumulation():
    r = rng(82)
    a = O.round_to(r.standard_normal((4, 3000)), "bf16")
    b = O.round_to(r.standard_normal((5, 3000)), "bf16")
    exact = a @ b.T
    f32 = np.zeros((4, 5), np.float32)
    for k in range(3000):          # sequential float32 accumulation
        f32 += (a[:, k:k + 1].astype(np.float32) * b[:, k].astype(np.float32)[None, :])
    bnd = O.matmul_error_bound(np.abs(a), np.abs(b), 3000)
    assert np.all(np.abs(f32.astype(np.float64) - exact) <= bnd)


# ---------------------------------------------------------------------------
# score error bound and the pages' hyperparameters


def test_score_error_bound_covers_fp32_evaluation():
    r = rng(50)
    q = r.standard_normal((3, 64, 128))
    k = r.standard_normal((200, 128))
    w = r.random((3, 64))
    exact = O.index_scores(q, k, w, np.full(3, 200))
    q32, k32, w32 = (torch.from_numpy(a.astype(np.float32)) for a in (q, k, w))
    dots = torch.einsum("thd,sd->ths", q32, k32)
    f32 = torch.einsum("th,ths->ts", w32, torch.relu(dots)).double().numpy()
    q32d, k32d = q32.double().numpy(), k32.double().numpy()
    bound = O.score_error_bound(q32d, k32d, w32.double().numpy())
    exact32 = O.index_scores(q32d, k32d, w32.double().numpy(), np.full(3, 200))
    assert np.all(np.abs(f32 - exact32) <= bound)
    assert np.all(bound < 1e-3 * np.abs(exact).max())


def test_pages_hyperparameters():
    from synth.configs import CSA_DECODE_1M, HCA_DECODE, HYBRID_DECODE_1M, OUT_PROJ_DECODE, OUT_PROJ_PREFILL
    g = json.load(open(os.path.join(GOLD, "hyperparams.json")))
    cfg = CSA_DECODE_1M
    assert cfg.m == g["csa_rate_m"]["value"] and cfg.k == g["csa_topk"]["value"]
    assert cfg.H_I == g["indexer_heads"]["value"] and cfg.d_I == g["indexer_head_dim"]["value"]
    assert cfg.n_win == g["window_n_win"]["value"] and cfg.c == g["head_dim_c"]["value"]
    assert HCA_DECODE.m == g["hca_rate_m_prime"]["value"] == HYBRID_DECODE_1M.m_hca
    assert HYBRID_DECODE_1M.rope_dims == g["rope_dims"]["value"]
    assert cfg.ctx == g["context_tokens"]["value"]
    assert np.lcm(cfg.m, HCA_DECODE.m) == g["cache_block_tokens_lcm"]["value"]
    assert cfg.k == g["entries_attended_at_1m"]["value"]
    assert OUT_PROJ_DECODE.d == OUT_PROJ_PREFILL.d == g["hidden_dim_d_v4_pro"]["value"]
    assert OUT_PROJ_DECODE.c == g["head_dim_c"]["value"]
    assert int(O.visible([cfg.ctx - 1], cfg.m, 10 ** 9)[0]) == 262144


def test_compress_error_bound_covers_fp32_pooling():
    """The bound covers an fp32 evaluation of the pooling + RMSNorm (emulated with
    numpy float32 arithmetic) and is far below an ulp of bf16 at unit scale."""
    r = rng(60)
    m, c = 4, 256
    C, Z = r.standard_normal((64, c)), r.standard_normal((64, c))
    P = r.standard_normal((8, c)) * 0.1
    exact = O.rmsnorm(O.compress(C, Z, P, m, True))
    bound = O.compress_error_bound(C, Z, P, m, True)
    C32, Z32, P32 = (a.astype(np.float32) for a in (C, Z, P))
    cand = np.concatenate([np.concatenate([np.zeros((1, m, c), np.float32), C32.reshape(-1, m, c)[:-1]], 0),
                           C32.reshape(-1, m, c)], 1)
    lg = np.concatenate([np.concatenate([np.full((1, m, c), -np.inf, np.float32), Z32.reshape(-1, m, c)[:-1]], 0),
                         Z32.reshape(-1, m, c)], 1) + P32[None]
    e = np.exp(lg - lg.max(1, keepdims=True)).astype(np.float32)
    E32 = ((e * cand).sum(1, dtype=np.float32) / e.sum(1, dtype=np.float32)).astype(np.float32)
    y32 = E32 / np.sqrt((E32 * E32).mean(-1, keepdims=True, dtype=np.float32) + np.float32(1e-6))
    assert np.all(np.abs(y32 - exact) <= bound)
    assert bound.max() < 1e-4


# ---------------------------------------------------------------------------
# the chunked-prefill branch and the decode state rebuilt from its physical layout


@pytest.mark.parametrize("mode,m,rope_base", [("csa", 4, 0.0), ("csa", 4, 10000.0), ("hca", 8, 0.0),
                                               ("hca", 8, 300.0)])
def test_chunked_prefill_equals_one_shot_and_brute_force(mode, m, rope_base):
    """A prefill of n1 + n2 tokens in one call equals the prefill of the last n2
    tokens at pos0 = n1 fed the first part's stored entries (cache_prefix), its
    last n_win - 1 stored window rows (win_prefix) and, for CSA, its last block's
    candidates and gate logits (prevC, prevZ: the overlap with the previous block
    reaches across the chunk boundary, "DeepSeek V4 Architecture Tricks",
    compressed-KV tricks).  Entries, window rows, selections, outputs and lse are
    bit-identical; the chunk also equals the brute-force twin of the whole
    sequence (which turns entry s at (s+1)m-1 under RoPE, so the chunk's entry
    positions carry the prefix offset)."""
    n1, n2, H, n_win, k, kv = 24, 16, 2, 6, 3, "bf16"
    c = 80 if rope_base else 16
    n = n1 + n2
    d = _tiny_layer_inputs(70 + m, n=n, c=c, H=H, m=m)
    P = d["P"][: 2 * m if mode == "csa" else m]
    tau = 1 / math.sqrt(c)
    kw = dict(mode=mode, m=m, k=k, n_win=n_win, tau=tau, eps=1e-6, kv_fmt=kv, out_fmt="f32",
              rope_base=rope_base)
    full = O.prefill_layer(pos0=0, C=d["C"], Z=d["Z"], P=P, q=d["q"], cache_prefix=np.zeros((0, c)),
                           qI=d["qI"], kI=d["kI"], w=d["w"], **kw)
    csa = mode == "csa"
    chunk = O.prefill_layer(pos0=n1, C=d["C"][n1:], Z=d["Z"][n1:], P=P, q=d["q"][n1:],
                            cache_prefix=full["entries"][: n1 // m],
                            prevC=d["C"][n1 - m:n1] if csa else None,
                            prevZ=d["Z"][n1 - m:n1] if csa else None,
                            win_prefix=full["window"][n1 - (n_win - 1):n1],
                            qI=d["qI"][n1:], kI=d["kI"], w=d["w"][n1:], **kw)
    assert np.array_equal(chunk["entries"], full["entries"][n1 // m:])
    assert np.array_equal(chunk["window"], full["window"][n1:])
    assert np.array_equal(chunk["out"], full["out"][n1:])
    assert np.array_equal(chunk["lse"], full["lse"][n1:])
    if csa:
        assert np.array_equal(chunk["idx"], full["idx"][n1:])
    rk = (lambda row: O.round_to(np.array(row), kv).tolist())
    outs, idxs, entries = brute.layer(mode=mode, m=m, k=k, n_win=n_win, tau=tau, eps=1e-6,
                                      C=d["C"].tolist(), Z=d["Z"].tolist(), P=P.tolist(),
                                      q=d["q"].tolist(), qI=d["qI"].tolist(), kI=d["kI"].tolist(),
                                      w=d["w"].tolist(), round_kv=rk, rope_base=rope_base)
    assert np.allclose(chunk["entries"], np.array(entries)[n1 // m:], rtol=1e-12, atol=1e-12)
    if csa:
        assert np.array_equal(chunk["idx"], np.array(idxs)[n1:])
    assert np.allclose(chunk["out"], np.array(outs)[n1:], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("mode,m,L", [("csa", 4, 37), ("csa", 4, 40), ("csa", 4, 2), ("csa", 4, 5),
                                      ("hca", 8, 45), ("hca", 8, 40), ("hca", 8, 3)])
def test_decode_state_from_physical_layout_equals_stepped_state(mode, m, L):
    """oracle_decode_state rebuilds a sequence's logical decode state from the
    physical layout the library's header documents -- the token at position p
    in tail row ((p/m) % 2) * m + p % m (CSA: the current and the previous
    block) or p % m (HCA), its stored window row in ring slot p % n_win, entries
    in cache rows 0 .. L/m - 1, L in the token counter.  Laid out here from
    tokens stepped through a DecodeState from empty, it must give that state
    back, and one more step from either state must give the same results."""
    from oracle.workloads import oracle_decode_state
    from synth.configs import TINY_CSA_PREFILL
    c, n_win, H, HI, dI, k = 16, 6, 2, 3, 8, 3
    r = rng(80 + L + m)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731  (stored exactly in f32)
    C, Z = f32(r.standard_normal((L + 1, c))), f32(r.standard_normal((L + 1, c)))
    q = r.standard_normal((L + 1, H, c))
    qI, kI, w = r.standard_normal((L + 1, HI, dI)), r.standard_normal(((L + 1) // m + 1, dI)), r.random((L + 1, HI))
    P = f32(r.standard_normal((2 * m if mode == "csa" else m, c)) * 0.1)
    kw = dict(tau=0.25, eps=1e-6, kv_fmt="f32", out_fmt="f32")
    ckw = (lambda t: dict(k=k, qI=qI[t], kI=kI, w=w[t])) if mode == "csa" else (lambda t: {})
    ref = O.DecodeState(mode=mode, m=m, n_win=n_win, c=c)
    stored_win = []
    for t in range(L):
        res = O.decode_step(ref, tokC=C[t], tokZ=Z[t], P=P, q=q[t], **kw, **ckw(t))
        stored_win.append(res["window_row"])
    # the physical layout, written from the header's formulas
    T = 2 * m if mode == "csa" else m
    tailC, tailZ = np.zeros((T, c), np.float32), np.zeros((T, c), np.float32)
    ring = np.zeros((n_win, c), np.float32)
    for p in range(L):
        row = ((p // m) % 2) * m + p % m if mode == "csa" else p % m
        tailC[row], tailZ[row] = C[p], Z[p]
        ring[p % n_win] = stored_win[p]
    n_ent = L // m
    cache = np.zeros((n_ent + 2, c), np.float32)
    cache[:n_ent] = ref.rows(np.arange(n_ent))
    d = {"kind": "C" if mode == "csa" else "H", "m": m, "n_tokens": np.array([L], np.int32),
         "tailC": tailC[None], "tailZ": tailZ[None], "ring": ring[None], "cache": cache[None]}
    cfg = TINY_CSA_PREFILL.with_(c=c, n_win=n_win, io_dtype="f32", kv_dtype="f32")
    st = oracle_decode_state(cfg, d, 0)
    assert st.L == ref.L and st.n_entries == ref.n_entries
    for a, b in zip(st.cur, ref.cur):
        assert np.array_equal(a.reshape(-1, c), b.reshape(-1, c))
    if mode == "csa":                    # HCA pools no previous block (its prev is unused)
        assert (st.prev is None) == (ref.prev is None)
    if mode == "csa" and ref.prev is not None:
        for a, b in zip(st.prev, ref.prev):
            assert np.array_equal(a.reshape(-1, c), b.reshape(-1, c))
    assert np.array_equal(np.array(list(st.window)).reshape(-1, c), np.array(list(ref.window)).reshape(-1, c))
    assert np.array_equal(st.rows(np.arange(n_ent)), ref.rows(np.arange(n_ent)))
    a = O.decode_step(st, tokC=C[L], tokZ=Z[L], P=P, q=q[L], **kw, **ckw(L))
    b = O.decode_step(ref, tokC=C[L], tokZ=Z[L], P=P, q=q[L], **kw, **ckw(L))
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])
    assert (a["new_entry"] is None) == (b["new_entry"] is None)
    if a["new_entry"] is not None:
        assert np.array_equal(a["new_entry"], b["new_entry"])
    if mode == "csa":
        assert np.array_equal(a["idx"], b["idx"])


def _pool_gpu_arith(C, Z, P, m, overlap, r):
    """The compressor's float32 arithmetic with the error model of its hardware
    functions: per channel, an online softmax over the candidates in time order
    (running maximum; every rescale and weight through exp(x) = 2^(x log2 e) with
    the product rounded to float32 and the exp2 result off by one ulp in a random
    direction), the pooled value times a reciprocal of the weight sum (one ulp),
    then RMSNorm with a reciprocal square root (one ulp).  Entry 0 of a CSA chunk
    has no previous block."""
    f = np.float32
    n, c = C.shape
    nb = n // m
    C32, Z32, P32 = C.astype(f), Z.astype(f), P.astype(f)
    log2e = f(1.4426950408889634)

    def ulp_off(x):
        s = r.choice([-1.0, 1.0], size=x.shape).astype(f)
        return (x * (f(1) + s * f(2.0 ** -23))).astype(f)

    def exp_hw(x):
        y = (x.astype(f) * log2e).astype(f)
        return ulp_off(np.exp2(y.astype(np.float64)).astype(f))

    out = np.zeros((nb, c), f)
    for s in range(nb):
        cand = []
        if overlap and s > 0:
            cand += [(C32[(s - 1) * m + i], Z32[(s - 1) * m + i] + P32[i]) for i in range(m)]
        slot0 = m if overlap else 0
        cand += [(C32[s * m + i], (Z32[s * m + i] + P32[slot0 + i]).astype(f)) for i in range(m)]
        mx = np.full(c, -np.inf, f)
        sm, acc = np.zeros(c, f), np.zeros(c, f)
        for cv, zv in cand:
            nm = np.maximum(mx, zv)
            with np.errstate(invalid="ignore"):
                sc = np.where(np.isfinite(mx), exp_hw(mx - nm), f(0))
            e = exp_hw(zv - nm)
            sm = (sm * sc + e).astype(f)
            acc = (acc * sc + e * cv).astype(f)
            mx = nm
        rcp = ulp_off((f(1) / sm).astype(f))
        out[s] = (acc * rcp).astype(f)
    ss = (out * out).sum(-1, dtype=f)
    rs = ulp_off((f(1) / np.sqrt(ss / f(c) + f(1e-6))).astype(f))
    return (out * rs[:, None]).astype(np.float64)


@pytest.mark.parametrize("overlap,m,zscale", [(True, 4, 1.0), (False, 128, 1.0), (True, 4, 3.0),
                                              (False, 128, 2.0)])
def test_compress_error_bound_covers_the_kernel_arithmetic(overlap, m, zscale):
    """compress_error_bound's gamma(2W + 32): 2W units for the W rescaling
    multiply-adds and W products of a weight's path, plus 32 units for the
    exponentials (exp(x) as 2^(x log2 e) carries about |x| units from the
    rounded product, and along any weight's path the arguments of its exps sum
    to at most twice the spread of the window's logits) and for the reciprocal
    and reciprocal square root.  Checked against an emulation of the kernel's
    float32 operation order with one-ulp hardware functions, at the workloads'
    logit spread (gate logits N(0,1), bias N(0, 0.1^2)) and beyond it."""
    r = rng(90 + m)
    c = 256
    n = 8 * m
    C = r.standard_normal((n, c))
    Z = r.standard_normal((n, c)) * zscale
    P = r.standard_normal((2 * m if overlap else m, c)) * 0.1
    C, Z, P = (a.astype(np.float32).astype(np.float64) for a in (C, Z, P))
    exact = O.rmsnorm(O.compress(C, Z, P, m, overlap))
    bound = O.compress_error_bound(C, Z, P, m, overlap)
    for trial in range(3):
        y = _pool_gpu_arith(C, Z, P, m, overlap, rng(trial))
        err = np.abs(y - exact)
        assert np.all(err <= bound), f"trial {trial}: worst err/bound {(err / bound).max():.3g}"
