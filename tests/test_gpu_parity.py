"""GPU parity of every step of the path against the float64 oracle, through the
C ABI.  Tolerances: outputs within 1e-4 (fp32 I/O) or 2e-2 (bf16 I/O) max
absolute error; stored entries and window rows within one ulp of their storage
format plus the oracle's fp32-evaluation bound (fp32: 1e-5); indexer scores within the fp32 evaluation bound; top-k
indices bit-exact on the select stage and on every certified row."""
import numpy as np
import pytest
import torch

import oracle_side as OS
from long_context_attention_14_amd import ops, pipeline
from oracle import lca_oracle as O
from synth import encode as enc
from synth import gen
from synth.configs import (CSA_DECODE_1M, CSA_PREFILL_CHUNK, HCA_DECODE, HYBRID_DECODE_1M,
                           TINY_CSA_PREFILL)

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
# lse: the fp32 path is exact to rounding; the bf16 path feeds the MFMA with the
# normalised query rounded to bf16, which moves each logit tau*q.k by at most
# 2^-9 * tau * |q| |k| = 2^-9 * sqrt(c) for RMS-normalised q and k (c = 512),
# and rounds P to bf16 (at most 2^-9 relative in the denominator).
LSE_TOL = {"f32": 1e-5, "bf16": 2.0 ** -9 * 512 ** 0.5 * 1.01 + 2.0 ** -8}


def say(*a):
    print(*a, flush=True)


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def out_f64(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return host(t).astype(np.float64)


# ---------------------------------------------------------------------------
# top-k on adversarial score arrays (select stage, bit-exact)


def _scores(kind, rows, N, rng):
    if kind == "ties":
        s = rng.integers(-3, 4, (rows, N)).astype(np.float32)
        s[:, ::7] = -0.0
    elif kind == "normal":
        s = rng.standard_normal((rows, N)).astype(np.float32)
    elif kind == "constant":
        s = np.full((rows, N), 1.5, np.float32)
    elif kind == "special":
        s = rng.standard_normal((rows, N)).astype(np.float32)
        s[:, ::5] = np.nan
        s[:, 1::11] = -np.inf
        s[:, 2::13] = np.inf
        s[:, 3::17] = -0.0
        s[:, 4::17] = 0.0
        s[:, 6::19] = np.float32(1e-45)     # denormal
    else:
        raise ValueError(kind)
    return s


@pytest.mark.parametrize("N,k,kind", [
    (300, 32, "ties"), (4097, 1024, "normal"), (36864, 1024, "ties"), (20000, 4096, "special"),
    (36865, 1024, "normal"), (100003, 1024, "ties"), (262148, 1024, "special"),
    (262148, 1024, "constant"), (70000, 1, "normal")])
def test_topk_select_stage_bit_exact(N, k, kind):
    say(f"topk N={N} k={k} kind={kind}")
    rng = np.random.default_rng(N + k)
    B, n_q = 2, 3
    s = _scores(kind, B * n_q, N, rng)
    vis = np.array([0, max(0, k - 1), k, min(N, k + 1), N, N - 3])[: B * n_q]
    q_pos = T((vis - 1).astype(np.int32).reshape(B, n_q))
    n_ent = T(np.full(B, N, np.int32))
    idx = torch.full((B, n_q, k), -7, dtype=torch.int32, device=DEV)
    ops.lca_topk(B, n_q, N, T(s.reshape(B, n_q, N)), q_pos, 1, n_ent, k, idx)
    got = host(idx).reshape(B * n_q, k)
    for r in range(B * n_q):
        want = O.topk(s[r:r + 1].astype(np.float64), [vis[r]], k)[0]
        assert np.array_equal(got[r], want), f"row {r} vis {vis[r]}"


@pytest.mark.parametrize("N,k,kind", [
    (300, 32, "ties"), (36864, 1024, "normal"), (36864, 1024, "ties"), (20000, 1024, "special"),
    (100003, 1024, "normal"), (262148, 1024, "ties"), (70000, 1, "normal")])
def test_topk_bf16_select_stage_bit_exact(N, k, kind):
    """The BF16-score selector over bf16 arrays: equal to the oracle's stable
    top-k of the same bf16 values (rounding normal scores to bf16 makes ties
    common at the threshold)."""
    say(f"topk bf16 N={N} k={k} kind={kind}")
    rng = np.random.default_rng(N + 3 * k)
    B, n_q = 2, 3
    s16 = enc.to_bf16_bits(_scores(kind, B * n_q, N, rng))
    s = O.decode(s16, "bf16")
    vis = np.array([0, max(0, k - 1), k, min(N, k + 1), N, N - 3])[: B * n_q]
    q_pos = T((vis - 1).astype(np.int32).reshape(B, n_q))
    n_ent = T(np.full(B, N, np.int32))
    idx = torch.full((B, n_q, k), -7, dtype=torch.int32, device=DEV)
    ops.lca_topk(B, n_q, N, T(s16.reshape(B, n_q, N)), q_pos, 1, n_ent, k, idx, score_fmt="bf16")
    got = host(idx).reshape(B * n_q, k)
    for r in range(B * n_q):
        want = O.topk(s[r:r + 1], [vis[r]], k)[0]
        assert np.array_equal(got[r], want), f"row {r} vis {vis[r]}"


def test_topk_random_shapes_bit_exact():
    """Seeded random shapes for both score formats and both top-k paths: N from
    1 to 300000, k from 1 to 4096, visible lengths anywhere in [0, N], scores
    drawn from tie-heavy distributions (small integers, a few distinct values,
    normal values rounded to a coarse grid) as well as plain normal ones; every
    row equal to the oracle's stable top-k."""
    rng = np.random.default_rng(2024)
    for case in range(30):
        N = int(rng.choice([int(rng.integers(1, 2000)), int(rng.integers(2000, 40000)),
                            int(rng.integers(40000, 300000))]))
        k = int(rng.integers(1, 4097))
        rows = int(rng.integers(1, 5))
        kind = ["ints", "few", "grid", "normal"][case % 4]
        if kind == "ints":
            s = rng.integers(-5, 6, (rows, N)).astype(np.float32)
        elif kind == "few":
            s = rng.choice(np.array([-1.5, 0.25, 3.0], np.float32), (rows, N))
        elif kind == "grid":
            s = (np.round(rng.standard_normal((rows, N)) * 8) / 8).astype(np.float32)
        else:
            s = rng.standard_normal((rows, N)).astype(np.float32)
        fmt = "bf16" if case % 3 == 0 else "f32"
        if fmt == "bf16":
            s_dev = enc.to_bf16_bits(s)
            s_ref = O.decode(s_dev, "bf16")
        else:
            s_dev, s_ref = s, s.astype(np.float64)
        vis = rng.integers(0, N + 1, rows)
        vis[0] = N
        say(f"random topk case {case}: N={N} k={k} rows={rows} {kind} {fmt}")
        idx = torch.full((1, rows, k), -7, dtype=torch.int32, device=DEV)
        ops.lca_topk(1, rows, N, T(s_dev.reshape(1, rows, N)), T((vis - 1).astype(np.int32).reshape(1, rows)),
                     1, T(np.array([N], np.int32)), k, idx, score_fmt=fmt)
        got = host(idx).reshape(rows, k)
        for r in range(rows):
            want = O.topk(s_ref[r:r + 1], [int(vis[r])], k)[0]
            assert np.array_equal(got[r], want), f"case {case} row {r}: N={N} k={k} vis={vis[r]} {kind} {fmt}"


# ---------------------------------------------------------------------------
# indexer


@pytest.mark.parametrize("fmt,HI,dI", [("f32", 4, 32), ("f32", 16, 64), ("fp8", 64, 128),
                                       ("mxfp4", 64, 128)])
def test_indexer_scores_within_bound(fmt, HI, dI):
    say(f"indexer {fmt} {HI}x{dI}")
    rng = np.random.default_rng(7)
    B, n_q, N, m = 2, 3, 5003, 4
    qf = rng.standard_normal((B, n_q, HI, dI))
    kf = rng.standard_normal((B, N, dI))
    w = rng.random((B, n_q, HI)).astype(np.float32)
    if fmt == "mxfp4":
        qb, qs = enc.to_mxfp4(qf)
        kb, ks = enc.to_mxfp4(kf)
        qd, kd = O.decode_mxfp4(qb, qs), O.decode_mxfp4(kb, ks)
        qs_t, ks_t = T(qs), T(ks)
    else:
        qb, kb = enc.encode(qf, fmt), enc.encode(kf, fmt)
        qd, kd = O.decode(qb, fmt), O.decode(kb, fmt)
        qs_t = ks_t = None
    pos = np.array([[3, 100, 20011], [4 * N + 50, 0, 9999]], np.int32)[:, :n_q]
    n_ent = np.array([N, N - 17], np.int32)
    scores = torch.full((B, n_q, N), 12345.0, dtype=torch.float32, device=DEV)
    ops.lca_indexer_scores(B, n_q, HI, dI, fmt, T(qb), qs_t, T(kb), ks_t, N, T(w), T(pos), m,
                           T(n_ent), scores)
    got = host(scores)
    for b in range(B):
        for t in range(n_q):
            vis = int(O.visible([pos[b, t]], m, n_ent[b])[0])
            ref = O.index_scores(qd[b, t][None], kd[b, :vis], w[b, t][None].astype(np.float64), [vis])[0]
            bnd = O.score_error_bound(qd[b, t][None], kd[b, :vis], w[b, t][None].astype(np.float64))[0]
            err = np.abs(got[b, t, :vis] - ref)
            assert np.all(err <= bnd + 1e-30), f"b{b} t{t}: err {err.max():.3g}"
            assert np.all(got[b, t, vis:] == 12345.0), "entries past vis were written"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_indexer_scores_many_rows(fmt):
    """Many query rows per sequence (the row-group kernel): 75 rows (a ragged last
    group of 8), 2000 entries (a ragged last tile), visible lengths from 0 to all
    entries mixed within each group."""
    say(f"indexer {fmt} many rows")
    rng = np.random.default_rng(11)
    B, n_q, N, m, HI, dI = 2, 75, 2000, 4, 64, 128
    qf = rng.standard_normal((B, n_q, HI, dI))
    kf = rng.standard_normal((B, N, dI))
    w = rng.random((B, n_q, HI)).astype(np.float32)
    if fmt == "mxfp4":
        qb, qs = enc.to_mxfp4(qf)
        kb, ks = enc.to_mxfp4(kf)
        qd, kd = O.decode_mxfp4(qb, qs), O.decode_mxfp4(kb, ks)
        qs_t, ks_t = T(qs), T(ks)
    else:
        qb, kb = enc.encode(qf, fmt), enc.encode(kf, fmt)
        qd, kd = O.decode(qb, fmt), O.decode(kb, fmt)
        qs_t = ks_t = None
    pos = rng.integers(-1, 4 * N + 40, (B, n_q)).astype(np.int32)
    pos[0, :8] = np.arange(8) * 3          # the first group: tiny visible lengths
    n_ent = np.array([N, N - 17], np.int32)
    scores = torch.full((B, n_q, N), 12345.0, dtype=torch.float32, device=DEV)
    ops.lca_indexer_scores(B, n_q, HI, dI, fmt, T(qb), qs_t, T(kb), ks_t, N, T(w), T(pos), m,
                           T(n_ent), scores)
    got = host(scores)
    for b in range(B):
        for t in range(n_q):
            vis = int(O.visible([pos[b, t]], m, n_ent[b])[0])
            if vis:
                ref = O.index_scores(qd[b, t][None], kd[b, :vis], w[b, t][None].astype(np.float64), [vis])[0]
                bnd = O.score_error_bound(qd[b, t][None], kd[b, :vis], w[b, t][None].astype(np.float64))[0]
                err = np.abs(got[b, t, :vis] - ref)
                assert np.all(err <= bnd + 1e-30), f"b{b} t{t}: err {err.max():.3g}"
            assert np.all(got[b, t, vis:] == 12345.0), f"b{b} t{t}: entries past vis were written"


@pytest.mark.parametrize("fmt,n_q", [("fp8", 3), ("fp8", 75), ("mxfp4", 75), ("f32", 3)])
def test_indexer_scores_bf16_is_rounded_fp32(fmt, n_q):
    """The bf16 scores are the round-to-nearest-even of the float32 scores the
    float32 entry point writes for the same inputs (one-row and row-group
    kernels); entries past vis are untouched."""
    say(f"indexer bf16 scores {fmt} n_q={n_q}")
    rng = np.random.default_rng(5 + n_q)
    HI, dI = (4, 32) if fmt == "f32" else (64, 128)
    B, N, m = 2, 3001, 4
    qf = rng.standard_normal((B, n_q, HI, dI))
    kf = rng.standard_normal((B, N, dI))
    w = rng.random((B, n_q, HI)).astype(np.float32)
    if fmt == "mxfp4":
        qb, qs = enc.to_mxfp4(qf)
        kb, ks = enc.to_mxfp4(kf)
        qs_t, ks_t = T(qs), T(ks)
    else:
        qb, kb = enc.encode(qf, fmt), enc.encode(kf, fmt)
        qs_t = ks_t = None
    pos = rng.integers(-1, 4 * N + 40, (B, n_q)).astype(np.int32)
    n_ent = np.array([N, N - 17], np.int32)
    s32 = torch.full((B, n_q, N), 12345.0, dtype=torch.float32, device=DEV)
    s16 = torch.full((B, n_q, N), 0x1234, dtype=torch.int16, device=DEV)
    args = (B, n_q, HI, dI, fmt, T(qb), qs_t, T(kb), ks_t, N, T(w), T(pos), m, T(n_ent))
    ops.lca_indexer_scores(*args, s32)
    ops.lca_indexer_scores(*args, s16, score_fmt="bf16")
    g32 = host(s32)
    g16 = host(s16).view(np.uint16)
    for b in range(B):
        for t in range(n_q):
            vis = int(O.visible([pos[b, t]], m, n_ent[b])[0])
            assert np.array_equal(g16[b, t, :vis], enc.to_bf16_bits(g32[b, t, :vis])), f"b{b} t{t}"
            assert np.all(g16[b, t, vis:] == 0x1234), f"b{b} t{t}: entries past vis were written"


# ---------------------------------------------------------------------------
# compressor and window KV


@pytest.mark.parametrize("mode,m,io,kv,prev,rope", [("csa", 4, "bf16", "bf16", True, 0.0),
                                                    ("csa", 4, "f32", "f32", False, 0.0),
                                                    ("hca", 128, "bf16", "bf16", False, 0.0),
                                                    ("csa", 4, "bf16", "fp8_bf16rope", True, 0.0),
                                                    ("hca", 8, "f32", "fp8_bf16rope", False, 0.0),
                                                    ("csa", 4, "bf16", "bf16", True, 10000.0),
                                                    ("csa", 4, "f32", "f32", False, 10000.0),
                                                    ("hca", 128, "bf16", "fp8_bf16rope", False, 160.0)])
def test_compress_entries(mode, m, io, kv, prev, rope):
    say(f"compress {mode} m={m} {io}->{kv} prev={prev} rope={rope}")
    rng = np.random.default_rng(11)
    B, c, n = 2, 512 if kv != "f32" else 128, 4 * m if m > 4 else 1028
    C = enc.encode(rng.standard_normal((B, n, c)), io)
    Z = enc.encode(rng.standard_normal((B, n, c)), io)
    W = 2 * m if mode == "csa" else m
    P = (rng.standard_normal((W, c)) * 0.1).astype(np.float32)
    pC = enc.encode(rng.standard_normal((B, m, c)), io) if prev else None
    pZ = enc.encode(rng.standard_normal((B, m, c)), io) if prev else None
    # with RoPE the chunk starts deep in the sequence (entry positions near 2^21)
    first = 3 if not rope else (1 << 21) // m
    N_cap = first + n // m + 2
    rb = ops.row_bytes(kv, c)
    cache = torch.zeros(B * N_cap * rb, dtype=torch.uint8, device=DEV)
    ops.lca_compress(mode, m, B, n, c, T(C), T(Z), io, T(pC) if prev else None,
                     T(pZ) if prev else None, T(P), cache, kv, N_cap, first, rope_base=rope)
    got = host(cache).reshape(B, N_cap, rb)
    assert np.all(got[:, :first] == 0) and np.all(got[:, first + n // m:] == 0)
    for b in range(B):
        E = O.compress(O.decode(C[b], io), O.decode(Z[b], io), P, m, mode == "csa",
                       O.decode(pC[b], io) if prev else None, O.decode(pZ[b], io) if prev else None)
        exact = O.rope(O.rmsnorm(E), O.entry_position(first + np.arange(n // m), m), rope)
        want = O.round_to(exact, kv)
        bound = O.compress_error_bound(O.decode(C[b], io), O.decode(Z[b], io), P, m, mode == "csa",
                                       O.decode(pC[b], io) if prev else None,
                                       O.decode(pZ[b], io) if prev else None)
        if rope:
            bound = O.rope_error_bound(exact, bound)
        gb = got[b, first:first + n // m]
        g = O.decode(gb.view(np.float32) if kv == "f32" else gb.view(np.uint16) if kv == "bf16" else gb, kv)
        OS.assert_within_ulp(g, want, kv, slack=bound, what=f"entries b{b}")


@pytest.mark.parametrize("io,kv,c,rope", [("bf16", "bf16", 512, 0.0), ("f32", "f32", 512, 0.0),
                                           ("bf16", "fp8_bf16rope", 512, 0.0),
                                           ("bf16", "bf16", 512, 10000.0), ("f32", "f32", 128, 10000.0),
                                           ("bf16", "fp8_bf16rope", 256, 1e6)])
def test_rmsnorm_rows(io, kv, c, rope):
    say(f"rmsnorm rows {io}->{kv} c={c} rope={rope}")
    rng = np.random.default_rng(12)
    B, n, ys = 3, 37, 50
    pos0 = (1 << 20) + 3 if rope else 0
    x = enc.encode(rng.standard_normal((B, n, c)) * 3, io)
    rb = ops.row_bytes(kv, c)
    y = torch.zeros(B * ys * rb, dtype=torch.uint8, device=DEV)
    ops.lca_rmsnorm_rows(B, n, c, T(x), io, y, kv, ys, pos0=pos0, rope_base=rope)
    got = host(y).reshape(B, ys, rb)
    for b in range(B):
        gb = got[b, :n]
        g = O.decode(gb.view(np.float32) if kv == "f32" else gb.view(np.uint16) if kv == "bf16" else gb, kv)
        exact = O.rope(O.rmsnorm(O.decode(x[b], io)), pos0 + np.arange(n), rope)
        slack = O.rope_error_bound(exact, 0.0) if rope else None
        OS.assert_within_ulp(g, O.round_to(exact, kv), kv, slack=slack, what=f"rows b{b}")
        assert np.all(got[b, n:] == 0)


# ---------------------------------------------------------------------------
# core attention alone at decode shapes: empty slots, ragged splits, window
# positions before 0, a running maximum that moves on every tile


def _as_bytes(enc_rows, fmt):
    return np.ascontiguousarray(enc_rows).view(np.uint8)


def _mqa_case(case, rng):
    c, H, n_win, eps = (128, 8, 128, 1e-6) if "_c128" in case else (512, 64, 128, 1e-6)
    tau = 1.0 / np.sqrt(c)
    kv = "fp8_bf16rope" if case.startswith("fp8") else "bf16"
    rope = 10000.0 if "_rope" in case else 0.0
    q_fmt = "f32" if "_f32q" in case else "bf16"
    case = case.split("_rope")[0].split("_f32q")[0].split("_c128")[0]
    if case == "rows300":                  # one split per row: the direct-output path
        B, N_cap, k, m = 300, 256, 128, 4
        q_pos = rng.integers(600, 2000, B) + (2 ** 21 if rope else 0)
        n_entries = np.minimum((q_pos + 1) // m, N_cap)
    elif case == "bf16_dense":             # HCA: every visible entry, many empty slots
        B, N_cap, k, m = 2, 700, 0, 128
        q_pos = np.array([300 * 128 + 5, 700 * 128 + 900])
        n_entries = np.array([300, 700])
    elif case.endswith("window_only"):     # no compressed entries at all (N_cap = 0), and
        B, N_cap, k, m = 3, 0, 0, 4        # windows that start before position 0
        q_pos = np.array([5, 70, 3000])
        n_entries = np.zeros(B, np.int64)
    else:                                  # CSA: k = 200 selected, -1 padded
        B, N_cap, k, m = 3, 5000, 200, 4
        q_pos = np.array([5, 4000, 20000]) + (2 ** 21 if rope else 0)
        n_entries = np.array([2, 1000, 5000])
    vis = np.minimum(np.minimum((q_pos + 1) // m, n_entries), N_cap)
    cache_f = rng.standard_normal((B, max(N_cap, 1), c))   # one unused row when N_cap = 0
    win_f = rng.standard_normal((B, n_win, c))
    q_f = rng.standard_normal((B, H, c))
    if case == "rows300":
        # rows aligned ever more with one query direction along the candidate
        # list (selected entries 0..127, then the window oldest first): the
        # logits climb by about 11 per 64-row tile, so the running maximum moves
        # on every tile
        u = rng.standard_normal(c)
        u /= np.linalg.norm(u)
        q_f = u[None, None, :] * np.sqrt(c) + 0.1 * rng.standard_normal((B, H, c))

        def aligned(cosv, shape):
            noise = rng.standard_normal(shape)
            noise -= (noise @ u)[..., None] * u
            noise /= np.linalg.norm(noise, axis=-1, keepdims=True)
            return np.sqrt(c) * (cosv[..., None] * u + np.sqrt(1 - cosv ** 2)[..., None] * noise)

        cache_f = aligned(np.broadcast_to(np.linspace(-1.0, 1.0, N_cap), (B, N_cap)), (B, N_cap, c))
        age = (np.arange(n_win)[None, :] - (q_pos[:, None] - (n_win - 1))) % n_win   # slot -> window order
        win_f = aligned(age / (n_win - 1.0), (B, n_win, c))
    if k:
        idx = np.full((B, k), -1, np.int32)
        for b in range(B):
            n = min(k, int(vis[b]))
            idx[b, :n] = np.sort(rng.choice(int(vis[b]), n, replace=False)) if case != "rows300" \
                else np.arange(n)
    else:
        idx = None
    sink = rng.standard_normal(H).astype(np.float32) if case in ("fp8_sink", "rows300") else None
    cache_e = enc.encode(cache_f, kv)
    win_e = enc.encode(win_f, kv)
    q_e = enc.encode(q_f, q_fmt)
    return dict(B=B, N_cap=N_cap, k=k, m=m, q_pos=q_pos.astype(np.int32), n_entries=n_entries.astype(np.int32),
                vis=vis, idx=idx, sink=sink, kv=kv, cache=cache_e, win=win_e, q=q_e, c=c, H=H,
                n_win=n_win, tau=tau, eps=eps, rope=rope, q_fmt=q_fmt)


@pytest.mark.parametrize("case", ["bf16_sparse", "fp8_sink", "bf16_dense", "rows300", "window_only",
                                  "fp8_window_only", "bf16_sparse_rope", "fp8_sink_rope", "rows300_rope",
                                  "rows300_f32q_rope", "bf16_sparse_f32q_rope", "bf16_sparse_c128_rope",
                                  "rows300_c128_rope"])
def test_sparse_mqa_decode_shapes(case):
    """Core attention alone: the decode kernel over splits with the merge, or one
    split writing the output itself (rows300), the float32-query kernel (_f32q)
    and the generic kernel (_c128: 8 heads x 128), with partial RoPE (_rope:
    the query turned to its position, the output turned back, at positions
    near 2^21)."""
    rng = np.random.default_rng(7)
    t = _mqa_case(case, rng)
    B, H, c, kv = t["B"], t["H"], t["c"], t["kv"]
    say(f"sparse MQA {case}: B={B} k={t['k']} N_cap={t['N_cap']} c={c} q={t['q_fmt']} rope={t['rope']}")
    out = torch.zeros(B * H * c, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(B * H, dtype=torch.float32, device=DEV)
    ops.lca_sparse_mqa(B, 1, H, c, T(t["q"]), t["q_fmt"], T(_as_bytes(t["cache"], kv)), kv, t["N_cap"],
                       None if t["idx"] is None else T(t["idx"]), t["k"], T(t["q_pos"]), t["m"],
                       T(t["n_entries"]), T(_as_bytes(t["win"], kv)), t["n_win"], 0, t["n_win"],
                       t["tau"], t["eps"], None if t["sink"] is None else T(t["sink"]), t["rope"], out,
                       "bf16", lse=lse)
    got = out_f64(out).reshape(B, H, c)
    got_lse = host(lse).reshape(B, H)
    check = range(B) if B <= 8 else [0, 1, 2, 150, 298, 299]
    for b in check:
        tp = int(t["q_pos"][b])
        if t["idx"] is None:
            sel = np.arange(int(t["vis"][b]))
        else:
            sel = t["idx"][b][(t["idx"][b] >= 0) & (t["idx"][b] < t["vis"][b])]
        wpos = O.window_positions(tp, t["n_win"])
        rows = np.concatenate([O.decode(t["cache"][b, sel], kv).reshape(-1, c),
                               O.decode(t["win"][b, wpos % t["n_win"]], kv).reshape(-1, c)])
        o_ref, lse_ref = O.core_attention(O.decode(t["q"][b], t["q_fmt"]), [rows], t["tau"], t["eps"], tp,
                                          sink=t["sink"], rope_base=t["rope"])
        err = np.abs(got[b] - o_ref).max()
        assert err <= OUT_TOL["bf16"], f"b{b}: out err {err:.3g}"
        lerr = np.abs(got_lse[b] - lse_ref).max()
        assert lerr <= LSE_TOL["bf16"], f"b{b}: lse err {lerr:.3g}"


# ---------------------------------------------------------------------------
# whole prefill layers


def _stored(arr_u8, fmt):
    return arr_u8.view(np.float32) if fmt == "f32" else arr_u8.view(np.uint16) if fmt == "bf16" else arr_u8


def run_prefill_parity(cfg, queries, check_entries=True):
    d = gen.prefill_inputs(cfg)
    layer = pipeline.PrefillLayer(cfg, d, DEV)
    layer.run()
    torch.cuda.synchronize()
    scores = host(layer.scores)
    idx = host(layer.idx)
    out = out_f64(layer.out)
    lse = host(layer.lse)
    kv, io = cfg.kv_dtype, cfg.io_dtype
    cache = layer.logical_cache()
    n_cert = 0
    for b in range(cfg.B):
        ref = OS.oracle_prefill(cfg, d, b, queries)
        if check_entries:
            g = O.decode(_stored(cache[b, d["n_prefix"]:], kv), kv)
            OS.assert_within_ulp(g, ref["entries"], kv, slack=ref["entries_bound"], what="new entries")
        kI_sc = d.get("kI_scale")
        kI = O.decode(d["kI"][b], cfg.idx_dtype, None if kI_sc is None else kI_sc[b])
        qI_rows = OS.LazyRows(d["qI"][b], cfg.idx_dtype,
                              None if d.get("qI_scale") is None else d["qI_scale"][b])
        for r, i in enumerate(queries):
            t = d["pos0"] + int(i)
            vis = int(O.visible([t], cfg.m, layer.N_cap)[0])
            bnd = O.score_error_bound(qI_rows[int(i)][None], kI[:vis], d["w"][b, i][None].astype(np.float64))[0]
            n_cert += OS.check_selection(idx[b, i], scores[b, i], ref["scores"][r], bnd, vis, cfg.k,
                                         what=f"b{b} q{i}")
        ref2 = OS.oracle_prefill(cfg, d, b, queries, idx_given=idx[b, queries])
        err = np.abs(out[b, queries] - ref2["out"])
        assert err.max() <= OUT_TOL[io], f"out err {err.max():.3g}"
        lerr = np.abs(lse[b, queries] - ref2["lse"])
        assert lerr.max() <= LSE_TOL[io], f"lse err {lerr.max():.3g}"
    say(f"{cfg.name}: {n_cert} of {cfg.B * len(queries)} rows certified")
    return layer


def test_tiny_csa_prefill_end_to_end():
    say("tiny CSA prefill fp32")
    run_prefill_parity(TINY_CSA_PREFILL, np.arange(TINY_CSA_PREFILL.n_new))


def test_csa_prefill_chunk_reduced():
    cfg = CSA_PREFILL_CHUNK.with_(ctx=8192, n_new=1024)
    say(f"prefill {cfg.ctx}+{cfg.n_new}")
    q = np.concatenate([np.arange(0, 1024, 37), [1023]])
    run_prefill_parity(cfg, q)


def test_tiny_csa_prefill_end_to_end_rope():
    cfg = TINY_CSA_PREFILL.with_(rope_base=10000.0)
    say("tiny CSA prefill fp32 with partial RoPE")
    run_prefill_parity(cfg, np.arange(cfg.n_new))


def test_csa_prefill_chunk_reduced_rope():
    cfg = CSA_PREFILL_CHUNK.with_(ctx=8192, n_new=1024, rope_base=10000.0)
    say(f"prefill {cfg.ctx}+{cfg.n_new} with partial RoPE")
    q = np.concatenate([np.arange(0, 1024, 37), [1023]])
    run_prefill_parity(cfg, q)


def test_csa_prefill_chunk_full_size_sampled():
    cfg = CSA_PREFILL_CHUNK
    say("prefill chunk 8192 on 131072, sampled rows")
    q = np.array([0, 1, 2, 3, 1000, 4095, 4096, 8188, 8189, 8190, 8191])
    run_prefill_parity(cfg, q, check_entries=True)


# ---------------------------------------------------------------------------
# decode steps


def _gpu_decode_scores(layer, cfg, d, pos):
    """Float32 index scores of each sequence's decode query at position pos[b]
    (after the step's append), written by lca_indexer_scores from the layer's own
    indexer inputs.  The decode step's selection (the fused indexer + selection
    kernel for long rows, the score-writing kernel for short ones) scores every
    entry with the same MFMA tiles and the same reduction order, so these are
    the scores it selected from; the select stage is checked on them bit for
    bit."""
    m, B = d["m"], cfg.B
    pos = np.asarray(pos, np.int64).reshape(B)
    n_ent = ((pos + 1) // m).astype(np.int32)
    scores = torch.full((B, 1, layer.N_cap), float("nan"), dtype=torch.float32, device=DEV)
    ops.lca_indexer_scores(B, 1, cfg.H_I, cfg.d_I, cfg.idx_dtype, layer.qI, layer.qI_scale, layer.kI,
                           layer.kI_scale, layer.N_cap, layer.w, T(pos.astype(np.int32).reshape(B, 1)),
                           m, T(n_ent), scores)
    return host(scores).reshape(B, layer.N_cap)


def _check_decode_selection(cfg, d, b, idx_row, gpu_scores_row, oracle_scores, p, kI_rows=None,
                            what=""):
    """Selection parity of one decode row (every row, certified or not): the select
    stage bit-exact on the GPU's own float32 scores, those scores within the fp32
    evaluation bound of the oracle's, and the selection equal to the oracle's on a
    certified row, else holding every clear winner and no clear loser.  Returns
    True when the row was certified."""
    m = d["m"]
    vis = (p + 1) // m
    sc = d.get("kI_scale")
    if kI_rows is None:
        kI_rows = O.decode(d["kI"][b, :vis], cfg.idx_dtype, None if sc is None else sc[b, :vis])
    qI = O.decode(d["qI"][b], cfg.idx_dtype, None if d.get("qI_scale") is None else d["qI_scale"][b])
    bnd = O.score_error_bound(qI[None], kI_rows[:vis], d["w"][b][None].astype(np.float64))[0]
    return OS.check_selection(idx_row, gpu_scores_row[:vis], np.asarray(oracle_scores)[:vis], bnd, vis,
                              cfg.k, what=what)


def _decode_parity(cfg, d, seqs, layer=None):
    if layer is None:
        layer = pipeline.DecodeLayer(cfg, d, DEV)
    layer.step()
    torch.cuda.synchronize()
    out = out_f64(layer.out)
    lse = host(layer.lse)
    idx = host(layer.idx)
    ntok = host(layer.n_tokens)
    io, kv, m = cfg.io_dtype, cfg.kv_dtype, d["m"]
    rb = ops.row_bytes(kv, cfg.c)
    cache = layer.logical_cache()
    ring = host(layer.ring).view(np.uint8).reshape(cfg.B, cfg.n_win, rb)
    assert np.array_equal(ntok, d["n_tokens"] + 1)
    csa = d["kind"] == "C"
    gscores = _gpu_decode_scores(layer, cfg, d, d["n_tokens"]) if csa else None
    n_cert = n_rows = 0
    for b in seqs:
        ref = OS.oracle_decode(cfg, d, b)
        p = int(d["n_tokens"][b])
        OS.assert_within_ulp(O.decode(_stored(ring[b, p % cfg.n_win], kv), kv), ref["window_row"], kv,
                             slack=ref["window_row_bound"], what="ring row")
        if ref["new_entry"] is not None:
            s = (p + 1) // m - 1
            OS.assert_within_ulp(O.decode(_stored(cache[b, s], kv), kv), ref["new_entry"], kv,
                                 slack=ref["new_entry_bound"], what="new entry")
        if csa:
            # every row's selection: select stage bit-exact on the GPU's scores,
            # scores within bound, certified rows equal to the oracle's top-k,
            # the others with every clear winner and no clear loser
            n_cert += _check_decode_selection(cfg, d, b, idx[b], gscores[b], ref["scores"], p,
                                              what=f"b{b}")
            n_rows += 1
            ref = OS.oracle_decode(cfg, d, b, idx_given=idx[b])
        err = np.abs(out[b] - ref["out"])
        assert err.max() <= OUT_TOL[io], f"b{b}: out err {err.max():.3g}"
        lerr = np.abs(lse[b] - ref["lse"])
        assert lerr.max() <= LSE_TOL[io], f"b{b}: lse err {lerr.max():.3g}"
    if csa:
        assert n_rows == len(list(seqs)) and n_rows > 0
        say(f"{cfg.name}: selection checked on {n_rows} CSA rows ({n_cert} certified, "
            f"{n_rows - n_cert} by select stage + clear winners/losers)")
    return layer


@pytest.mark.parametrize("ctx", [1 << 14, 1 << 18])
def test_csa_decode_reduced(ctx):
    cfg = CSA_DECODE_1M.with_(B=4, ctx=ctx)
    say(f"CSA decode B=4 ctx={ctx}")
    d = gen.decode_inputs(cfg)
    _decode_parity(cfg, d, range(cfg.B))


def test_csa_decode_rows_longer_than_one_bitmap_pass():
    """One sequence of about 2.1M tokens: more than 2^19 visible entries, so the
    selection writes its ascending output in two bitmap passes, and the row's
    256 indexer workgroups give each finish wave 16 regions to read."""
    cfg = CSA_DECODE_1M.with_(B=1, ctx=(1 << 21) + (1 << 15))
    say(f"CSA decode B=1 ctx={cfg.ctx}")
    d = gen.decode_inputs(cfg)
    assert d["n_cap"] > (1 << 19)
    _decode_parity(cfg, d, range(cfg.B))


def test_csa_decode_random_batches_fused_selection():
    """Seeded random batch sizes and context lengths in the fused selection's
    range (more than 36864 entries per row), fp8 keys: every row's selection
    bit-exact on the select stage (and against the oracle's when certified),
    with every clear winner and no clear loser, and the outputs within tolerance."""
    rng = np.random.default_rng(77)
    for case in range(4):
        B = int(rng.choice([1, 2, 3]))
        ctx = int(rng.integers(150000, 420000))
        cfg = CSA_DECODE_1M.with_(B=B, ctx=ctx, seed=100 + case)
        say(f"random fused decode case {case}: B={B} ctx={ctx}")
        d = gen.decode_inputs(cfg)
        assert d["n_cap"] > 36864
        _decode_parity(cfg, d, range(B))


@pytest.mark.parametrize("k", [1, 7, 2048, 4096])
def test_csa_decode_fused_selection_k_range(k):
    """The fused selection at the ends of the interface's k range (1 .. 4096):
    every row's selection bit-exact on the select stage (the oracle's top-k of
    the GPU's own scores), with every clear winner and no clear loser, and the
    outputs within tolerance (k + 128 attended rows)."""
    cfg = CSA_DECODE_1M.with_(B=2, ctx=1 << 18, k=k, seed=40 + k % 13)
    say(f"fused decode selection with k={k}")
    d = gen.decode_inputs(cfg)
    assert d["n_cap"] > 36864
    _decode_parity(cfg, d, range(cfg.B))


@pytest.mark.parametrize("kind", ["csa", "hca", "hybrid_csa"])
def test_decode_rope(kind):
    """Decode steps with partial RoPE: the ring row and a completed entry turned
    at the token's position, the query turned, the output turned back."""
    if kind == "csa":
        cfg = CSA_DECODE_1M.with_(B=4, ctx=1 << 14, rope_base=10000.0)
        d = gen.decode_inputs(cfg)
    elif kind == "hca":
        cfg = HCA_DECODE.with_(B=4, ctx=1 << 14, rope_base=10000.0)
        d = gen.decode_inputs(cfg)
    else:                              # fp8 KV with bf16 RoPE dims, MXFP4 indexer
        cfg = HYBRID_DECODE_1M.with_(ctx=1 << 16, rope_base=10000.0)
        d = gen.hybrid_inputs(cfg)[2]
        assert d["kind"] == "C"
    say(f"decode with RoPE: {cfg.name} B={cfg.B} ctx={cfg.ctx}")
    _decode_parity(cfg, d, range(cfg.B))


def test_csa_decode_1m_full_size_sampled():
    cfg = CSA_DECODE_1M
    say("CSA decode 1M B=16 (sampled sequences)")
    d = gen.decode_inputs(cfg)
    _decode_parity(cfg, d, [0, 7, 15])


@pytest.mark.parametrize("case", ["constant_keys", "three_keys", "rows_shorter_than_k"])
def test_csa_decode_selection_degenerate(case):
    """Rows longer than the LDS top-k takes (the fused indexer selection): every
    key equal (all scores tie: the first k entries), three distinct keys (ties
    across the threshold: lowest indices first) and rows with fewer visible
    entries than k (all of them, then -1)."""
    if case == "rows_shorter_than_k":
        cfg = CSA_DECODE_1M.with_(B=2, ctx=2048)
        d = gen.decode_inputs(cfg, extra_entries=40000)
    else:
        cfg = CSA_DECODE_1M.with_(B=2, ctx=1 << 18)
        d = gen.decode_inputs(cfg)
        kI = d["kI"]
        pick = np.zeros(kI.shape[1], np.int64) if case == "constant_keys" else np.arange(kI.shape[1]) % 3
        d["kI"] = np.ascontiguousarray(kI[:, pick])
    say(f"degenerate selection: {case}, N_cap {d['n_cap']}")
    assert d["n_cap"] > 36864
    layer = _decode_parity(cfg, d, range(cfg.B))
    idx = host(layer.idx)
    for b in range(cfg.B):
        vis = int((d["n_tokens"][b] + 1) // d["m"])
        if case == "constant_keys":
            assert np.array_equal(idx[b], np.arange(cfg.k)), f"b{b}"
        elif case == "rows_shorter_than_k":
            assert vis < cfg.k
            want = np.concatenate([np.arange(vis), np.full(cfg.k - vis, -1)])
            assert np.array_equal(idx[b], want), f"b{b}"
        else:
            ref = OS.oracle_decode(cfg, d, b)
            vals = np.unique(ref["scores"][:vis])
            assert len(vals) == 3
            kIb = O.decode(d["kI"][b, :3], cfg.idx_dtype)
            qIb = O.decode(d["qI"][b], cfg.idx_dtype)
            bnd = O.score_error_bound(qIb[None], kIb, d["w"][b][None].astype(np.float64))[0].max()
            if np.diff(vals).min() > 2 * bnd:   # the three values rank the same in fp32
                assert np.array_equal(idx[b], ref["idx"]), f"b{b}"


def test_hca_decode_full_size():
    cfg = HCA_DECODE
    say("HCA decode B=32 131072")
    d = gen.decode_inputs(cfg)
    _decode_parity(cfg, d, range(cfg.B))


def test_hybrid_decode_reduced_all_layers():
    cfg = HYBRID_DECODE_1M.with_(ctx=1 << 16)
    say("hybrid decode 8 layers ctx 65536")
    for i, d in enumerate(gen.hybrid_inputs(cfg)):
        say(f"  layer {i} {d['kind']}")
        lc = cfg.with_(m=d["m"]) if d["kind"] == "H" else cfg
        _decode_parity(lc, d, range(cfg.B))


@pytest.mark.parametrize("rope", [0.0, 10000.0])
def test_decode_multi_step_matches_oracle_stepping(rope):
    """Nine steps of a CSA and an HCA layer (blocks complete along the way, so
    entries made by the steps, turned at their last token with RoPE, are
    attended by later steps)."""
    for cfg in (CSA_DECODE_1M.with_(B=2, ctx=4096, rope_base=rope),
                HCA_DECODE.with_(B=2, ctx=1024, m=8, rope_base=rope)):
        say(f"multi-step {cfg.name}")
        d = gen.decode_inputs(cfg, extra_entries=4)
        layer = pipeline.DecodeLayer(cfg, d, DEV)
        states = [OS.oracle_decode_state(cfg, d, b) for b in range(cfg.B)]
        rng = np.random.default_rng(3)
        for step in range(9):
            if step:
                for name in ("tokC", "tokZ", "q"):
                    new = enc.encode(rng.standard_normal(d[name].shape), cfg.io_dtype)
                    d[name] = new
                    getattr(layer, name).copy_(T(new))
            layer.step()
            out = out_f64(layer.out)
            idx = host(layer.idx)
            pos = [states[b].L for b in range(cfg.B)]
            gsc = _gpu_decode_scores(layer, cfg, d, pos) if d["kind"] == "C" else None
            for b in range(cfg.B):
                kw = {}
                if d["kind"] == "C":
                    L = states[b].L + 1
                    kw = dict(k=cfg.k, qI=O.decode(d["qI"][b], cfg.idx_dtype),
                              kI=O.decode(d["kI"][b, :L // d["m"]], cfg.idx_dtype), w=d["w"][b],
                              idx_given=idx[b])
                r = O.decode_step(states[b], tokC=O.decode(d["tokC"][b], cfg.io_dtype),
                                  tokZ=O.decode(d["tokZ"][b], cfg.io_dtype), P=d["P"],
                                  q=O.decode(d["q"][b], cfg.io_dtype), tau=cfg.tau, eps=cfg.eps,
                                  kv_fmt=cfg.kv_dtype, out_fmt=cfg.io_dtype, rope_base=cfg.rope_base,
                                  **kw)
                if d["kind"] == "C":
                    _check_decode_selection(cfg, d, b, idx[b], gsc[b], r["scores"], pos[b],
                                            kI_rows=kw["kI"], what=f"step {step} b{b}")
                err = np.abs(out[b] - r["out"]).max()
                assert err <= OUT_TOL[cfg.io_dtype], f"step {step} b{b}: {err:.3g}"


def _hybrid_csa_layer(ctx, B=None):
    """The first CSA layer of the hybrid stack (layer 2: MXFP4 indexer keys, KV in
    fp8 with bf16 RoPE dims), drawn as the stack draws it."""
    cfg = HYBRID_DECODE_1M.with_(ctx=ctx) if B is None else HYBRID_DECODE_1M.with_(ctx=ctx, B=B)
    d = gen.decode_layer(cfg, "C", cfg.m, gen.hybrid_lengths(cfg), layer=2)
    return cfg, d


@pytest.mark.parametrize("ctx", [1 << 18, 1 << 20])
def test_hybrid_csa_decode_mxfp4_fused_selection(ctx):
    """A CSA layer of the hybrid stack on rows longer than the LDS top-k takes
    (65536 and 262144 entries), so the MXFP4 instance of the fused indexer +
    selection runs; at 2^20 tokens this is the stack's own CSA layer (batch 4)."""
    cfg, d = _hybrid_csa_layer(ctx)
    say(f"hybrid CSA layer (MXFP4 keys, fp8+bf16 KV) B={cfg.B} ctx={ctx} N_cap={d['n_cap']}")
    assert d["n_cap"] > 36864
    _decode_parity(cfg, d, range(cfg.B))


def test_hybrid_hca_layer_full_size():
    """An HCA layer of the hybrid stack at its own size (batch 4, 2^20 tokens:
    8192 compressed entries in fp8 with bf16 RoPE dims, dense attention over all
    of them plus the window; about 44 attention splits per row, merged 16 at a
    time), drawn as the stack draws its layer 0."""
    cfg = HYBRID_DECODE_1M
    d = gen.decode_layer(cfg, "H", cfg.m_hca, gen.hybrid_lengths(cfg), layer=0)
    lc = cfg.with_(m=d["m"])
    say(f"hybrid HCA layer (fp8+bf16 KV) B={cfg.B} ctx={cfg.ctx} N_cap={d['n_cap']}")
    assert d["n_cap"] > 8192
    _decode_parity(lc, d, range(cfg.B))


def _seq_slice(d, B, sel):
    return {k: (np.ascontiguousarray(v[sel]) if isinstance(v, np.ndarray) and v.ndim >= 1 and
                v.shape[0] == B else v) for k, v in d.items()}


def _decode_bits(cfg, d):
    layer = pipeline.DecodeLayer(cfg, d, DEV)
    layer.step()
    torch.cuda.synchronize()
    return {"out": host(layer.out.view(torch.int16)), "idx": host(layer.idx), "lse": host(layer.lse),
            "cache": layer.logical_cache(), "ring": host(layer.ring).view(np.uint8)}


@pytest.mark.parametrize("fmt,ctx", [("fp8", 1 << 16), ("fp8", 1 << 18), ("mxfp4", 1 << 18)])
def test_decode_deterministic_and_batch_invariant(fmt, ctx):
    """Two runs give the same bits; sequence 1 run alone (B = 1) gives the bits it
    gets inside a batch of 3; and other inputs for sequences 0 and 2 leave
    sequence 1's bits unchanged.  At 2^18 tokens (65536 entries) the rows take
    the fused indexer + selection, whose workgroup split of a row, dynamic group
    counter and emission order all change with the batch; at 2^16 the
    score-array path.  (B = 1 and B = 3 share the attention's split plan: it
    depends on the batch size only through the number of query rows.)"""
    if fmt == "fp8":
        cfg = CSA_DECODE_1M.with_(B=3, ctx=ctx)
        d = gen.decode_inputs(cfg)
    else:
        cfg, d = _hybrid_csa_layer(ctx, B=3)
    say(f"determinism / batch invariance {fmt} ctx={ctx} N_cap={d['n_cap']}")
    runs = [_decode_bits(cfg, d) for _ in range(2)]
    for name in runs[0]:
        assert np.array_equal(runs[0][name], runs[1][name]), f"{name} differs between two runs"
    one = _decode_bits(cfg.with_(B=1), _seq_slice(d, cfg.B, slice(1, 2)))
    for name in ("out", "idx", "lse"):
        assert np.array_equal(one[name][0], runs[0][name][1]), f"{name}: B=1 differs from B=3"
    assert np.array_equal(one["cache"][0], runs[0]["cache"][1])
    # sequences 0 and 2 swap every per-sequence input: sequence 1 is unchanged
    sw = dict(d)
    for k, v in d.items():
        if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == cfg.B and k not in (
                "lengths", "n_tokens"):
            v2 = v.copy()
            v2[0], v2[2] = v[2], v[0]
            sw[k] = v2
    other = _decode_bits(cfg, sw)
    for name in ("out", "idx", "lse"):
        assert np.array_equal(other[name][1], runs[0][name][1]), f"{name}: depends on other sequences"


@pytest.mark.parametrize("kind,split_rows", [("csa", 128), ("hca", 192), ("hca", 1024)])
def test_decode_fixed_split_rows_is_batch_invariant(kind, split_rows):
    """With a fixed attention split length (lca_decode_layer.split_rows) a
    sequence's bits do not depend on the batch size: sequence 5 alone equals
    sequence 5 in a batch of 16 (whose automatic plan would use other splits),
    and the batch agrees with the oracle.  CSA at 2^18 tokens takes the fused
    selection; HCA with 1024 rows per split runs one split per sequence, so no
    merge follows the attention (which then advances the token count itself)."""
    if kind == "csa":
        cfg = CSA_DECODE_1M.with_(B=16, ctx=1 << 18)
    else:
        cfg = HCA_DECODE.with_(B=16, ctx=1 << 16)
    d = gen.decode_inputs(cfg)
    say(f"fixed split_rows={split_rows}: {kind} B=16 vs B=1, N_cap {d['n_cap']}")

    def bits(c, dd):
        layer = pipeline.DecodeLayer(c, dd, DEV, split_rows=split_rows)
        layer.step()
        torch.cuda.synchronize()
        r = {"out": host(layer.out.view(torch.int16)), "lse": host(layer.lse)}
        if kind == "csa":
            r["idx"] = host(layer.idx)
        return r

    full = bits(cfg, d)
    one = bits(cfg.with_(B=1), _seq_slice(d, cfg.B, slice(5, 6)))
    for name in full:
        assert np.array_equal(one[name][0], full[name][5]), f"{name}: B=1 differs from B=16"
    _decode_parity(cfg, d, [0, 5, 15],
                   layer=pipeline.DecodeLayer(cfg, d, DEV, split_rows=split_rows))


@pytest.mark.parametrize("case", ["bf16", "fp8_rope_paged", "bf16_one_split", "random0", "random1",
                                  "random2"])
def test_hca_decode_step_equals_append_then_attention(case):
    """An HCA decode step on the few-row decode kernel appends the token inside
    the attention launch.  It must give the bits of lca_state_append followed by
    lca_sparse_mqa (same split plan) on a copy of the same state, step after step
    over 140 steps (every sequence completes a block; with RoPE, a paged cache
    and fp8 rows; with one split per sequence, where no merge follows): outputs,
    lse, ring, tail rows, compressed cache and token counts."""
    if case.startswith("random"):
        # seeded shapes: the split plan, and so which splits hold the new rows, varies
        rng = np.random.default_rng(100 + int(case[-1]))
        cfg = HCA_DECODE.with_(B=int(rng.integers(1, 40)), ctx=int(rng.integers(1 << 12, 1 << 18)),
                               kv_dtype=["bf16", "fp8_bf16rope"][int(rng.integers(0, 2))],
                               rope_base=[0.0, 10000.0][int(rng.integers(0, 2))], seed=int(rng.integers(0, 99)))
        paged = {"seed": 7} if rng.integers(0, 2) else None
        split_rows = [0, 0, 64 * int(rng.integers(1, 9))][int(rng.integers(0, 3))]
    elif case == "bf16":
        cfg, paged, split_rows = HCA_DECODE.with_(B=8, ctx=1 << 15), None, 0
    elif case == "fp8_rope_paged":
        cfg = HCA_DECODE.with_(B=4, ctx=1 << 16, kv_dtype="fp8_bf16rope", rope_base=10000.0)
        paged, split_rows = {"seed": 2}, 0
    else:
        cfg, paged, split_rows = HCA_DECODE.with_(B=3, ctx=1 << 15), None, 4096
    d = gen.decode_inputs(cfg, extra_entries=4)
    say(f"HCA step == append + attention: {case}, B={cfg.B}, ctx={cfg.ctx}, kv={cfg.kv_dtype}, "
        f"rope={cfg.rope_base}, paged={paged is not None}, split_rows={split_rows}, N_cap {d['n_cap']}")
    fused = pipeline.DecodeLayer(cfg, d, DEV, paged=paged, split_rows=split_rows)
    ref = pipeline.DecodeLayer(cfg, d, DEV, paged=paged, split_rows=split_rows)
    B, m, c, H = cfg.B, d["m"], cfg.c, cfg.H
    q_pos = torch.empty(B, dtype=torch.int32, device=DEV)
    n_ent = torch.empty(B, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(1, ops.sparse_mqa_workspace_size(B, 1, H, c, cfg.kv_dtype, 0, d["n_cap"],
                                                          cfg.n_win, True, split_rows)),
                     dtype=torch.uint8, device=DEV)
    out_r = torch.empty_like(ref.out)
    lse_r = torch.empty_like(ref.lse)
    pages = ref.paged.struct(DEV) if paged else None
    bits = lambda v: host(v.view(torch.int16) if v.dtype == torch.bfloat16 else v)  # noqa: E731
    for st in range(140):
        fused.step()
        ops.lca_state_append("hca", m, B, c, cfg.n_win, ref.tokC, ref.tokZ, cfg.io_dtype, ref.tailC,
                             ref.tailZ, ref.ring, cfg.kv_dtype, ref.P, ref.cache, d["n_cap"], ref.n_tokens,
                             q_pos, n_ent, cfg.eps, cfg.rope_base, pages=pages)
        ops.lca_sparse_mqa(B, 1, H, c, ref.q, cfg.io_dtype, ref.cache, cfg.kv_dtype, d["n_cap"], None, 0,
                           q_pos, m, n_ent, ref.ring, cfg.n_win, 0, cfg.n_win, cfg.tau, cfg.eps, None,
                           cfg.rope_base, out_r, cfg.io_dtype, lse=lse_r, workspace=ws, pages=pages,
                           split_rows=split_rows)
        if st % 20 == 0 or st == 139:
            torch.cuda.synchronize()
            assert np.array_equal(bits(fused.out), bits(out_r)), f"step {st}: out"
            assert np.array_equal(bits(fused.lse), bits(lse_r)), f"step {st}: lse"
    torch.cuda.synchronize()
    for name in ("ring", "tailC", "tailZ", "cache", "n_tokens"):
        assert np.array_equal(bits(getattr(fused, name)), bits(getattr(ref, name))), f"state {name}"
    assert np.array_equal(host(fused.n_tokens), d["n_tokens"] + 140)
    assert ((d["n_tokens"] + 140) // m > (d["n_tokens"] + 1) // m).all(), "every sequence completes a block"


@pytest.mark.parametrize("case", ["fp8", "mxfp4_fp8kv_paged_rope", "random0", "random1"])
def test_csa_decode_step_equals_separate_calls(case):
    """A CSA decode step with the fused selection runs its state append beside
    the selection's finish pass (the indexer takes its positions from the token
    counts, the histogram is the layer's sel_hist).  It must give the bits of the
    separate calls on a copy of the same state: lca_state_append,
    lca_indexer_scores + lca_topk and
    lca_sparse_mqa, step after step over 40 steps (a block completes every 4):
    outputs, lse, selections, ring, tail rows, compressed cache, token counts."""
    if case.startswith("random"):
        # seeded shapes in the fused selection's range (more than 36864 entries)
        rng = np.random.default_rng(200 + int(case[-1]))
        cfg = CSA_DECODE_1M.with_(B=int(rng.integers(1, 13)), ctx=int(rng.integers(150_000, 1 << 20)),
                                  idx_dtype=["fp8", "mxfp4"][int(rng.integers(0, 2))],
                                  kv_dtype=["bf16", "fp8_bf16rope"][int(rng.integers(0, 2))],
                                  rope_base=[0.0, 10000.0][int(rng.integers(0, 2))],
                                  seed=int(rng.integers(0, 99)))
        paged = {"seed": 9} if rng.integers(0, 2) else None
    elif case == "fp8":
        cfg, paged = CSA_DECODE_1M.with_(B=4, ctx=1 << 18), None
    else:
        cfg = CSA_DECODE_1M.with_(B=2, ctx=1 << 18, idx_dtype="mxfp4", kv_dtype="fp8_bf16rope",
                                  rope_base=10000.0)
        paged = {"seed": 4}
    d = gen.decode_inputs(cfg, extra_entries=12)
    say(f"CSA step == separate calls: {case}, B={cfg.B}, ctx={cfg.ctx}, idx={cfg.idx_dtype}, "
        f"kv={cfg.kv_dtype}, rope={cfg.rope_base}, paged={paged is not None}, N_cap {d['n_cap']}")
    fused = pipeline.DecodeLayer(cfg, d, DEV, paged=paged)
    ref = pipeline.DecodeLayer(cfg, d, DEV, paged=paged)
    B, m, c, H, N_cap, k = cfg.B, d["m"], cfg.c, cfg.H, d["n_cap"], cfg.k
    q_pos = torch.empty(B, dtype=torch.int32, device=DEV)
    n_ent = torch.empty(B, dtype=torch.int32, device=DEV)
    scores = torch.empty((B, N_cap), dtype=torch.float32, device=DEV)
    idx_r = torch.empty((B, k), dtype=torch.int32, device=DEV)
    ws_t = torch.empty(max(1, ops.topk_workspace_size(B, 1, N_cap, k)), dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(max(1, ops.sparse_mqa_workspace_size(B, 1, H, c, cfg.kv_dtype, k, N_cap, cfg.n_win,
                                                            False)), dtype=torch.uint8, device=DEV)
    out_r = torch.empty_like(ref.out)
    lse_r = torch.empty_like(ref.lse)
    pages = ref.paged.struct(DEV) if paged else None
    bits = lambda v: host(v.view(torch.int16) if v.dtype == torch.bfloat16 else v)  # noqa: E731
    for st in range(40):
        fused.step()
        ops.lca_state_append("csa", m, B, c, cfg.n_win, ref.tokC, ref.tokZ, cfg.io_dtype, ref.tailC,
                             ref.tailZ, ref.ring, cfg.kv_dtype, ref.P, ref.cache, N_cap, ref.n_tokens,
                             q_pos, n_ent, cfg.eps, cfg.rope_base, pages=pages)
        ops.lca_indexer_scores(B, 1, cfg.H_I, cfg.d_I, cfg.idx_dtype, ref.qI, ref.qI_scale, ref.kI,
                               ref.kI_scale, N_cap, ref.w, q_pos, m, n_ent, scores)
        ops.lca_topk(B, 1, N_cap, scores, q_pos, m, n_ent, k, idx_r, ws_t)
        ops.lca_sparse_mqa(B, 1, H, c, ref.q, cfg.io_dtype, ref.cache, cfg.kv_dtype, N_cap, idx_r, k,
                           q_pos, m, n_ent, ref.ring, cfg.n_win, 0, cfg.n_win, cfg.tau, cfg.eps, None,
                           cfg.rope_base, out_r, cfg.io_dtype, lse=lse_r, workspace=ws_a, pages=pages)
        if st % 8 == 0 or st == 39:
            torch.cuda.synchronize()
            assert np.array_equal(host(fused.idx), host(idx_r)), f"step {st}: selection"
            assert np.array_equal(bits(fused.out), bits(out_r)), f"step {st}: out"
            assert np.array_equal(bits(fused.lse), bits(lse_r)), f"step {st}: lse"
    torch.cuda.synchronize()
    for name in ("ring", "tailC", "tailZ", "cache", "n_tokens"):
        assert np.array_equal(bits(getattr(fused, name)), bits(getattr(ref, name))), f"state {name}"
    assert np.array_equal(host(fused.n_tokens), d["n_tokens"] + 40)


@pytest.mark.parametrize("idx_dtype", ["fp8", "mxfp4"])
def test_csa_decode_sel_hist_equals_workspace_histogram(idx_dtype):
    """The fused selection's histogram kept with the layer's state (sel_hist:
    no launch before the indexer; the finish pass leaves it zero-filled) gives
    the bits of the step that clears a workspace histogram first, step after
    step, and sel_hist is all zeros after every step.  One sequence starts with
    at most k visible entries (the indexer writes its selection directly)."""
    cfg = CSA_DECODE_1M.with_(B=3, ctx=1 << 18, idx_dtype=idx_dtype)
    d = gen.decode_inputs(cfg, extra_entries=12)
    d["n_tokens"] = d["n_tokens"].copy()
    d["n_tokens"][1] = 4 * cfg.k - 9  # vis <= k for the first steps, then k + 1, ...
    say(f"sel_hist == workspace histogram: idx={idx_dtype}, N_cap {d['n_cap']}, "
        f"n_tokens {d['n_tokens'].tolist()}")
    a = pipeline.DecodeLayer(cfg, d, DEV)
    b = pipeline.DecodeLayer(cfg, d, DEV, sel_hist=False)
    assert a.sel_hist is not None and b.sel_hist is None
    bits = lambda v: host(v.view(torch.int16) if v.dtype == torch.bfloat16 else v)  # noqa: E731
    for st in range(24):
        a.step()
        b.step()
        torch.cuda.synchronize()
        assert not host(a.sel_hist).any(), f"step {st}: sel_hist left non-zero"
        if st == 0:  # sequence 1 sees 1022 entries: all of them, then -1
            want = np.concatenate([np.arange(cfg.k - 2), [-1, -1]])
            assert np.array_equal(host(a.idx)[1], want), "step 0: short row's selection"
        if st % 4 == 0 or st == 23:
            assert np.array_equal(host(a.idx), host(b.idx)), f"step {st}: selection"
            assert np.array_equal(bits(a.out), bits(b.out)), f"step {st}: out"
            assert np.array_equal(bits(a.lse), bits(b.lse)), f"step {st}: lse"
    for name in ("ring", "tailC", "tailZ", "cache", "n_tokens"):
        assert np.array_equal(bits(getattr(a, name)), bits(getattr(b, name))), f"state {name}"
    assert (host(a.idx)[1] >= 0).sum() == cfg.k  # 1027 visible by the last step


def test_sink_logit():
    cfg = HCA_DECODE.with_(B=2, ctx=4096, m=128)
    say("sink")
    d = gen.decode_inputs(cfg)
    sink = np.linspace(-2, 3, cfg.H).astype(np.float32)
    layer = pipeline.DecodeLayer(cfg, d, DEV, sink=sink)
    layer.step()
    out = out_f64(layer.out)
    for b in range(cfg.B):
        ref = OS.oracle_decode(cfg, d, b, sink=sink.astype(np.float64))
        assert np.abs(out[b] - ref["out"]).max() <= OUT_TOL["bf16"]


# ---------------------------------------------------------------------------
# paged compressed-KV cache (128-token pages, random block tables over a shared
# pool): every result equals the contiguous layout's bit for bit, and the
# oracle's


def _paged_pool(cache_e, kv, m, seed=5, page_tokens=128, bad_page=None):
    B, N_cap = cache_e.shape[0], cache_e.shape[1]
    pg = pipeline.Paged(B, N_cap, m, page_tokens=page_tokens, seed=seed)
    pool = pipeline.to_pool(_as_bytes(cache_e, kv).reshape(B, N_cap, -1), pg.epp, pg.table, pg.n_pages)
    if bad_page is not None:            # (b, logical page) -> a page id outside the pool
        pg.table[bad_page] = pg.n_pages + 7
    return pg, pool


@pytest.mark.parametrize("case", ["bf16_sparse", "fp8_sink", "bf16_dense", "rows300_f32q",
                                  "bf16_sparse_c128_rope", "bf16_sparse_badpage"])
def test_sparse_mqa_paged_equals_contiguous(case):
    """The gather through a block table (decode kernel with its page prefetch,
    the float32-query and generic kernels): bit-identical to the contiguous
    cache; an entry whose page id lies outside the pool counts as absent."""
    rng = np.random.default_rng(7)
    bad = "_badpage" in case
    t = _mqa_case(case.replace("_badpage", ""), rng)
    B, H, c, kv = t["B"], t["H"], t["c"], t["kv"]
    say(f"paged MQA {case}: B={B} k={t['k']} N_cap={t['N_cap']} m={t['m']}")
    bad_page = (1, 3) if bad else None
    pg, pool = _paged_pool(t["cache"], kv, t["m"], bad_page=bad_page)
    idx = t["idx"]
    if bad:                                   # the contiguous run without that page's entries
        idx = idx.copy()
        lo, hi = 3 * pg.epp, 4 * pg.epp
        assert ((idx[1] >= lo) & (idx[1] < hi)).any()
        idx[1][(idx[1] >= lo) & (idx[1] < hi)] = -1
    outs = []
    for paged in (False, True):
        out = torch.zeros(B * H * c, dtype=torch.bfloat16, device=DEV)
        lse = torch.zeros(B * H, dtype=torch.float32, device=DEV)
        cache = T(pool) if paged else T(_as_bytes(t["cache"], kv))
        pages = pg.struct(DEV) if paged else None
        use_idx = t["idx"] if paged else idx
        ops.lca_sparse_mqa(B, 1, H, c, T(t["q"]), t["q_fmt"], cache, kv, t["N_cap"],
                           None if use_idx is None else T(use_idx), t["k"], T(t["q_pos"]), t["m"],
                           T(t["n_entries"]), T(_as_bytes(t["win"], kv)), t["n_win"], 0, t["n_win"],
                           t["tau"], t["eps"], None if t["sink"] is None else T(t["sink"]), t["rope"],
                           out, "bf16", lse=lse, pages=pages)
        outs.append((host(out.view(torch.int16)), host(lse)))
    assert np.array_equal(outs[0][0], outs[1][0]), "outputs differ"
    assert np.array_equal(outs[0][1], outs[1][1]), "lse differs"


def _decode_cfg(kind):
    if kind == "csa":
        cfg = CSA_DECODE_1M.with_(B=4, ctx=1 << 14)
        return cfg, gen.decode_inputs(cfg)
    if kind == "hca":
        cfg = HCA_DECODE.with_(B=4, ctx=1 << 14)
        return cfg, gen.decode_inputs(cfg)
    cfg = HYBRID_DECODE_1M.with_(ctx=1 << 16)       # a CSA layer: fp8+bf16-rope KV, MXFP4 keys
    d = gen.hybrid_inputs(cfg)[2]
    assert d["kind"] == "C"
    return cfg, d


@pytest.mark.parametrize("kind", ["csa", "hca", "hybrid_csa"])
def test_decode_paged_equals_contiguous(kind):
    cfg, d = _decode_cfg(kind)
    say(f"paged decode {kind}: B={cfg.B} ctx={cfg.ctx}")
    res = []
    for paged in (None, {"seed": 11}):
        layer = pipeline.DecodeLayer(cfg, d, DEV, paged=paged)
        layer.step()
        torch.cuda.synchronize()
        res.append({"out": host(layer.out.view(torch.int16)), "lse": host(layer.lse),
                    "cache": layer.logical_cache()})
        if d["kind"] == "C":               # an HCA layer writes no selection
            res[-1]["idx"] = host(layer.idx)
    for name in res[0]:
        assert np.array_equal(res[0][name], res[1][name]), f"{name} differs"
    # and against the oracle (a fresh paged layer; the helper steps it once)
    _decode_parity(cfg, d, range(cfg.B), layer=pipeline.DecodeLayer(cfg, d, DEV, paged={"seed": 11}))


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_decode_steps_paged_multi_step(kind):
    """Nine steps in one lca_decode_steps call on a paged cache against nine
    lca_decode_step calls on the contiguous cache: every step's output and
    selection, and the cache with the entries the steps made, bit for bit; the
    last step against the oracle stepped from the same state."""
    if kind == "csa":
        cfg = CSA_DECODE_1M.with_(B=2, ctx=4096)
    else:
        cfg = HCA_DECODE.with_(B=2, ctx=1024, m=8)
    d = gen.decode_inputs(cfg, extra_entries=4)
    say(f"paged multi-step {kind}")
    n = 9
    rng = np.random.default_rng(21)
    toks = [{name: enc.encode(rng.standard_normal(d[name].shape), cfg.io_dtype)
             for name in ("tokC", "tokZ", "q")} for _ in range(n)]
    csa = kind == "csa"
    # contiguous: one call per step
    ref = pipeline.DecodeLayer(cfg, d, DEV)
    ref_out, ref_idx = [], []
    for st in toks:
        for name in ("tokC", "tokZ", "q"):
            getattr(ref, name).copy_(T(st[name]))
        ref.step()
        ref_out.append(host(ref.out.view(torch.int16)))
        ref_idx.append(host(ref.idx))
    # paged: all steps in one call
    lay = pipeline.DecodeLayer(cfg, d, DEV, paged={"seed": 4})
    steps = []
    for st in toks:
        e = {name: T(st[name]) for name in ("tokC", "tokZ", "q")}
        e["out"] = torch.empty_like(lay.out)
        e["lse"] = torch.empty_like(lay.lse)
        if csa:
            e.update(qI=lay.qI, qI_scale=lay.qI_scale, w=lay.w, idx_out=torch.empty_like(lay.idx))
        steps.append(e)
    ops.lca_decode_steps(lay.state, steps, cfg.io_dtype, workspace=lay.workspace)
    torch.cuda.synchronize()
    for i, e in enumerate(steps):
        assert np.array_equal(host(e["out"].view(torch.int16)), ref_out[i]), f"step {i} out"
        if csa:
            assert np.array_equal(host(e["idx_out"]), ref_idx[i]), f"step {i} idx"
    assert np.array_equal(lay.logical_cache(), ref.logical_cache())
    assert np.array_equal(host(lay.n_tokens), host(ref.n_tokens))
    # the oracle, stepped through the same tokens, agrees on every step's output
    # and selection
    states = [OS.oracle_decode_state(cfg, d, b) for b in range(cfg.B)]
    for i, st in enumerate(toks):
        pos = [states[b].L for b in range(cfg.B)]
        gsc = _gpu_decode_scores(lay, cfg, d, pos) if csa else None
        for b in range(cfg.B):
            kw = {}
            if csa:
                L = states[b].L + 1
                kw = dict(k=cfg.k, qI=O.decode(d["qI"][b], cfg.idx_dtype),
                          kI=O.decode(d["kI"][b, :L // d["m"]], cfg.idx_dtype), w=d["w"][b],
                          idx_given=host(steps[i]["idx_out"])[b])
            r = O.decode_step(states[b], tokC=O.decode(st["tokC"][b], cfg.io_dtype),
                              tokZ=O.decode(st["tokZ"][b], cfg.io_dtype), P=d["P"],
                              q=O.decode(st["q"][b], cfg.io_dtype), tau=cfg.tau, eps=cfg.eps,
                              kv_fmt=cfg.kv_dtype, out_fmt=cfg.io_dtype, **kw)
            if csa:
                _check_decode_selection(cfg, d, b, kw["idx_given"], gsc[b], r["scores"], pos[b],
                                        kI_rows=kw["kI"], what=f"step {i} b{b}")
            got = out_f64(steps[i]["out"])[b]
            err = np.abs(got - r["out"]).max()
            assert err <= OUT_TOL[cfg.io_dtype], f"step {i} b{b}: {err:.3g}"


@pytest.mark.parametrize("which", ["tiny", "chunk"])
def test_prefill_paged_equals_contiguous(which):
    """Prefill with the compressor writing through the block table and the
    attention gathering through it: new entries and outputs bit for bit."""
    if which == "tiny":
        cfg = TINY_CSA_PREFILL
    else:
        cfg = CSA_PREFILL_CHUNK.with_(ctx=8192, n_new=1024)
    say(f"paged prefill {cfg.name} ctx={cfg.ctx} n={cfg.n_new}")
    d = gen.prefill_inputs(cfg)
    res = []
    for paged in (None, {"seed": 2}):
        layer = pipeline.PrefillLayer(cfg, d, DEV, paged=paged)
        layer.run()
        torch.cuda.synchronize()
        res.append((layer.logical_cache(), host(layer.out.view(torch.int16) if layer.out.dtype ==
                                                torch.bfloat16 else layer.out), host(layer.idx)))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# grouped output projection: the bf16 intermediate within one ulp plus the fp32
# accumulation bound of the oracle's exact value, the output within the bound of
# the oracle's product over the GPU's own intermediate (each stage on the same
# inputs as the oracle)


def _out_proj_inputs(nt, n_h, c, g, d_g, d, seed):
    rng = np.random.default_rng(seed)
    kin = n_h // g * c
    o = enc.to_bf16_bits(rng.standard_normal((nt, n_h, c)) * 0.5)
    W_g = enc.to_bf16_bits(rng.standard_normal((g, d_g, kin)) / np.sqrt(kin))
    W_o = enc.to_bf16_bits(rng.standard_normal((d, g * d_g)) / np.sqrt(g * d_g))
    return o, W_g, W_o


def _check_out_proj(nt, n_h, c, g, d_g, d, out_fmt, rows=None, seed=3):
    o, W_g, W_o = _out_proj_inputs(nt, n_h, c, g, d_g, d, seed)
    z = torch.empty((nt, g * d_g), dtype=torch.int16, device=DEV)
    out = torch.empty((nt, d), dtype=torch.float32 if out_fmt == "f32" else torch.bfloat16, device=DEV)
    ops.lca_grouped_out_proj(nt, n_h, c, g, d_g, d, T(o), T(W_g), T(W_o), z, out, out_fmt)
    zg = O.decode_bf16(host(z).view(np.uint16))
    og = out_f64(out)
    rows = np.arange(nt) if rows is None else np.asarray(rows)
    od, Wgd, Wod = O.decode_bf16(o[rows]), O.decode_bf16(W_g), O.decode_bf16(W_o)
    _, z_exact = O.grouped_output_projection(od, Wgd, Wod)
    kin = n_h // g * c
    x = np.abs(od).reshape(len(rows), g, kin)
    zb = np.concatenate([O.matmul_error_bound(x[:, j], np.abs(Wgd[j]), kin) for j in range(g)], axis=1)
    OS.assert_within_ulp(zg[rows], O.round_to(z_exact, "bf16"), "bf16", slack=zb, what="z")
    want = zg[rows] @ Wod.T
    ob = O.matmul_error_bound(np.abs(zg[rows]), np.abs(Wod), g * d_g)
    if out_fmt == "f32":
        err = np.abs(og[rows] - want)
        assert np.all(err <= ob + 1e-30), f"out err {err.max():.3g} > bound {ob.max():.3g}"
    else:
        OS.assert_within_ulp(og[rows], O.round_to(want, "bf16"), "bf16", slack=ob, what="out")
    return host(z), host(out.view(torch.int16) if out.dtype == torch.bfloat16 else out)


@pytest.mark.parametrize("nt,n_h,c,g,d_g,d,out_fmt", [
    (16, 64, 512, 8, 1024, 7168, "bf16"),     # the decode batch at the V4-Pro shape (K split)
    (5, 8, 128, 2, 128, 256, "f32"),          # small, K split, ragged rows
    (40, 16, 256, 4, 256, 384, "f32"),        # 32-row tiles
    (300, 16, 256, 8, 256, 1024, "bf16"),     # 128-row tiles with a ragged last tile
    (1, 64, 512, 1, 128, 128, "f32"),         # one group, one token
    # few-token kernel: K chunks of four steps taken from a per-workgroup start
    (7, 5, 128, 1, 128, 256, "f32"),          # 10 and 2 K steps: last chunk partial
    (3, 24, 128, 8, 1024, 256, "bf16"),       # 6 K steps (256 workgroups), then 128
    (32, 16, 256, 4, 256, 384, "f32"),        # the most tokens the few-token kernel takes
])
def test_grouped_out_proj(nt, n_h, c, g, d_g, d, out_fmt):
    say(f"grouped out proj T={nt} n_h={n_h} c={c} g={g} d_g={d_g} d={d} -> {out_fmt}")
    a = _check_out_proj(nt, n_h, c, g, d_g, d, out_fmt)
    b = _check_out_proj(nt, n_h, c, g, d_g, d, out_fmt)       # deterministic
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_grouped_out_proj_prefill_full_size_sampled():
    say("grouped out proj T=8192 at the V4-Pro shape, sampled rows")
    _check_out_proj(8192, 64, 512, 8, 1024, 7168, "bf16", rows=[0, 1, 127, 128, 4095, 8190, 8191])


# ---------------------------------------------------------------------------
# GPU decode path == GPU prefill path, and a saved decode state resumes to the
# same bits ("DeepSeek V4 Architecture Tricks", section "Heterogeneous KV Cache
# Layout": the state cache holds the window KV and the tail tokens)


def _prefill_and_decode(mode, rope, seed=31):
    """n tokens of a layer run two ways on the GPU: one prefill call chain from
    position 0 (lca_compress, lca_rmsnorm_rows, lca_indexer_scores, lca_topk,
    lca_sparse_mqa) and n lca_decode_step calls from an empty state.  Returns both
    results plus the decode state's tensors and the per-step inputs."""
    csa = mode == "csa"
    m = 4 if csa else 8
    B, n, c, H, HI, dI, n_win, k = 2, 640 if csa else 256, 512, 64, 64, 128, 128, 32
    N_cap = n // m
    tau, eps = c ** -0.5, 1e-6
    rng = np.random.default_rng(seed)
    enc16 = lambda a: enc.encode(a, "bf16")  # noqa: E731
    C, Z = enc16(rng.standard_normal((B, n, c))), enc16(rng.standard_normal((B, n, c)))
    P = (rng.standard_normal((2 * m if csa else m, c)) * 0.1).astype(np.float32)
    q = enc16(rng.standard_normal((B, n, H, c)))
    qI = enc.encode(rng.standard_normal((B, n, HI, dI)), "fp8")
    kI = enc.encode(rng.standard_normal((B, N_cap, dI)), "fp8")
    w = rng.random((B, n, HI)).astype(np.float32)
    rb = ops.row_bytes("bf16", c)
    # prefill
    cache_p = torch.zeros(B * N_cap * rb, dtype=torch.uint8, device=DEV)
    ops.lca_compress(mode, m, B, n, c, T(C), T(Z), "bf16", None, None, T(P), cache_p, "bf16", N_cap, 0,
                     eps, rope)
    win_p = torch.zeros(B * n * rb, dtype=torch.uint8, device=DEV)
    ops.lca_rmsnorm_rows(B, n, c, T(C), "bf16", win_p, "bf16", n, eps, 0, rope)
    q_pos = T(np.tile(np.arange(n, dtype=np.int32), (B, 1)))
    n_ent = T(np.full(B, N_cap, np.int32))
    idx_p = None
    if csa:
        scores = torch.empty((B, n, N_cap), dtype=torch.float32, device=DEV)
        ops.lca_indexer_scores(B, n, HI, dI, "fp8", T(qI), None, T(kI), None, N_cap, T(w), q_pos, m,
                               n_ent, scores)
        idx_p = torch.empty((B, n, k), dtype=torch.int32, device=DEV)
        ops.lca_topk(B, n, N_cap, scores, q_pos, m, n_ent, k, idx_p)
    out_p = torch.empty((B, n, H, c), dtype=torch.bfloat16, device=DEV)
    lse_p = torch.empty((B, n, H), dtype=torch.float32, device=DEV)
    ops.lca_sparse_mqa(B, n, H, c, T(q), "bf16", cache_p, "bf16", N_cap, idx_p, k if csa else 0, q_pos, m,
                       n_ent, win_p, n, 0, n_win, tau, eps, None, rope, out_p, "bf16", lse=lse_p)
    # decode from an empty state, one token per step
    T_rows = 2 * m if csa else m
    st = {"tailC": torch.zeros(B * T_rows * c, dtype=torch.int16, device=DEV),
          "tailZ": torch.zeros(B * T_rows * c, dtype=torch.int16, device=DEV),
          "ring": torch.zeros(B * n_win * rb, dtype=torch.uint8, device=DEV),
          "cache": torch.zeros(B * N_cap * rb, dtype=torch.uint8, device=DEV),
          "n_tokens": torch.zeros(B, dtype=torch.int32, device=DEV)}
    Pd, kId = T(P), T(kI)
    lay = ops.DecodeLayerState(mode=mode, m=m, B=B, c=c, H=H, n_win=n_win, N_cap=N_cap, io_fmt="bf16",
                               kv_fmt="bf16", tailC=st["tailC"], tailZ=st["tailZ"], ring=st["ring"],
                               cache=st["cache"], n_tokens=st["n_tokens"], P=Pd, tau=tau, eps=eps, k=k,
                               H_I=HI, d_I=dI, idx_fmt="fp8", kI=kId, rope_base=rope)
    steps = {"tokC": T(np.ascontiguousarray(C.transpose(1, 0, 2))),
             "tokZ": T(np.ascontiguousarray(Z.transpose(1, 0, 2))),
             "q": T(np.ascontiguousarray(q.transpose(1, 0, 2, 3))),
             "qI": T(np.ascontiguousarray(qI.transpose(1, 0, 2, 3))),
             "w": T(np.ascontiguousarray(w.transpose(1, 0, 2)))}
    dec = {"out": torch.empty((n, B, H, c), dtype=torch.bfloat16, device=DEV),
           "lse": torch.empty((n, B, H), dtype=torch.float32, device=DEV),
           "idx": torch.empty((n, B, k), dtype=torch.int32, device=DEV)}
    ws = torch.empty(lay.workspace_size(), dtype=torch.uint8, device=DEV)

    def step(t):
        ops.lca_decode_step(lay, steps["tokC"][t], steps["tokZ"][t], steps["q"][t], dec["out"][t], "bf16",
                            qI=steps["qI"][t] if csa else None, w=steps["w"][t] if csa else None,
                            lse=dec["lse"][t], idx_out=dec["idx"][t] if csa else None, workspace=ws)

    return dict(B=B, n=n, m=m, c=c, k=k, n_win=n_win, N_cap=N_cap, rb=rb, csa=csa, cache_p=cache_p,
                C=C, Z=Z, P=P, q=q, qI=qI, kI=kI, w=w,
                win_p=win_p, idx_p=idx_p, out_p=out_p, lse_p=lse_p, st=st, dec=dec, step=step)


@pytest.mark.parametrize("mode,rope", [("csa", 0.0), ("csa", 10000.0), ("hca", 0.0)])
def test_gpu_decode_from_empty_equals_gpu_prefill(mode, rope):
    """n decode steps from an empty state against one prefill of the same n
    tokens, both on the GPU.  Bit for bit: every compressed entry (the decode
    append pools a completed block with the prefill compressor's slot split and
    combination order), the window rows left in the ring, and every step's
    selection (both indexer kernels score with the same MFMA tiles and reduction
    order, and both selections are exact).  The outputs agree within the bf16
    output tolerance, with each other and with the oracle on sampled positions,
    rather than bit for bit: the decode step splits a query's candidate rows
    over several workgroups merged by log-sum-exp, the prefill call runs each
    query row in one workgroup, so the probabilities are rounded against
    different running maxima and the float32 sums are ordered differently (each
    path is deterministic)."""
    r = _prefill_and_decode(mode, rope)
    say(f"GPU decode == GPU prefill: {mode} rope={rope} n={r['n']}")
    for t in range(r["n"]):
        r["step"](t)
    torch.cuda.synchronize()
    B, n, N_cap, rb, n_win = r["B"], r["n"], r["N_cap"], r["rb"], r["n_win"]
    cp = host(r["cache_p"]).reshape(B, N_cap, rb)
    cd = host(r["st"]["cache"]).reshape(B, N_cap, rb)
    assert np.array_equal(cd, cp), f"entries differ in {(cd != cp).any(-1).sum()} rows"
    wp = host(r["win_p"]).reshape(B, n, rb)
    ring = host(r["st"]["ring"]).reshape(B, n_win, rb)
    for pos in range(n - n_win, n):
        assert np.array_equal(ring[:, pos % n_win], wp[:, pos]), f"window row {pos}"
    assert np.array_equal(host(r["st"]["n_tokens"]), np.full(B, n))
    if r["csa"]:
        idx_d = host(r["dec"]["idx"]).transpose(1, 0, 2)
        assert np.array_equal(idx_d, host(r["idx_p"])), "selections differ"
    od = out_f64(r["dec"]["out"]).transpose(1, 0, 2, 3)
    op = out_f64(r["out_p"])
    err = np.abs(od - op).max()
    # the probabilities go to the PV product as bf16, rounded against each
    # workgroup's own running maximum, so the two paths differ by more than a
    # rounding of the same float32 value: each is held to the oracle's
    # tolerance, and so is their difference
    assert err <= OUT_TOL["bf16"], f"decode vs prefill out err {err:.3g}"
    qs = np.array([0, 1, 3, 4, 127, 128, r["n"] // 2 + 3, r["n"] - 1])
    ref = O.prefill_layer(mode=mode, m=r["m"], k=r["k"], n_win=n_win, tau=r["c"] ** -0.5, eps=1e-6,
                          kv_fmt="bf16", out_fmt="bf16", pos0=0, C=O.decode(r["C"][0], "bf16"),
                          Z=O.decode(r["Z"][0], "bf16"), P=r["P"], q=O.decode(r["q"][0], "bf16"),
                          cache_prefix=np.zeros((0, r["c"])), qI=O.decode(r["qI"][0], "fp8"),
                          kI=O.decode(r["kI"][0], "fp8"), w=r["w"][0], queries=qs,
                          idx_given=host(r["idx_p"])[0, qs] if r["csa"] else None, rope_base=rope)
    for name, o in (("decode", od[0, qs]), ("prefill", op[0, qs])):
        e = np.abs(o - ref["out"]).max()
        assert e <= OUT_TOL["bf16"], f"{name} vs oracle: {e:.3g}"
    lerr = np.abs(host(r["dec"]["lse"]).transpose(1, 0, 2) - host(r["lse_p"])).max()
    assert lerr <= LSE_TOL["bf16"], f"lse err {lerr:.3g}"
    say(f"  outputs: max |decode - prefill| = {err:.3g}, lse {lerr:.3g}")


@pytest.mark.parametrize("mode", ["csa", "hca"])
def test_decode_state_save_restore_resume(mode):
    """The decode state (tail rows, window ring, compressed cache, token counts)
    copied to host memory after some steps and written back later resumes to
    the same bits: the steps after the restore repeat the outputs, selections
    and final state of the steps first run after the save."""
    r = _prefill_and_decode(mode, 0.0, seed=47)
    n, n1 = r["n"], r["n"] // 2 + 3
    say(f"save / restore / resume: {mode}, save after {n1} of {n} steps")
    for t in range(n1):
        r["step"](t)
    torch.cuda.synchronize()
    saved = {name: v.cpu().clone() for name, v in r["st"].items()}
    for t in range(n1, n):
        r["step"](t)
    torch.cuda.synchronize()
    bits = lambda v: host(v.view(torch.int16) if v.dtype == torch.bfloat16 else v)  # noqa: E731
    first = {name: bits(v)[n1:].copy() for name, v in r["dec"].items()}
    end1 = {name: bits(v).copy() for name, v in r["st"].items()}
    for v in r["dec"].values():
        v.zero_()
    for name, v in r["st"].items():
        v.fill_(0x3 if v.dtype != torch.int32 else -5)   # scribble, then restore
        v.copy_(saved[name].to(DEV))
    for t in range(n1, n):
        r["step"](t)
    torch.cuda.synchronize()
    for name, v in r["dec"].items():
        if name == "idx" and not r["csa"]:
            continue
        assert np.array_equal(bits(v)[n1:], first[name]), f"{name} differs after the restore"
    for name, v in r["st"].items():
        assert np.array_equal(bits(v), end1[name]), f"state {name} differs after the restore"
