"""Feeds the seeded synthetic workloads (synth.gen dicts of stored bytes) to the
float64 oracle: decodes the bytes, rebuilds each sequence's logical decode
state from the physical tail/ring layout, and runs the oracle's layer or step.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
baseline); the library never imports it.
"""
import numpy as np

from . import lca_oracle as O


class LazyRows:
    """Rows of a stored byte array, decoded to float64 on access."""

    def __init__(self, raw, fmt, scales=None):
        self.raw, self.fmt, self.scales = raw, fmt, scales

    def __len__(self):
        return len(self.raw)

    def __getitem__(self, i):
        sc = None if self.scales is None else self.scales[i]
        return O.decode(self.raw[i], self.fmt, sc)


def idx_fmt_scales(d, name):
    return d.get(name + "_scale")


# ---------------------------------------------------------------------------
# prefill


def oracle_prefill(cfg, d, b, queries, idx_given=None, sink=None):
    io, kv, m = cfg.io_dtype, cfg.kv_dtype, cfg.m
    n_prefix = d["n_prefix"]
    kI_sc = d.get("kI_scale")
    kI = O.decode(d["kI"][b], cfg.idx_dtype, None if kI_sc is None else kI_sc[b])
    qI = LazyRows(d["qI"][b], cfg.idx_dtype, None if d.get("qI_scale") is None else d["qI_scale"][b])
    return O.prefill_layer(
        mode="csa", m=m, k=cfg.k, n_win=cfg.n_win, tau=cfg.tau, eps=cfg.eps, kv_fmt=kv, out_fmt=io,
        pos0=d["pos0"], C=O.decode(d["C"][b], io), Z=O.decode(d["Z"][b], io),
        P=np.asarray(d["P"], np.float64), q=LazyRows(d["q"][b], io),
        cache_prefix=O.decode(d["cache"][b, :n_prefix], kv),
        prevC=O.decode(d["prevC"][b], io) if "prevC" in d else None,
        prevZ=O.decode(d["prevZ"][b], io) if "prevZ" in d else None,
        win_prefix=O.decode(d["win_prefix"][b], kv) if "win_prefix" in d else None,
        qI=qI, kI=kI, w=d["w"][b], queries=queries, idx_given=idx_given, sink=sink,
        rope_base=cfg.rope_base)


# ---------------------------------------------------------------------------
# decode


def oracle_decode_state(cfg, d, b):
    """The oracle's logical DecodeState for sequence b of a decode_layer dict."""
    mode = "csa" if d["kind"] == "C" else "hca"
    m, c, io, kv, n_win = d["m"], cfg.c, cfg.io_dtype, cfg.kv_dtype, cfg.n_win
    p = int(d["n_tokens"][b])                      # position of the token the step appends
    blk = p // m
    tC, tZ = d["tailC"][b], d["tailZ"][b]
    if mode == "csa":
        half = blk % 2
        rows = [half * m + i for i in range(p % m)]
        prev = None
        if blk >= 1:
            ph = (blk - 1) % 2
            pr = [ph * m + i for i in range(m)]
            prev = (O.decode(tC[pr], io), O.decode(tZ[pr], io))
    else:
        rows = list(range(p % m))
        prev = None
    cur = (O.decode(tC[rows], io).reshape(-1, c), O.decode(tZ[rows], io).reshape(-1, c))
    wpos = [j for j in range(p - (n_win - 1), p) if j >= 0]
    window = [O.decode(d["ring"][b, j % n_win], kv) for j in wpos]
    n_pre = p // m
    entries = LazyRows(d["cache"][b, :n_pre], kv)
    return O.DecodeState(mode=mode, m=m, n_win=n_win, c=c, L=p, cur=cur, prev=prev, window=window,
                         entries=entries)


def oracle_decode(cfg, d, b, idx_given=None, sink=None):
    st = oracle_decode_state(cfg, d, b)
    io = cfg.io_dtype
    kw = {}
    if d["kind"] == "C":
        sc = d.get("kI_scale")
        L = int(d["n_tokens"][b]) + 1
        vis = L // d["m"]
        kw = dict(k=cfg.k, qI=O.decode(d["qI"][b], cfg.idx_dtype,
                                       None if d.get("qI_scale") is None else d["qI_scale"][b]),
                  kI=O.decode(d["kI"][b, :vis], cfg.idx_dtype, None if sc is None else sc[b, :vis]),
                  w=d["w"][b])
    r = O.decode_step(st, tokC=O.decode(d["tokC"][b], io), tokZ=O.decode(d["tokZ"][b], io),
                      P=np.asarray(d["P"], np.float64), q=O.decode(d["q"][b], io), tau=cfg.tau,
                      eps=cfg.eps, kv_fmt=cfg.kv_dtype, out_fmt=io, idx_given=idx_given, sink=sink,
                      rope_base=cfg.rope_base, **kw)
    r["state"] = st
    return r
