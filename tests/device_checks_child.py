"""Child process of tests/test_gpu_device_checks.py (not a test module itself).

Runs with LCA_LIB naming the device-check build of the library and prints one
JSON line: the violations counted by each case.  Valid inputs must count none;
the corrupted ones must count exactly the planted faults, which the kernels
treat as absent rows (so nothing here reads or writes out of bounds).
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from long_context_attention_14_amd import ops, pipeline  # noqa: E402
from synth import encode as enc  # noqa: E402
from synth import gen  # noqa: E402
from synth.configs import CSA_DECODE_1M, HCA_DECODE  # noqa: E402

DEV = "cuda"


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_case(cfg, paged=None):
    d = gen.decode_inputs(cfg)
    layer = pipeline.DecodeLayer(cfg, d, DEV, paged=paged)
    layer.step()
    torch.cuda.synchronize()
    return ops.lca_device_checks(reset=True)


def mqa_case(corrupt_idx, corrupt_pages):
    """Core attention over a k = 200 selection of 5000-entry rows (three queries),
    contiguous or paged, with planted faults: selected entries beyond the visible
    ones or below -1, or pages of selected entries moved outside the pool."""
    rng = np.random.default_rng(11)
    B, N_cap, k, m, c, H, n_win = 3, 5000, 200, 4, 512, 64, 128
    q_pos = np.array([5, 4000, 20000], np.int32)
    n_entries = np.array([2, 1000, 5000], np.int32)
    vis = np.minimum(np.minimum((q_pos + 1) // m, n_entries), N_cap)
    idx = np.full((B, k), -1, np.int32)
    for b in range(B):
        n = min(k, int(vis[b]))
        idx[b, :n] = np.sort(rng.choice(int(vis[b]), n, replace=False))
    planted = 0
    if corrupt_idx:
        idx[1, 10], idx[1, 50], idx[2, 199] = vis[1] + 3, -5, N_cap + 100
        planted = 3
    cache = enc.encode(rng.standard_normal((B, N_cap, c)), "bf16")
    win = enc.encode(rng.standard_normal((B, n_win, c)), "bf16")
    q = enc.encode(rng.standard_normal((B, H, c)), "bf16")
    rb = ops.row_bytes("bf16", c)
    cache_u8 = np.ascontiguousarray(cache).view(np.uint8).reshape(B, N_cap, rb)
    pages = None
    if corrupt_pages:
        pg = pipeline.Paged(B, N_cap, m, seed=5)
        pool = pipeline.to_pool(cache_u8, pg.epp, pg.table, pg.n_pages)
        table = pg.table.copy()
        # the logical pages of two selected entries of sequence 2 point outside the pool
        sel = idx[2][idx[2] >= 0]
        for j in sorted({int(sel[0]) // pg.epp, int(sel[150]) // pg.epp}):
            table[2, j] = pg.n_pages + 7
            planted += int(((sel // pg.epp) == j).sum())
        table_dev = T(table)
        pages = ops.kv_pages(table_dev, pg.page_tokens, pg.n_pages, B)
        cache_dev = T(pool)
    else:
        cache_dev = T(cache_u8)
    out = torch.zeros(B * H * c, dtype=torch.bfloat16, device=DEV)
    ops.lca_sparse_mqa(B, 1, H, c, T(q), "bf16", cache_dev, "bf16", N_cap, T(idx), k, T(q_pos), m,
                       T(n_entries), T(np.ascontiguousarray(win).view(np.uint8)), n_win, 0, n_win,
                       1.0 / np.sqrt(c), 1e-6, None, 0.0, out, "bf16", pages=pages)
    torch.cuda.synchronize()
    return ops.lca_device_checks(reset=True), planted


def main():
    res = {"initial": ops.lca_device_checks(reset=True)}
    say("csa decode 2^18 (fused selection)")
    res["csa_fused"] = decode_case(CSA_DECODE_1M.with_(B=2, ctx=1 << 18))
    say("csa decode 2^14 (score-array selection)")
    res["csa_lds"] = decode_case(CSA_DECODE_1M.with_(B=2, ctx=1 << 14))
    say("csa decode 2^18, paged cache")
    res["csa_paged"] = decode_case(CSA_DECODE_1M.with_(B=2, ctx=1 << 18), paged={"seed": 3})
    say("hca decode")
    res["hca"] = decode_case(HCA_DECODE.with_(B=2, ctx=1 << 15))
    say("sparse mqa, valid")
    res["mqa_valid"] = mqa_case(False, False)[0]
    say("sparse mqa, planted index faults")
    res["mqa_bad_idx"], res["mqa_bad_idx_planted"] = mqa_case(True, False)
    say("sparse mqa, planted page faults")
    res["mqa_bad_pages"], res["mqa_bad_pages_planted"] = mqa_case(False, True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
