"""Benchmark: CSA decode at 1M context on one MI355X.

Workload: CSA decode step, batch 16 sequences of 2^20 + T_b tokens (m = 4 ->
262144 compressed entries each), fp8 indexer keys (64 heads x 128), top-1024,
multi-query attention over the selected bf16 entries (64 heads x 512) plus a
128-token window, bf16 in / fp32 accumulate.  One step = one decode token per
sequence through every stage of the path: state append (window KV, tail
block, compression of a block the token completes), indexer scores, top-k,
sparse attention with the window branch and the log-sum-exp merge.  Steps run
back to back, so the state advances (blocks complete every 4 steps).

Other workloads (--workload): HCA decode at 128K (batch 32), the 8-layer hybrid
decode stack at 1M (batch 4, MXFP4 indexer, fp8+bf16 KV) and the CSA prefill
chunk (8192 tokens on a 131072 prefix); the default line is the 1M CSA decode.

Decode steps run with cold caches by default: they rotate over enough copies of
every layer's state that more than 1 GiB (four times the 256 MB Infinity Cache)
is touched between two uses of a copy; --warm runs every step on one copy.  The
line's config.caches says which.  Before the warmup every page of every copy is
read once (so that no copy is used for the first time inside the timed region)
and then 1 GiB of scratch memory is written, which empties the caches again.

Prints ONE JSON line.  The timed loop calls lca_decode_step.  For a CSA layer
the library launches the indexer (the dominant kernel) with two HIP events
(lca_decode_io.stage_events[1], [2]) as its dispatch's own start and end
stamps, on every 4th timed step, which gives that kernel's duration for the
roofline.  The events are created with hipEventDisableSystemFence: a default
event writes back and invalidates the caches when it is recorded, which cost
11 us of GPU time per stamped step; without the fence the stamps still leave
about 4 us idle around the dispatch, so the other steps carry none.  For HCA
alone the dominant kernel is the attention: every 4th step records two events
around its stage.
The per-stage breakdown ("stages_us") comes from an untimed diagnostic loop
that sets all five events (the recorded ones include that cost).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
WORKLOADS = ("csa_decode_1m", "hca_decode", "hybrid_decode_1m", "csa_prefill_chunk",
             "out_proj_decode", "out_proj_prefill", "hbm_ceiling")
BF16_PEAK_TFLOPS = 2500.0


class HipEvents:
    """hipEvent_t handles from the HIP runtime, recorded by the library itself on
    the stream its kernels run on."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")

    # hipEventDisableSystemFence: timing-only events; a default event's record
    # writes back and invalidates the caches, which costs several microseconds of
    # GPU time around every stamped dispatch.  The stamps are read after a device
    # synchronisation, so nothing needs the event itself to order memory.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def create(self):
        e = self.ct.c_void_p()
        assert self.lib.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE) == 0
        return e.value

    def elapsed_s(self, a, b):
        ms = self.ct.c_float()
        assert self.lib.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a), self.ct.c_void_p(b)) == 0
        return ms.value * 1e-3

    def destroy(self, e):
        self.lib.hipEventDestroy(self.ct.c_void_p(e))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="csa_decode_1m", choices=WORKLOADS,
                    help="the default is the headline workload; the others are reported in the "
                         "design notes")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--stamp-every", type=int, default=4,
                    help="stamp the dominant kernel (or stage) on every n-th timed step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-touch", action="store_true",
                    help="decode: skip the pass that makes every copy of the layer state resident "
                         "(one read per 4 KiB page, then a 1 GiB write that empties the caches) "
                         "before the warmup")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--detail", default=None, help="write per-stage timings (JSON) to this file")
    ap.add_argument("--rope-base", type=float, default=0.0,
                    help="partial RoPE base for every layer (0: off, as in the workloads above; "
                         "inputs are then taken as post-RoPE)")
    ap.add_argument("--paged", action="store_true",
                    help="compressed-KV cache in 128-token pages behind a random block table")
    ap.add_argument("--warm", action="store_true",
                    help="decode: run every step on one copy of the layer state (warm Infinity "
                         "Cache); by default the steps rotate over enough copies to touch more "
                         "than 1 GiB between two uses of a copy (cold)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before warmup, run one plain device-to-device copy of MIB MiB (a "
                         "kernel of known traffic for scaling rocprofv3 byte counters)")
    return ap.parse_args()


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline_decode(cfgs, ds, budget_s):
    """The float64 oracle (as is) on a bounded sample: whole decode steps (every
    layer) of the batch's sequences in order, repeated over the batch until about
    budget_s (at least one pass, at most 50)."""
    from oracle.workloads import oracle_decode
    B = cfgs[0].B
    done, t0 = 0, time.perf_counter()
    while done < 50 * B:
        for c, d in zip(cfgs, ds):
            oracle_decode(c, d, done % B)
        done += 1
        if done >= B and time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "query-tokens/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{done} sequence-steps ({done / B:.1f} passes over the {B} sequences), one full "
                      f"decode step each through {len(cfgs)} layer(s) ({el:.1f} s, float64 numpy)"}


def cpu_baseline_prefill(cfg, d, budget_s):
    """The float64 oracle on a bounded sample of query rows of the same chunk (the
    chunk's compression is computed once per call and included in the time)."""
    import numpy as np
    from oracle.workloads import oracle_prefill
    rows, t0, q0 = 0, time.perf_counter(), 0
    while rows < cfg.n_new:
        qs = np.arange(q0, min(q0 + 16, cfg.n_new))
        oracle_prefill(cfg, d, 0, qs)
        rows += len(qs)
        q0 = (q0 + 997) % max(1, cfg.n_new - 16)
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": rows / el, "unit": "query-tokens/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{rows} of {cfg.n_new} query rows in blocks of 16, each block with the "
                      f"chunk's compression ({el:.1f} s, float64 numpy)"}


def _calibrate_copy(mib, dev):
    import torch
    if mib:
        src = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()


def _touch_pages(objs, dev):
    """Make the inputs resident before the untimed warmup: read one byte of every
    4 KiB of every device tensor the layer objects hold (the decode workloads
    rotate over up to 27 copies of the layer state, most of which a short warmup
    never reaches, so their first use, with its page-table walks, fell inside the
    timed region), then write 1 GiB of scratch memory so that the caches are cold
    again when the steps start."""
    import torch
    seen = set()

    def visit(o, depth=0):
        if isinstance(o, torch.Tensor):
            if o.is_cuda and o.numel() and o.data_ptr() not in seen:
                seen.add(o.data_ptr())
                b = o.view(-1).view(torch.uint8) if o.is_contiguous() else None
                if b is not None:
                    b[::4096].sum()
        elif isinstance(o, (list, tuple)):
            for x in o:
                visit(x, depth)
        elif hasattr(o, "__dict__") and depth < 3:
            for x in vars(o).values():
                visit(x, depth + 1)
    visit(objs)
    scratch = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)  # > 4x the 256 MB Infinity Cache
    torch.cuda.synchronize()
    del scratch


def _indexer_traffic():
    """HBM bytes per launch of the fp8 indexer (the fused indexer + selection
    kernel) from the committed counter summary, if it was taken with the current
    kernel source."""
    import hashlib
    tfile = os.path.join(ROOT, "profiles", "indexer_fp8_decode_b16_1m_counters.txt")
    if not os.path.exists(tfile):
        return None
    kv = dict(l.split(":", 1) for l in open(tfile) if ":" in l and not l.startswith("#"))
    src = os.path.join(ROOT, "long_context_attention_14_amd", "csrc", "indexer.hip")
    cur = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if kv.get("indexer_source_sha256_16", "").strip() == cur and "hbm_bytes_per_launch" in kv:
        return float(kv["hbm_bytes_per_launch"])
    return None


DECODE_STAGES = ["append", "indexer", "topk", "attention"]


def run_decode(args, workload):
    import numpy as np
    import torch

    from long_context_attention_14_amd import ops, pipeline
    from synth import gen
    from synth.configs import CSA_DECODE_1M, HCA_DECODE, HYBRID_DECODE_1M

    dev = "cuda"
    total_steps = args.warmup + args.steps
    if workload == "hybrid_decode_1m":
        base = HYBRID_DECODE_1M.with_(rope_base=args.rope_base)
        ds = gen.hybrid_inputs(base, extra_entries=total_steps // base.m + 2)
        cfgs = [base if d["kind"] == "C" else base.with_(m=d["m"]) for d in ds]
    else:
        base = (CSA_DECODE_1M if workload == "csa_decode_1m" else HCA_DECODE).with_(
            rope_base=args.rope_base)
        ds = [gen.decode_inputs(base, extra_entries=total_steps // base.m + 2)]
        cfgs = [base]
    paged = {"seed": 1} if args.paged else None
    B = base.B

    def touched_bytes(c, d):
        """HBM bytes one decode step of this layer reads or writes (algorithmic)."""
        rb = ops.row_bytes(c.kv_dtype, c.c)
        vis = float((d["lengths"] // d["m"]).sum())
        n = (B * c.k if d["kind"] == "C" else vis) + B * c.n_win
        b = n * rb + 2 * B * c.H * c.c * 2
        if d["kind"] == "C":
            b += vis * (ops.row_bytes(c.idx_dtype, c.d_I) + (4 if c.idx_dtype == "mxfp4" else 0))
        return b

    # Cold caches: the steps rotate over n_copies copies of every layer's state,
    # so that more than 1 GiB -- four times the 256 MB Infinity Cache -- is touched
    # between two uses of the same copy and no step finds its inputs cached.
    est = sum(touched_bytes(c, d) for c, d in zip(cfgs, ds))
    n_copies = 1 if args.warm else max(2, int(np.ceil(float(1 << 30) / est)) + 1)
    sets = [[pipeline.DecodeLayer(c, d, dev, paged=paged) for c, d in zip(cfgs, ds)]
            for _ in range(n_copies)]
    layers = sets[0]
    hip = HipEvents()
    it = [0]

    def step(evs=None):
        ls = sets[it[0] % n_copies]
        it[0] += 1
        for i, (c, L) in enumerate(zip(cfgs, ls)):
            csa = L.mode == "csa"
            ops.lca_decode_step(L.state, L.tokC, L.tokZ, L.q, L.out, c.io_dtype,
                                qI=L.qI if csa else None, qI_scale=L.qI_scale if csa else None,
                                w=L.w if csa else None, lse=L.lse, idx_out=L.idx if csa else None,
                                workspace=L.workspace, stage_events=evs[i] if evs else None)

    _calibrate_copy(args.calibrate_copy, dev)
    if not args.no_touch:
        _touch_pages(sets, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: on every 4th step, the indexer's dispatch stamps (CSA) or two
    # events around the attention stage (HCA alone).
    csa_layers = [i for i, L in enumerate(layers) if L.mode == "csa"]
    dom_layers = csa_layers if csa_layers else [0]
    dom = (1, 2) if csa_layers else (3, 4)          # indexer or attention stage
    SAMPLE = args.stamp_every  # stamped steps: the event packets themselves cost GPU time
    sampled = {}
    for i in range(0, args.steps, SAMPLE):
        sampled[i] = {li: (hip.create(), hip.create()) for li in dom_layers}

    def evs_for(i):
        if i not in sampled:
            return None
        out = []
        for li in range(len(layers)):
            e = [None] * 5
            if li in sampled[i]:
                e[dom[0]], e[dom[1]] = sampled[i][li]
            out.append(e)
        return out

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs_for(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_time = float(np.mean([hip.elapsed_s(*sampled[i][li]) for i in sampled for li in dom_layers]))
    for i in sampled:
        for a, b in sampled[i].values():
            hip.destroy(a)
            hip.destroy(b)
    # per-(layer, stage) breakdown from an untimed diagnostic loop with all events
    n_diag = min(args.steps, 10)
    events = [[[hip.create() for _ in range(5)] for _ in layers] for _ in range(n_diag)]
    for i in range(n_diag):
        step(events[i])
    torch.cuda.synchronize()
    per = np.zeros((len(layers), 4))
    for ev in events:
        for li, le in enumerate(ev):
            for j in range(4):
                per[li, j] += hip.elapsed_s(le[j], le[j + 1])
    per /= n_diag
    for ev in events:
        for le in ev:
            for e in le:
                hip.destroy(e)
    ms_per_step = elapsed / args.steps * 1e3
    value = B * args.steps / elapsed
    # tokens each copy's sequences have when a timed step runs (the copies advance in turn)
    steps_done = (np.arange(args.steps) + args.warmup) // n_copies

    def vis_mean(d):
        return float(np.mean([((d["lengths"] + s) // d["m"]).sum() for s in steps_done]))

    step_bytes = 0.0
    for c, d, L in zip(cfgs, ds, layers):
        rb = ops.row_bytes(c.kv_dtype, c.c)
        nsel = B * c.k if L.mode == "csa" else vis_mean(d)
        step_bytes += (nsel + B * c.n_win) * rb + 2 * B * c.H * c.c * 2
        if L.mode == "csa":
            step_bytes += vis_mean(d) * ops.row_bytes(c.idx_dtype, c.d_I) * (1 + (4 / 64 if c.idx_dtype == "mxfp4" else 0))
    if csa_layers:
        # dominant kernel: the indexer; algorithmic bytes per launch = every visible
        # key (+ its E8M0 scales for MXFP4) + queries and head weights
        c0 = cfgs[csa_layers[0]]
        key_b = ops.row_bytes(c0.idx_dtype, c0.d_I) + (4 if c0.idx_dtype == "mxfp4" else 0)
        idx_bytes = np.mean([vis_mean(ds[i]) * key_b + B * c0.H_I * (key_b + 4) for i in csa_layers])
        achieved = idx_bytes / dom_time / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": _indexer_traffic() if workload == "csa_decode_1m" else None,
                # rows of this length take the fused indexer + selection kernel
                "kernel": f"indexer_select_kernel<{c0.idx_dtype}>"}
    else:
        # HCA only: dominant kernel is the attention over all visible entries + window
        c0, d0 = cfgs[0], ds[0]
        rb = ops.row_bytes(c0.kv_dtype, c0.c)
        att_bytes = (vis_mean(d0) + B * c0.n_win) * rb + 2 * B * c0.H * c0.c * 2
        achieved = att_bytes / dom_time / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                "kernel": "attention stage: attn_decode_kernel + attn_merge4_kernel"}
    desc = {
        "csa_decode_1m": "csa_decode_b16_1m: batch 16, context 2^20 + U{0..3}, m=4 (262144 entries), "
                         "fp8 indexer 64x128, top-1024, MQA 64x512 bf16, window 128",
        "hca_decode": "hca_decode_b32_128k: batch 32, context 131072 + U{0..127}, m'=128 (1024 "
                      "entries), dense MQA 64x512 bf16, window 128",
        "hybrid_decode_1m": "hybrid8_decode_b4_1m: batch 4, context 2^20 + U{0..127}, layers "
                            "H,H,C,H,C,H,C,H, MXFP4 indexer 64x128, top-1024, KV fp8 + bf16 rope "
                            "dims, MQA 64x512, window 128",
    }[workload]
    result = {
        "metric": "CSA/HCA decode query-tokens/s at 1M ctx + achieved HBM GB/s vs peak",
        "value": value, "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"csa_decode_1m": "fp8 indexer / bf16 KV / fp32 accumulate",
                  "hca_decode": "bf16 KV / fp32 accumulate",
                  "hybrid_decode_1m": "mxfp4 indexer / fp8+bf16 KV / fp32 accumulate"}[workload],
        "data": "synthetic (seeded; N(0,1) and RMS-normalised rows)",
        "config": {"workload": desc, "global_batch": B, "seq_len": int(base.ctx),
                   "parallelism": "single GPU",
                   **({"rope_base": args.rope_base} if args.rope_base else {}),
                   **({"kv_cache": "paged, 128-token pages"} if args.paged else {}),
                   "caches": (f"cold: steps rotate over {n_copies} copies of the layer state, "
                              f"{(n_copies - 1) * est / 2 ** 30:.2f} GiB touched between two uses of a "
                              "copy (the Infinity Cache holds 256 MB)"
                              + ("" if args.no_touch else "; every copy made resident and the caches "
                                 "emptied before the warmup")) if n_copies > 1 else
                             "warm: one copy of the layer state, steps back to back"},
        "roofline": {**roof,
                     # the whole step's algorithmic bytes over its time, beside the
                     # dominant kernel's own fraction
                     "step_achieved": step_bytes / (ms_per_step * 1e-3) / 1e9,
                     "step_frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "dominant_kernel_us": dom_time * 1e6,
        "stages_us": {s: float(per[:, j].sum()) * 1e6 for j, s in enumerate(DECODE_STAGES)},
        "step_algorithmic_GBs": step_bytes / (ms_per_step * 1e-3) / 1e9,
    }
    if len(layers) > 1:
        result["layers_us"] = [{"kind": L.mode, **{s: float(per[i, j]) * 1e6 for j, s in
                                                   enumerate(DECODE_STAGES)}}
                               for i, L in enumerate(layers)]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(cfgs, ds, args.cpu_seconds)
    return result, per


def run_prefill(args):
    import numpy as np
    import torch

    from long_context_attention_14_amd import pipeline
    from synth import gen
    from synth.configs import CSA_PREFILL_CHUNK

    cfg = CSA_PREFILL_CHUNK.with_(rope_base=args.rope_base)
    dev = "cuda"
    d = gen.prefill_inputs(cfg)
    layer = pipeline.PrefillLayer(cfg, d, dev, paged={"seed": 1} if args.paged else None)
    stages = [("compress", layer.compress), ("window", layer.window_kv), ("indexer", layer.indexer),
              ("topk", layer.topk), ("attention", layer.attention)]
    _calibrate_copy(args.calibrate_copy, dev)
    for _ in range(args.warmup):
        layer.run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        for j, (_, f) in enumerate(stages):
            f()
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e-3
           for j, (n, _) in enumerate(stages)}
    ms_per_step = elapsed / args.steps * 1e3
    # dominant kernel: the indexer, MFMA-bound; algorithmic flops = every visible
    # (query, entry) pair x 64 heads x 128 dims x 2
    pos = cfg.ctx + np.arange(cfg.n_new)
    pairs = float(np.minimum((pos + 1) // cfg.m, layer.N_cap).sum())
    flops = pairs * cfg.H_I * cfg.d_I * 2
    achieved = flops / per["indexer"] / 1e12
    result = {
        "metric": "CSA prefill query-tokens/s + indexer MFMA TFLOP/s vs peak",
        "value": cfg.n_new * args.steps / elapsed, "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 indexer / bf16 KV / fp32 accumulate",
        "data": "synthetic (seeded; N(0,1) and RMS-normalised rows)",
        "config": {"workload": "csa_prefill_8k_on_128k: 8192 new tokens after a 131072-token "
                               "prefix, m=4 (34816 entries), fp8 indexer 64x128, top-1024, MQA "
                               "64x512 bf16, window 128",
                   "global_batch": 1, "seq_len": cfg.ctx + cfg.n_new, "parallelism": "single GPU",
                   **({"rope_base": args.rope_base} if args.rope_base else {}),
                   **({"kv_cache": "paged, 128-token pages"} if args.paged else {})},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP8_PEAK_TFLOPS, "traffic": None,
                     "kernel": "indexer_rows_kernel<fp8>"},
        "stages_us": {k: v * 1e6 for k, v in per.items()},
        "bf16_selector": bf16_selector(layer, args.steps),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefill(cfg, d, args.cpu_seconds)
    return result, per


def run_out_proj(args):
    """The grouped output projection after the attention (V4-Pro shape: 64 heads x
    512 in 8 groups -> 8 x 1024 -> 7168) for a decode batch (16 tokens: streams the
    184 MB of bf16 weights, HBM-bound) or a prefill chunk (8192 tokens: MFMA-bound)."""
    import numpy as np
    import torch

    from long_context_attention_14_amd import ops
    from synth import encode as enc
    from synth.configs import OUT_PROJ_DECODE, OUT_PROJ_PREFILL

    cfg = OUT_PROJ_DECODE if args.workload == "out_proj_decode" else OUT_PROJ_PREFILL
    T, n_h, c, g, d_g, d = cfg.T, cfg.n_h, cfg.c, cfg.g, cfg.d_g, cfg.d
    kin = n_h // g * c
    rng = np.random.default_rng(cfg.seed)
    dev = "cuda"
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    o = up(enc.to_bf16_bits(rng.standard_normal((T, n_h, c), dtype=np.float32) * 0.5))
    W_g = up(enc.to_bf16_bits(rng.standard_normal((g, d_g, kin), dtype=np.float32) / np.sqrt(kin)))
    W_o = up(enc.to_bf16_bits(rng.standard_normal((d, g * d_g), dtype=np.float32) / np.sqrt(g * d_g)))
    z = torch.empty((T, g * d_g), dtype=torch.int16, device=dev)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, ops.grouped_out_proj_workspace_size(T, n_h, c, g, d_g, d)),
                     dtype=torch.uint8, device=dev)
    call = lambda: ops.lca_grouped_out_proj(T, n_h, c, g, d_g, d, o, W_g, W_o, z, out, "bf16", ws)  # noqa: E731
    _calibrate_copy(args.calibrate_copy, dev)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(args.steps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per = ev[0].elapsed_time(ev[1]) * 1e-3 / args.steps
    flops = 2.0 * T * (g * d_g * kin + d * g * d_g)
    wbytes = 2.0 * (g * d_g * kin + d * g * d_g)
    io_bytes = 2.0 * T * (n_h * c + 2 * g * d_g + d)
    if T <= 64:
        roof = {"bound": "hbm", "achieved": (wbytes + io_bytes) / per / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / per / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof.update(frac=roof["achieved"] / roof["peak"], traffic=None,
                kernel="gemm_skinny_kernel" if T <= 32 else "gemm_bf16_kernel<128>")
    result = {
        "metric": "grouped output projection tokens/s", "value": T * args.steps / elapsed,
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 / fp32 accumulate",
        "data": "synthetic (seeded; N(0, 1/fan_in) weights)",
        "config": {"workload": f"{cfg.name}: {T} tokens, {n_h} heads x {c} in {g} groups -> "
                               f"{g} x {d_g} -> {d}", "global_batch": T, "seq_len": 0,
                   "parallelism": "single GPU"},
        "roofline": roof, "us_per_call": per * 1e6, "tflops": flops / per / 1e12,
        "weight_GBs": wbytes / per / 1e9,
    }
    return result, {"us_per_call": per * 1e6}


def run_hbm_ceiling(args):
    """The achievable HBM bandwidth on this GPU, for context beside the roofline
    fractions (which are quoted against the 8 TB/s specification): the library's
    read probe (every byte of a 512 MiB buffer read once; the buffer is twice the
    256 MB Infinity Cache, so repeated reads stream from HBM) and, for
    comparison, a 512 MiB device-to-device copy by torch (read + write)."""
    import torch

    from long_context_attention_14_amd import ops

    dev = "cuda"
    nbytes = 512 << 20
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(buf)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(args.steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e-3 / args.steps

    t_read = timed(lambda: ops.lca_read_bandwidth_probe(buf, sink))
    t_copy = timed(lambda: dst.copy_(buf))
    read_gbs = nbytes / t_read / 1e9
    copy_gbs = 2 * nbytes / t_copy / 1e9
    result = {
        "metric": "achievable HBM bandwidth (context for the roofline fractions)", "value": read_gbs,
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_read * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic (a 512 MiB buffer)",
        "config": {"workload": "hbm_ceiling: 512 MiB read once per step by lca_read_bandwidth_probe "
                               "(256 workgroups x 768 threads, two 16-byte loads per lane in flight)",
                   "global_batch": 1, "seq_len": 0, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": read_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": read_gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "read_probe_kernel"},
        "read_us": t_read * 1e6, "copy_us": t_copy * 1e6, "copy_GBs_read_plus_write": copy_gbs,
    }
    return result, {"read_us": t_read * 1e6, "copy_us": t_copy * 1e6}


def bf16_selector(layer, steps):
    """The pages' BF16-score variant of the indexer + top-k on the same chunk:
    its stage times, and the share of the float32 selection (layer.idx, from the
    timed runs) that it keeps; context, not a parity claim (each selection is
    exact for its own scores)."""
    import numpy as np
    import torch

    layer.indexer_bf16()
    layer.topk_bf16()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        layer.indexer_bf16()
        e[1].record()
        layer.topk_bf16()
        e[2].record()
    torch.cuda.synchronize()
    a = layer.idx.reshape(-1, layer.idx.shape[-1]).long()
    b = layer.idx16.reshape(-1, layer.idx16.shape[-1]).long()
    big = 1 << 40
    a_s = torch.where(a < 0, torch.full_like(a, big), a)
    pos = torch.searchsorted(a_s, torch.where(b < 0, torch.full_like(b, big + 1), b)).clamp(max=a.shape[1] - 1)
    hit = (torch.gather(a_s, 1, pos) == b) & (b >= 0)
    recall = float(hit.sum().item() / max(1, int((a >= 0).sum().item())))
    rows_equal = float((a == b).all(dim=1).float().mean().item())
    return {"indexer_us": float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3,
            "topk_us": float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3,
            "recall_vs_f32": recall, "rows_identical": rows_equal}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no "
              "multi-GPU path; batch sharding across GPUs is described in the design notes.",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "csa_prefill_chunk":
        result, per = run_prefill(args)
    elif args.workload.startswith("out_proj"):
        result, per = run_out_proj(args)
    elif args.workload == "hbm_ceiling":
        result, per = run_hbm_ceiling(args)
    else:
        result, per = run_decode(args, args.workload)
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"per_stage": per if isinstance(per, dict) else per.tolist(), "result": result}, f)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
