"""Benchmark: CSA decode at 1M context on one MI355X.

Workload: CSA decode step, batch 16 sequences of 2^20 + T_b tokens (m = 4 ->
262144 compressed entries each), fp8 indexer keys (64 heads x 128), top-1024,
multi-query attention over the selected bf16 entries (64 heads x 512) plus a
128-token window, bf16 in / fp32 accumulate.  One step = one decode token per
sequence through every stage of the path: state append (window KV, tail
block, compression of a block the token completes), indexer scores, top-k,
sparse attention with the window branch and the log-sum-exp merge.  Steps run
back to back, so the state advances (blocks complete every 4 steps).

Prints ONE JSON line.  The timed loop calls lca_decode_step; per-stage times
come from HIP events that the library records on the stream its kernels run on
(lca_decode_io.stage_events), over the timed region itself.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


class HipEvents:
    """hipEvent_t handles from the HIP runtime, recorded by the library itself on
    the stream its kernels run on."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")

    def create(self):
        e = self.ct.c_void_p()
        assert self.lib.hipEventCreate(self.ct.byref(e)) == 0
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--detail", default=None, help="write per-stage timings (JSON) to this file")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before warmup, run one plain device-to-device copy of MIB MiB (a "
                         "kernel of known traffic for scaling rocprofv3 byte counters)")
    return ap.parse_args()


def cpu_baseline(cfg, d, budget_s):
    """The float64 oracle (as is) on a bounded sample: whole decode steps of the
    first sequences of the same batch, until about budget_s of CPU time."""
    import numpy as np
    from oracle.workloads import oracle_decode
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    done, t0 = 0, time.perf_counter()
    while done < cfg.B:
        oracle_decode(cfg, d, done)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {cfg.B} sequences, one full decode step each "
                      f"({el:.1f} s, float64 numpy)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no "
              "multi-GPU path; batch sharding across GPUs is described in the design notes.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from long_context_attention_14_amd import ops, pipeline
    from synth import gen
    from synth.configs import CSA_DECODE_1M

    cfg = CSA_DECODE_1M
    dev = "cuda"
    total_steps = args.warmup + args.steps
    d = gen.decode_inputs(cfg, extra_entries=total_steps // cfg.m + 2)
    layer = pipeline.DecodeLayer(cfg, d, dev)
    B, m = cfg.B, cfg.m
    stages = ["append", "indexer", "topk", "attention"]
    hip = HipEvents()

    def step(ev=None):
        ops.lca_decode_step(layer.state, layer.tokC, layer.tokZ, layer.q, layer.out, cfg.io_dtype,
                            qI=layer.qI, w=layer.w, lse=layer.lse, idx_out=layer.idx,
                            workspace=layer.workspace, stage_events=ev)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[hip.create() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_stage = {s: [] for s in stages}
    for ev in events:
        for j, s in enumerate(stages):
            per_stage[s].append(hip.elapsed_s(ev[j], ev[j + 1]))
    for ev in events:
        for e in ev:
            hip.destroy(e)
    avg = {s: float(np.mean(v)) for s, v in per_stage.items()}
    ms_per_step = elapsed / args.steps * 1e3
    value = B * args.steps / elapsed

    # dominant kernel: the indexer.  Algorithmic bytes per launch: every visible
    # entry's 128-byte fp8 key, plus the 64x128 fp8 query and 64 fp32 weights of
    # each sequence (the fp32 score output is not counted).
    n_vis_mean = float(np.mean([((d["lengths"] + args.warmup + i) // m).sum() for i in range(args.steps)]))
    idx_bytes = n_vis_mean * cfg.d_I + B * cfg.H_I * (cfg.d_I + 4)
    achieved = idx_bytes / avg["indexer"] / 1e9
    # traffic from the committed rocprofv3 counter summary of this kernel, if current
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "indexer_fp8_decode_b16_1m_counters.txt")
    if os.path.exists(tfile):
        kv = dict(l.split(":", 1) for l in open(tfile) if ":" in l and not l.startswith("#"))
        src = os.path.join(ROOT, "long_context_attention_14_amd", "csrc", "indexer.hip")
        import hashlib
        cur = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if kv.get("indexer_source_sha256_16", "").strip() == cur and "hbm_bytes_per_launch" in kv:
            traffic = float(kv["hbm_bytes_per_launch"])
    step_bytes = idx_bytes + B * (cfg.k * cfg.c * 2 + cfg.n_win * cfg.c * 2 + 2 * cfg.H * cfg.c * 2)
    result = {
        "metric": "CSA/HCA decode query-tokens/s at 1M ctx + achieved HBM GB/s vs peak",
        "value": value, "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8 indexer / bf16 KV / fp32 accumulate",
        "data": "synthetic (seeded; N(0,1) and RMS-normalised rows)",
        "config": {"workload": "csa_decode_b16_1m: batch 16, context 2^20 + U{0..3}, m=4 "
                               "(262144 entries), fp8 indexer 64x128, top-1024, MQA 64x512 bf16, "
                               "window 128",
                   "global_batch": B, "seq_len": int(cfg.ctx), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "indexer_mfma_kernel<fp8>"},
        "stages_us": {s: v * 1e6 for s, v in avg.items()},
        "step_algorithmic_GBs": step_bytes / (ms_per_step * 1e-3) / 1e9,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_seconds)
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"per_stage_s": per_stage, "result": result}, f)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
