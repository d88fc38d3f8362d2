#!/usr/bin/env python3
"""Split-KV decode-attention benchmark on one MI355X.

Workload (default): few-KV-head long-context decode, B=1, one query token,
Hq=16, Hkv=2, D=256, L=5900 cached tokens, bf16, paged KV with page size 16
and a seeded random page permutation.  One step is one pass of the whole hot
path through the C ABI (splitkv_decode: the partial kernel, then the
log-sum-exp combine when a sequence has more than one split); the host plan is
made once per split count, outside the timed region, and its cost is reported
separately.

Cold cache: the page pool is replicated until the copies total >= 1 GiB and
step k reads copy k mod R through a block table offset by copy, so every step
streams its KV from HBM and not from L2 or MALL.  Outputs are bit-identical
across copies.

Prints ONE JSON line: metric / value (KV GB/s at the auto plan) / ms_per_step
/ the num_splits sweep / roofline of the dominant kernel / cpu_baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attention µs/step and KV GB/s (% of HBM peak) vs num_splits"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--L", type=int, default=5900)
    ap.add_argument("--sweep", type=str, default="1,2,3,4,6,8,12,16,24,32,48,64,96,128,192,256",
                    help="comma-separated num_splits to sweep ('' to skip); the workload's own "
                         "sweep is 1..64, larger counts are extra points")
    ap.add_argument("--only", type=int, default=None,
                    help="time one split count only (0 = auto); for profiler runs")
    ap.add_argument("--warm-cache", action="store_true", help="reuse one page pool copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def cold_copies(case, device, warm):
    """Replicate the page pool R times (>= 1 GiB total) with per-copy block tables."""
    import numpy as np
    import torch
    import synth
    t = synth.to_torch(case, device)
    pool = case.k_cache.nbytes + case.v_cache.nbytes
    R = 1 if warm else max(1, math.ceil((1 << 30) / pool))
    k = t["k_cache"].repeat(R, 1, 1, 1) if R > 1 else t["k_cache"]
    v = t["v_cache"].repeat(R, 1, 1, 1) if R > 1 else t["v_cache"]
    bt = case.block_table
    valid = bt != synth.INT32_MAX
    tables = []
    for r in range(R):
        b = bt.copy()
        b[valid] += r * case.num_pages
        tables.append(b)
    bts = torch.from_numpy(np.stack(tables)).to(device)
    return t["q"], k, v, bts, R


def time_steps(sess, bts, R, steps, warmup, stream):
    import torch
    for i in range(warmup):
        sess.set_block_table(bts[i % R])
        sess.decode()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        sess.set_block_table(bts[(warmup + i) % R])
        sess.decode()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / steps      # us per step


def time_steps_graph(sess, bts, R, steps, warmup, check=True):
    """Exactly `steps` decode steps replayed from one captured HIP graph.

    This is how a serving engine runs decode steps: the whole step sequence is
    captured once and replayed, so no host launch sits between kernels.  Step
    i of the graph reads page-pool copy i mod R.  The graph is replayed once
    untimed, then once timed.  With `check`, its output must equal the eager
    step's bit for bit.  Returns us per step.
    """
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(1, warmup)):
            sess.set_block_table(bts[i % R])
            sess.decode()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = sess.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            sess.set_block_table(bts[i % R])
            sess.decode()
    g.replay()
    torch.cuda.synchronize()
    if check:
        assert torch.equal(sess.out, ref), "graph replay output differs from the eager step"
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    if check:
        assert torch.equal(sess.out, ref), "graph replay output differs from the eager step"
    del g
    return start.elapsed_time(end) * 1e3 / steps


def time_partial_kernel(sess, bts, R, steps, stream):
    """Average duration of the partial kernel alone: an event pair around each launch."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        sess.set_block_table(bts[i % R])
        evs[i][0].record(stream)
        sess.partial()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) * 1e3 / steps


def cpu_baseline(case, seconds):
    """Time the fp64 oracle (as it stands) on the same workload, repeated ~`seconds`."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.attend(case)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_step = el / n
    return {"value": case.kv_bytes() / per_step / 1e9, "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{n} full oracle steps of the bench workload (fp64 numpy, {el:.1f} s); "
                      f"{per_step * 1e6:.0f} us per step"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is described in DESIGN.md, not run.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import synth
    import split_kv_amd
    from split_kv_amd.session import DecodeSession

    split_kv_amd.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    case = synth.few_kv_long(L=args.L, seed=1002)
    q, k, v, bts, R = cold_copies(case, dev, args.warm_cache)
    kv_bytes = case.kv_bytes()

    def session(n):
        t0 = time.perf_counter()
        s = DecodeSession(q=q, k_cache=k, v_cache=v, block_table=bts[0], seq_lens=case.seq_lens,
                          scale=case.scale, requested_splits=n, max_splits=256)
        return s, (time.perf_counter() - t0) * 1e6

    if args.only is not None:
        counts = [args.only]
    else:
        counts = [0] + [int(x) for x in args.sweep.split(",") if x.strip()]
    sweep = []
    head = None
    for n in counts:
        sess, plan_us = session(n)
        eager_us = time_steps(sess, bts, R, args.steps, args.warmup, stream)
        us = time_steps_graph(sess, bts, R, args.steps, args.warmup)
        rec = {"num_splits_requested": n, "num_splits": int(sess.num_splits_host[0]),
               "us_per_step": round(us, 3), "kv_GBps": round(kv_bytes / us / 1e3, 1),
               "pct_hbm_peak": round(100 * kv_bytes / us / 1e3 / HBM_PEAK_GBS, 2),
               "eager_us_per_step": round(eager_us, 3),
               "eager_kv_GBps": round(kv_bytes / eager_us / 1e3, 1)}
        if n == counts[0]:
            part_us = time_partial_kernel(sess, bts, R, args.steps, stream)
            head = dict(rec, plan_host_us=round(plan_us, 1), partial_kernel_us=round(part_us, 3),
                        sess=sess)
        sweep.append(rec)
        print(f"# n={n} -> {rec}", file=sys.stderr, flush=True)

    us = head["us_per_step"]
    part_us = head["partial_kernel_us"]
    achieved = kv_bytes / part_us / 1e3
    line = {
        "metric": METRIC,
        "value": head["kv_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "us_per_step": us,
        "pct_hbm_peak": head["pct_hbm_peak"],
        "timing": f"{args.steps} steps replayed from one captured HIP graph (step i reads "
                  f"page-pool copy i mod {R}), events around the replay; eager (one host "
                  f"launch per kernel): {head['eager_us_per_step']} us/step",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"few-KV-head long-context decode: B=1 T=1 Hq=16 Hkv=2 D=256 "
                               f"L={args.L} bf16 paged (P=16, permuted), "
                               f"{'warm' if args.warm_cache else 'cold'} cache ({R} pool copies)",
                   "num_splits": head["num_splits"],
                   "num_splits_requested": head["num_splits_requested"],
                   "kv_bytes_per_step": kv_bytes,
                   "plan_host_us": head["plan_host_us"]},
        "sweep": sweep,
        "roofline": {"bound": "hbm", "kernel": "gqa_partial_kernel<256,bf16>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_us": part_us},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
