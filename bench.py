#!/usr/bin/env python3
"""Split-KV decode-attention benchmark on one MI355X.

Workload of the bench line: few-KV-head long-context decode, B=1, one query
token, Hq=16, Hkv=2, D=256, L=5900 cached tokens, bf16, paged KV with page
size 16 and a seeded random page permutation.  One step is one pass of the
whole hot path through the C ABI (splitkv_decode: the partial kernel, then the
log-sum-exp combine when a sequence has more than one split); the host plan is
made once per split count, outside the timed region, and its cost is reported
separately.

Cold cache: the page pool is replicated until the copies total >= 1 GiB, and
every launch the bench makes -- eager or captured, warm-up or timed -- takes
the next copy of one rotation over all of them.  A copy is therefore read
again only after every other copy (>= 1 GiB, four times the 256 MB MALL) has
been streamed, whatever --steps is.  Outputs are bit-identical across copies.

Timing: K steps are captured in a HIP graph and replayed once untimed; then
five further graphs of K steps (each on the next K copies of the rotation) are
replayed between two events on their launch stream, and the median of the
five is reported.  The partial kernel alone is timed the same way for the
roofline object.

Prints ONE JSON line: metric / value (KV GB/s at the auto plan) /
ms_per_step / the num_splits sweep / roofline of the dominant kernel / the
floor (empty-kernel and plain-stream-read calibration) / cpu_baseline, plus an
`extra` list with the auto plan, sweep, roofline and monotonic check of every
other workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0
METRIC = "decode-attention µs/step and KV GB/s (% of HBM peak) vs num_splits"
BATCHES = 5
# Before the timed batches of a measurement, its first captured graph is
# replayed until this much GPU time has passed: a long kernel measured right
# after an idle spell reads several percent slow in its first batches (the MLA
# step at L=65536 gave 187.6, 178.8, 174.6, 172.0, 170.1 us over five batches
# after a 4 ms warm-up).
WARM_MS = 30.0
HEADLINE_SWEEP = "1,2,3,4,6,8,12,16,24,32,48,64,96,128,192,256"

# The other workloads, each carried in the default run's `extra` list: (name, L, split counts;
# 0 = the auto plan).
EXTRA = [
    ("tiny-gqa", 256, [0, 1, 2, 4]),
    ("few-kv-long", 260, [0, 1, 2, 4, 8, 16, 32, 64]),
    ("fp8-batched", None, [0, 1, 2, 4, 8, 16, 32]),
    ("mla", 2048, [0, 1, 4, 8, 16]),
    ("mla-fp8", 2048, [0, 1, 4, 8, 16]),
    ("mla-fp8q", 2048, [0, 1, 4, 8, 16]),
    ("mla", 65536, [0, 1, 4, 8]),
    ("mla-fp8", 65536, [0, 1, 4, 8]),
    ("mla-fp8q", 65536, [0, 1, 4, 8]),
    ("ragged", None, [0, 1, 4, 16, 64]),
]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="few-kv-long",
                    choices=["few-kv-long", "fp8-batched", "mla", "mla-fp8", "mla-fp8q", "ragged",
                             "tiny-gqa"],
                    help="few-kv-long is the headline; the others are extra measurements")
    ap.add_argument("--L", type=int, default=None, help="sequence length (few-kv-long, mla, mla-fp8, mla-fp8q, tiny-gqa)")
    ap.add_argument("--sweep", type=str, default=None,
                    help="comma-separated num_splits to sweep ('' to skip); the headline's own "
                         "sweep is 1..64, larger counts are extra points")
    ap.add_argument("--only", type=int, default=None,
                    help="time one split count only (0 = auto); for profiler runs")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--extra-steps", type=int, default=50,
                    help="steps per timed batch of the other workloads (at most --steps)")
    ap.add_argument("--warm-cache", action="store_true", help="reuse one page pool copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--append", action="store_true",
                    help="only time the KV append step (splitkv_append_kv) for the FP8 batch and "
                         "MLA decode shapes; an extra measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy, the known-size reference that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def make_workload(name, L):
    import synth
    if name == "few-kv-long":
        return synth.few_kv_long(L=L or 5900, seed=1002)
    if name == "fp8-batched":
        return synth.fp8_batched()
    if name == "mla":
        return synth.mla_decode(L=L or 65536)
    if name == "mla-fp8":
        return synth.mla_decode(L=L or 65536, kv_dtype=synth.KV_E4M3)
    if name == "mla-fp8q":
        return synth.mla_decode(L=L or 65536, kv_dtype=synth.KV_E4M3, fp8_queries=True)
    if name == "ragged":
        return synth.ragged()
    return synth.tiny_gqa(L=L or 256)


def describe(case, name):
    if name == "few-kv-long":
        return (f"few-KV-head long-context decode: B=1 T=1 Hq=16 Hkv=2 D=256 L={int(case.seq_lens[0])} "
                f"bf16 paged (P=16, permuted)")
    if name == "fp8-batched":
        return "batched GQA decode, e4m3 KV: B=8 T=1 Hq=32 Hkv=4 D=128 L=32000 P=16, bf16 Q"
    if name in ("mla", "mla-fp8", "mla-fp8q"):
        kind = "bf16"
        if case.kv_dtype == "e4m3":
            kind = "e4m3 cache, e4m3 Q (FP8 matrix path)" if case.q_scale else "e4m3 cache, bf16 Q"
        return f"MLA decode: B=1 T=6 Hq=128 latent 576/512 L={int(case.seq_lens[0])} P=64 {kind}"
    if name == "ragged":
        return f"ragged GQA decode: B=32 Hq=32 Hkv=8 D=128 bf16 P=16, sum L={int(case.seq_lens.sum())}"
    return (f"tiny GQA decode: B=1 T=1 Hq=8 Hkv=2 D=128 L={int(case.seq_lens[0])} contiguous bf16, "
            "fp32 out")


class Pool:
    """The workload's page pool replicated R times (>= 1 GiB in total), with one
    rotation shared by every launch: take(n) hands out the next n copies."""

    def __init__(self, case, device, warm):
        import numpy as np
        import torch
        import synth
        t = synth.to_torch(case, device)
        pool = case.k_cache.nbytes + (case.v_cache.nbytes if case.v_cache is not None else 0)
        R = 1 if warm else max(1, math.ceil((1 << 30) / pool))
        self.q = t["q"]
        self.k = t["k_cache"].repeat(R, 1, 1, 1) if R > 1 else t["k_cache"]
        v = t["v_cache"]
        self.v = v.repeat(R, 1, 1, 1) if (v is not None and R > 1) else v
        bt = case.block_table
        valid = bt != synth.INT32_MAX
        tables = []
        for r in range(R):
            b = bt.copy()
            b[valid] += r * case.num_pages
            tables.append(b)
        self.bts = torch.from_numpy(np.stack(tables)).to(device)
        self.R = R
        self.pool_bytes = pool
        self.i = 0

    def take(self, n):
        idx = [(self.i + j) % self.R for j in range(n)]
        self.i = (self.i + n) % self.R
        return idx


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def capture(sess, pool, n, fn, stream):
    """A HIP graph of n launches of fn, launch i reading the next copy of the rotation."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in pool.take(n):
            sess.set_block_table(pool.bts[c])
            fn()
    return g


def timed_graphs(sess, pool, fn, steps, stream, check=None):
    """us per launch of fn: untimed replays of one captured graph for at least
    WARM_MS of GPU time, then the median of BATCHES replays of freshly captured
    graphs, each between two events recorded on the stream the graph runs on
    (every timed graph reads the next `steps` copies of the rotation)."""
    import torch
    with torch.cuda.stream(stream):
        for c in pool.take(3):                # eager warm-up on the launch stream
            sess.set_block_table(pool.bts[c])
            fn()
    torch.cuda.synchronize()
    g = capture(sess, pool, steps, fn, stream)
    warm_ms, replays = 0.0, 0
    while warm_ms < WARM_MS and replays < 1000:
        e0, e1 = _events()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        warm_ms += e0.elapsed_time(e1)
        replays += 1
    del g
    if check:
        check()
    times = []
    for _ in range(BATCHES):
        g = capture(sess, pool, steps, fn, stream)
        e0, e1 = _events()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / steps)
        del g
        if check:
            check()
    return statistics.median(times), times


def time_eager(sess, pool, steps, stream):
    """us per step with one host launch per kernel (no graph)."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = _events()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for c in pool.take(steps):
            sess.set_block_table(pool.bts[c])
            sess.decode()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


COUNTERS = os.path.join(ROOT, "profiles", "gqa_partial_fewkv_L5900_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "split_kv_amd", "csrc", f) for f in ("gqa.hip", "device.h")]


def measured_traffic():
    """HBM bytes per launch of the headline partial kernel from the committed
    FETCH_SIZE / WRITE_SIZE counter runs, each scaled by what the same counter
    reads for a plain copy of known size; None when the kernel source has
    changed since the counters were taken (or they are missing)."""
    import hashlib
    try:
        vals = {}
        for line in open(COUNTERS):
            if ":" in line and not line.startswith(("#", " ", "|")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in KERNEL_SOURCES:
            h.update(open(f, "rb").read())
        if h.hexdigest()[:16] != vals["kernel_source_sha256_16"]:
            return None, "kernel changed since the counters were taken"
        copy = float(vals["copy_bytes"])
        fetch = float(vals["fetch_kib_per_dispatch"]) * copy / (1024 * float(vals["copy_fetch_kib"]))
        write = float(vals["write_kib_per_dispatch"]) * copy / (1024 * float(vals["copy_write_kib"]))
        return int(round((fetch + write) * 1024)), {
            "fetch_bytes": int(round(fetch * 1024)), "write_bytes": int(round(write * 1024)),
            "source": os.path.relpath(COUNTERS, ROOT)}
    except (OSError, KeyError, ValueError) as e:
        return None, f"counters unavailable: {e}"


def step_bytes(case, num_splits):
    """Bytes a step must move besides the KV (query in, output and LSE out),
    and the method's own overhead: the partials written by the partial kernel
    and read back by the combine (sequences with one split write their output
    directly and have none) -- fp32 m, l, o a row, or for MLA fp32 m, l, two
    scales and int16 codes of o."""
    rows = case.B * case.T * case.Hq
    q = rows * case.d_qk * 2
    out = rows * case.d_v * (4 if case.out_fp32 else 2) + rows * 4
    slots = int(sum(int(n) for n in num_splits if int(n) > 1))
    row_bytes = 2 * case.d_v + 16 if case.mla else (case.d_v + 2) * 4
    partials = slots * case.T * case.Hq * row_bytes
    return {"algorithmic_bytes_total": case.kv_bytes() + q + out,
            "partial_bytes_written_and_read": 2 * partials}


def monotonic(sweep, band=1.03):
    """The target's check: no split count slower than one split (within a
    3% run-to-run band), over the requested counts that were timed."""
    one = [r["us_per_step"] for r in sweep if r["num_splits_requested"] == 1]
    if not one:
        return None
    worst = max(sweep, key=lambda r: r["us_per_step"])
    ratio = worst["us_per_step"] / one[0]
    return {"ok": ratio <= band, "band": band, "worst_over_one_split": round(ratio, 4),
            "worst_request": worst["num_splits_requested"]}


def partial_kernel_name(case, sess=None):
    if case.mla:
        import split_kv_amd as sk
        if sess is not None and sk.splitkv_mla_short_range(sess.args):
            # the short-range kernels (64 rows, eight waves a workgroup)
            if case.q_scale:
                return "mla_short_q8_partial_kernel"
            return "mla_short_partial_kernel<%s>" % ("true" if case.kv_dtype == "e4m3" else "false")
        # kinds: 0 bf16 cache, 1 e4m3 cache with bf16 queries, 2 e4m3 cache and queries
        return "mla_partial_kernel<%d>" % (2 if case.q_scale else (1 if case.kv_dtype == "e4m3" else 0))
    return "gqa_partial_kernel<%d,%s>" % (case.d_qk, "e4m3" if case.kv_dtype == "e4m3" else "bf16")


def partial_grid(case, sess):
    """Workgroups of one partial-kernel launch."""
    if case.mla:
        import split_kv_amd as sk
        rows = case.T * case.Hq
        rpw = 64 if sk.splitkv_mla_short_range(sess.args) else sk.SPLITKV_ROWS_PER_WG_MLA
        return sess.total_slots * -(-rows // rpw)
    return sess.total_slots * case.Hkv * -(-(case.g * case.T) // 16)


def roofline(case, part_us, kernel=None):
    if case.mla:
        tokens = int(case.seq_lens.sum())
        flops_qk = 2 * case.T * case.Hq * case.d_qk * tokens
        flops_pv = 2 * case.T * case.Hq * case.d_v * tokens
        flops = flops_qk + flops_pv
        if case.q_scale and (kernel or "").startswith("mla_short_q8"):
            # the short-range e4m3-query kernel runs both products on FP8
            peak = MFMA_FP8_PEAK_TFLOPS
        elif case.q_scale:
            # e4m3 queries put the scores on the FP8 matrix path and keep the
            # value product on bf16: the peak is the rate of that mix, each
            # part at its own dtype's peak
            peak = round(flops / (flops_qk / MFMA_FP8_PEAK_TFLOPS + flops_pv / MFMA_BF16_PEAK_TFLOPS), 1)
        else:
            peak = MFMA_BF16_PEAK_TFLOPS
        return {"bound": "mfma", "kernel": kernel or partial_kernel_name(case),
                "achieved": round(flops / part_us / 1e6, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(flops / part_us / 1e6 / peak, 4),
                "traffic": None, "kernel_us": round(part_us, 3), "flops_per_launch": flops}
    kv = case.kv_bytes()
    achieved = kv / part_us / 1e3
    return {"bound": "hbm", "kernel": kernel or partial_kernel_name(case), "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None, "kernel_us": round(part_us, 3), "bytes_per_launch": kv}


KERNEL_LAUNCHES = 100


def measure(case, pool, counts, steps, stream, eager=True, log_prefix=""):
    """Sweep the split counts: us/step from graph replays (median of BATCHES),
    plus the partial kernel alone at the first count.  Returns (sweep, head)."""
    import torch
    from split_kv_amd.session import DecodeSession
    kv_bytes = case.kv_bytes()

    def session(n):
        t0 = time.perf_counter()
        s = DecodeSession(q=pool.q, k_cache=pool.k, v_cache=pool.v, block_table=pool.bts[0],
                          seq_lens=case.seq_lens, scale=case.scale, k_scale=case.k_scale,
                          v_scale=case.v_scale, mla=case.mla, requested_splits=n, max_splits=256,
                          out_fp32=case.out_fp32, q_scale=case.q_scale)
        return s, (time.perf_counter() - t0) * 1e6

    sweep, head = [], None
    for n in counts:
        sess, plan_us = session(n)
        eager_us = time_eager(sess, pool, steps, stream) if eager else None
        ref = {}

        def check():
            # every replayed step writes the same bits as the first eager step
            if not ref:
                ref["out"] = sess.out.clone()
            assert torch.equal(sess.out, ref["out"]), "graph replay output differs from the eager step"

        sess.set_block_table(pool.bts[pool.take(1)[0]])
        with torch.cuda.stream(stream):
            sess.decode()
        torch.cuda.synchronize()
        check()
        us, batches = timed_graphs(sess, pool, sess.decode, steps, stream, check=check)
        rec = {"num_splits_requested": n, "num_splits": int(sess.num_splits_host.max()),
               "total_slots": sess.total_slots,
               "us_per_step": round(us, 3), "kv_GBps": round(kv_bytes / us / 1e3, 1),
               "pct_hbm_peak": round(100 * kv_bytes / us / 1e3 / HBM_PEAK_GBS, 2),
               "batches_us": [round(x, 3) for x in batches]}
        if eager_us is not None:
            rec["eager_us_per_step"] = round(eager_us, 3)
        if n == counts[0]:
            # the kernel alone: graphs of at least KERNEL_LAUNCHES launches, so that a
            # graph's own launch cost is a small share of each launch at any --steps
            part_n = max(steps, KERNEL_LAUNCHES)
            part_us, part_batches = timed_graphs(sess, pool, sess.partial, part_n, stream)
            head = dict(rec, plan_host_us=round(plan_us, 1), partial_kernel_us=round(part_us, 3),
                        partial_batches_us=[round(x, 3) for x in part_batches],
                        partial_launches_per_graph=part_n,
                        partial_workgroups=partial_grid(case, sess),
                        partial_kernel=partial_kernel_name(case, sess),
                        num_splits_host=sess.num_splits_host.copy())
            if not case.mla:
                # the whole step as one launch (ticketed last-arriver merge), for comparison;
                # splitkv_decode takes it by itself only where it measured faster.  Its
                # merge adds in another order, so its replays are checked against its own
                # eager step.
                sess.set_block_table(pool.bts[pool.take(1)[0]])
                with torch.cuda.stream(stream):
                    sess.decode_single_launch()
                torch.cuda.synchronize()
                ref1 = sess.out.clone()

                def check1():
                    assert torch.equal(sess.out, ref1), "single-launch replay differs from its eager step"
                sl_us, _ = timed_graphs(sess, pool, sess.decode_single_launch, steps, stream, check=check1)
                head["single_launch_us_per_step"] = round(sl_us, 3)
        sweep.append(rec)
        print(f"# {log_prefix}n={n} -> {rec}", file=sys.stderr, flush=True)
        del sess
    return sweep, head


def floor_measurement(kv_bytes, grids, steps, stream):
    """Floors of a decode step on this GPU, measured with the library's
    calibration kernels from captured graphs: one empty kernel per node, a
    step of two empty kernels (the partial + combine shape), and a plain
    streaming read of the step's KV bytes with the given workgroup counts
    (each launch on the next chunk of a 1 GiB rotation, so from HBM), plus a
    1 GiB read with 4096 workgroups (the stream peak)."""
    import torch
    import split_kv_amd as sk
    dev = torch.device("cuda:0")
    gib = 1 << 30
    buf = torch.ones(gib // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    base = buf.data_ptr()
    chunk = -(-kv_bytes // (1 << 18)) * (1 << 18)
    nchunks = max(1, (gib - kv_bytes) // chunk)
    rot = {"i": 0}

    def graph_time(body, n_launch, reps=BATCHES):
        times = []
        for r in range(reps + 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(n_launch):
                    body()
            e0, e1 = _events()
            with torch.cuda.stream(stream):
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            if r:
                times.append(e0.elapsed_time(e1) * 1e3 / n_launch)
            del g
        return statistics.median(times)

    def empty():
        sk.splitkv_calib_empty(torch.cuda.current_stream().cuda_stream)

    def two_empty():
        empty()
        empty()

    out = {"empty_kernel_graph_us": round(graph_time(empty, steps), 3),
           "empty_two_kernel_step_us": round(graph_time(two_empty, steps), 3)}
    reads = []
    for wgs in grids:
        def read(wgs=wgs):
            off = (rot["i"] % nchunks) * chunk
            rot["i"] += 1
            sk.splitkv_calib_stream_read(base + off, kv_bytes, wgs, sink.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
        us = graph_time(read, steps)
        reads.append({"workgroups": wgs, "bytes": kv_bytes, "us": round(us, 3),
                      "GBps": round(kv_bytes / us / 1e3, 1)})

    def read_all():
        sk.splitkv_calib_stream_read(base, gib, 4096, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    us = graph_time(read_all, 4)
    reads.append({"workgroups": 4096, "bytes": gib, "us": round(us, 3), "GBps": round(gib / us / 1e3, 1)})
    out["stream_read"] = reads
    del buf
    out.update(unit_rates(sink, stream))
    del sink
    torch.cuda.empty_cache()
    return out


def unit_rates(sink, stream):
    """What the compute-bound (MLA) kernels' two inner resources deliver on
    this GPU, measured with the library's calibration kernels: the bf16
    32x32x16 matrix product issued back to back on every SIMD (one
    workgroup of four waves per CU), and conflict-free LDS reads (16-byte and
    transposing 8-byte) by four waves per CU.  Rates are per launch (events)
    and per core clock (the kernels' own s_memtime cycle counts)."""
    import numpy as np
    import torch
    import split_kv_amd as sk
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream

    def run(launch):
        launch()                                   # warm-up
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record()
        launch()
        e1.record()
        torch.cuda.synchronize()
        cyc = sink[:8 * cus].view(-1, 2)[:, 1].cpu().numpy().astype(np.uint32).astype(np.float64)
        return e0.elapsed_time(e1) * 1e3, float(np.median(cyc))

    iters = 20000
    us, cyc = run(lambda: sk.splitkv_calib_mfma(cus, iters, sink.data_ptr(), st))
    flops = cus * 4 * iters * 4 * 2 * 32 * 32 * 16
    out = {"mfma_bf16_32x32x16": {"tflops": round(flops / us / 1e6, 1),
                                  "cycles_per_product": round(cyc / (iters * 4), 2),
                                  "clock_ghz": round(cyc / us / 1e3, 3), "us": round(us, 1)}}
    lds = {}
    for mode, name, per_read in ((0, "ds_read_b128", 1024), (1, "ds_read_b64_tr_b16", 512)):
        it = 4000
        us, cyc = run(lambda: sk.splitkv_calib_lds_read(cus, it, mode, sink.data_ptr(), st))
        lds[name] = {"bytes_per_clock_per_cu": round(4 * it * 16 * per_read / cyc, 1), "us": round(us, 1)}
    out["lds_read"] = lds
    return out


def cpu_baseline(case, seconds):
    """Time the fp64 oracle (as it stands) on the same workload, repeated ~`seconds`,
    with its BLAS held to one thread (its per-row loops use one core either way)."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        n = 0
        while True:
            oracle.attend(case)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    per_step = el / n
    return {"value": round(case.kv_bytes() / per_step / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} full oracle steps of the bench workload (fp64 numpy, one thread, "
                      f"{el:.1f} s); {per_step * 1e6:.0f} us per step"}


def extra_record(name, L, counts, steps, stream, dev):
    import torch
    case = make_workload(name, L)
    pool = Pool(case, dev, False)
    sweep, head = measure(case, pool, counts, steps, stream, eager=False, log_prefix=f"{name} L={L} ")
    roof = roofline(case, head["partial_kernel_us"], head.get("partial_kernel"))
    rec = {"workload": describe(case, name),
           "kv_bytes_per_step": case.kv_bytes(),
           "cold_copies": pool.R,
           "auto": {"num_splits": head["num_splits"], "total_slots": head["total_slots"],
                    "us_per_step": head["us_per_step"], "kv_GBps": head["kv_GBps"],
                    "single_launch_us_per_step": head.get("single_launch_us_per_step"),
                    "pct_hbm_peak": head["pct_hbm_peak"], "plan_host_us": head["plan_host_us"],
                    **step_bytes(case, head["num_splits_host"])},
           "sweep": [{"n_req": r["num_splits_requested"], "n": r["num_splits"], "slots": r["total_slots"],
                      "us": r["us_per_step"], "GBps": r["kv_GBps"]} for r in sweep],
           "monotonic": monotonic(sweep),
           "roofline": roof}
    del pool
    torch.cuda.empty_cache()
    return rec


def copy_calibration():
    """A plain device-to-device copy of 256 MiB, repeated 5 times.

    Under rocprofv3 --pmc FETCH_SIZE (or WRITE_SIZE) the copy kernel's counter
    divided by 256 MiB is the factor that turns the counter into HBM bytes.
    """
    import torch
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def append_measurement(steps, warmup):
    """Time splitkv_append_kv from a captured graph for two decode shapes.

    FP8 batch: B=8 sequences, one new token, 4 KV heads of 128, e4m3 cache
    (keys and values quantised); MLA: one sequence, six new tokens of the
    576-wide latent row, bf16 cache.  Bytes = bf16 rows read + cache bytes
    written.  The append is latency-bound at these sizes (a few KB per call).
    """
    import numpy as np
    import torch
    import synth
    import split_kv_amd as sk
    sk.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = []
    shapes = [("fp8-batch append: B=8 T=1 Hkv=4 D=128 e4m3 cache", dict(
                   B=8, T=1, Hq=32, Hkv=4, d_qk=128, d_v=128, seq_lens=[4096] * 8, page_size=16,
                   kv_dtype=synth.KV_E4M3, seed=1003)),
              ("mla append: B=1 T=6 latent 576 bf16 cache", dict(
                   B=1, T=6, Hq=128, Hkv=1, d_qk=576, d_v=512, seq_lens=[4096], page_size=64,
                   mla=True, std=0.5, seed=1004))]
    for desc, kw in shapes:
        case = synth.make_case("append", **kw)
        t = synth.to_torch(case, dev)
        rng = np.random.default_rng(7)
        Tn, Hkv = case.T, case.Hkv
        kn = torch.from_numpy(synth.to_bf16_codes(rng.standard_normal(
            (case.B, Tn, Hkv, case.d_qk), dtype=np.float32)).view(np.int16)).to(dev)
        vn = None if case.mla else torch.from_numpy(synth.to_bf16_codes(rng.standard_normal(
            (case.B, Tn, Hkv, case.d_v), dtype=np.float32)).view(np.int16)).to(dev)
        pos = torch.from_numpy((case.seq_lens - Tn).astype(np.int32)).to(dev)
        kc, vc, bt = t["k_cache"], t["v_cache"], t["block_table"]
        a = sk.splitkv_append_args()
        a.k_new, a.v_new = kn.data_ptr(), (vn.data_ptr() if vn is not None else None)
        a.k_new_stride_b, a.k_new_stride_t, a.k_new_stride_h = kn.stride()[:3]
        if vn is not None:
            a.v_new_stride_b, a.v_new_stride_t, a.v_new_stride_h = vn.stride()[:3]
        a.k_cache, a.v_cache = kc.data_ptr(), (vc.data_ptr() if vc is not None else None)
        a.k_stride_page, a.k_stride_head, a.k_stride_tok = kc.stride()[:3]
        if vc is not None:
            a.v_stride_page, a.v_stride_head, a.v_stride_tok = vc.stride()[:3]
        a.block_table, a.bt_stride, a.positions = bt.data_ptr(), bt.shape[1], pos.data_ptr()
        a.B, a.T, a.Hkv, a.d_k, a.d_v = case.B, Tn, Hkv, case.d_qk, case.d_v
        a.page_size, a.num_pages = case.page_size, case.num_pages
        a.kv_dtype = sk.SPLITKV_KV_E4M3 if case.kv_dtype == synth.KV_E4M3 else sk.SPLITKV_KV_BF16
        a.k_scale, a.v_scale = case.k_scale, case.v_scale
        for _ in range(warmup):
            sk.splitkv_append_kv(a, stream.cuda_stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                sk.splitkv_append_kv(a, torch.cuda.current_stream().cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        elem = 1 if case.kv_dtype == synth.KV_E4M3 else 2
        rows = case.B * Tn * Hkv
        nbytes = rows * (case.d_qk + (0 if case.mla else case.d_v)) * (2 + elem)
        out.append({"workload": desc, "us_per_append": round(us, 3), "bytes": nbytes,
                    "GBps": round(nbytes / us / 1e3, 2)})
        print(f"# {desc}: {us:.3f} us per append ({nbytes} bytes read + written)", file=sys.stderr,
              flush=True)
    print(json.dumps({"metric": "KV append us per call", "unit": "us", "higher_is_better": False,
                      "data": "synthetic", "steps": steps, "timing": f"{steps} appends replayed "
                      "from one captured HIP graph, events around the replay",
                      "results": out, "note": "extra measurement; the bench line is the "
                      "few-kv-long workload"}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.append:
        append_measurement(args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the path would "
              "shard by sequence or KV head, or by KV range with one exchange of the partials "
              "before the combine, but no multi-GPU run is made.", file=sys.stderr)
        sys.exit(2)
    import torch
    import split_kv_amd

    split_kv_amd.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()          # every timed launch and its events live on this stream
    case = make_workload(args.workload, args.L)
    headline = args.workload == "few-kv-long" and args.L is None
    pool = Pool(case, dev, args.warm_cache)
    kv_bytes = case.kv_bytes()

    if args.only is not None:
        counts = [args.only]
    elif args.sweep is not None:
        counts = [0] + [int(x) for x in args.sweep.split(",") if x.strip()]
    elif args.workload == "few-kv-long":
        counts = [0] + [int(x) for x in HEADLINE_SWEEP.split(",")]
    else:
        counts = [0, 1, 4, 8, 16]
    # Warm-up: W eager steps and one discarded rehearsal of the first
    # configuration's measurement (the first captured-graph timing of a
    # process reads a few percent slow).
    from split_kv_amd.session import DecodeSession
    s0 = DecodeSession(q=pool.q, k_cache=pool.k, v_cache=pool.v, block_table=pool.bts[0],
                       seq_lens=case.seq_lens, scale=case.scale, k_scale=case.k_scale,
                       v_scale=case.v_scale, mla=case.mla, requested_splits=counts[0], max_splits=256,
                       out_fp32=case.out_fp32, q_scale=case.q_scale)
    time_eager(s0, pool, max(1, args.warmup), stream)
    timed_graphs(s0, pool, s0.decode, args.steps, stream)
    del s0
    sweep, head = measure(case, pool, counts, args.steps, stream)

    us = head["us_per_step"]
    roof = roofline(case, head["partial_kernel_us"], head.get("partial_kernel"))
    if headline and head["num_splits_requested"] == 0 and not args.warm_cache:
        traffic, detail = measured_traffic()
        roof["traffic"] = traffic
        roof["traffic_detail"] = detail
    timed_bytes = args.steps * kv_bytes
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
        "timing": f"median of {BATCHES} timed batches; each batch is {args.steps} steps replayed "
                  f"from one freshly captured HIP graph between two events on its launch stream; "
                  f"every launch of the run reads the next page-pool copy of one rotation over "
                  f"{pool.R} copies, so a copy is re-read only after >= 1 GiB of other copies; "
                  f"batches: {head['batches_us']} us/step; eager (one host launch per kernel): "
                  f"{head['eager_us_per_step']} us/step",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e4m3" if case.q_scale else "e4m3-kv/bf16") if case.kv_dtype == "e4m3" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{describe(case, args.workload)}, "
                               f"{'warm' if args.warm_cache else 'cold'} cache ({pool.R} pool copies)",
                   "num_splits": head["num_splits"],
                   "num_splits_requested": head["num_splits_requested"],
                   "step": "partial kernel, then combine kernel (skipped when every sequence has one split)",
                   "kv_bytes_per_step": kv_bytes,
                   "timed_batch_kv_bytes": timed_bytes,
                   "pool_copy_bytes": pool.pool_bytes,
                   **step_bytes(case, head["num_splits_host"]),
                   "plan_host_us": head["plan_host_us"],
                   "single_launch_us_per_step": head.get("single_launch_us_per_step")},
        "sweep": sweep,
        "monotonic": monotonic(sweep),
        "roofline": roof,
    }
    if not args.no_extra or headline:
        fl = floor_measurement(kv_bytes, sorted({head["partial_workgroups"], 256, 1024}), args.steps, stream)
        same = [r for r in fl["stream_read"] if r["workgroups"] == head["partial_workgroups"]][0]
        peak = fl["stream_read"][-1]
        fl["partial_pct_of_stream_same_grid"] = round(100 * roof["achieved"] / same["GBps"], 1) \
            if roof["unit"] == "GB/s" else None
        fl["step_pct_of_stream_peak"] = round(100 * head["kv_GBps"] / peak["GBps"], 1)
        fl["partial_workgroups"] = head["partial_workgroups"]
        line["floor"] = fl
    if not headline:
        line["note"] = "extra measurement; the bench line is the few-kv-long workload at L=5900"
    if headline and not args.no_extra and args.only is None:
        steps_x = max(1, min(args.steps, args.extra_steps))
        extra = []
        del pool
        torch.cuda.empty_cache()
        for name, L, cnts in EXTRA:
            t0 = time.perf_counter()
            rec = extra_record(name, L, cnts, steps_x, stream, dev)
            rec["steps_per_batch"] = steps_x
            extra.append(rec)
            print(f"# extra {name} L={L}: auto {rec['auto']['us_per_step']} us/step "
                  f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
        line["extra"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
