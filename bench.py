#!/usr/bin/env python3
"""Benchmark of the fused FP8 MQA-logits + top-k prefill path on one MI355X.

One step = one mqa_topk_prefill call over the whole 16384-row x 131072-key
chunk (row i sees keys [0, 114689 + i), top-2048), inputs resident in HBM.
Prints ONE JSON line (rank 0):
  value    = visible (row, key) scores per second (sum of the rows' visible
             keys / seconds per step);
  roofline = FP8 MFMA roofline of the scan kernel (the dominant one of the
             call's ten launches): 8192 flop per visible pair (2 * 32 heads *
             128 dims) over its average duration, timed with HIP events that
             the library records on the call's stream around that kernel
             (MQA_FLAG_TIME_SCAN) during the timed steps, against the MI355X
             dense FP8 peak (5.0 PFLOP/s); traffic = HBM bytes per launch from
             the committed rocprofv3 counter summary when it was taken on the
             current kernel sources, else null; measured_peak = the FP8 MFMA
             rate this GPU sustains on the scan's head-tile instruction (the
             mqa_mfma_peak probe, best of 3 launches) and measured_frac =
             achieved / measured_peak; call_frac = the whole call's FP8
             fraction (8192 flop per visible pair over ms_per_step);
  timing   = per-call medians and minima of 10 single calls, warm and with a
             512 MiB buffer written before each call (flushed caches);
  cpu_baseline = the CPU oracle (exact logits + full sort) timed on this
             host's cores over a bounded sample of the same rows.
Flags: --gpus N (only 1 is supported), --steps K, --warmup W, --no-cpu,
--dense (also time the chunked dense logits + top-k path, for context: serially
and with its chunk pairs on two streams, reporting the faster; --dense-serial
times the serial schedule only),
--config N (workload 1..5), --deterministic (MQA_FLAG_DETERMINISTIC: ties at
the k-th score to the smallest keys, outputs sorted), --heads 64 (the same
workload with 64 index heads), --paged P (read the keys
from a paged indexer cache of P-token pages through mqa_topk_prefill_paged
instead of the gathered keys and decoded scales), --decode N [--decode-rows R
--decode-ctx C] (instead of the benchmark: the decode-shaped path over N
requests of R rows, each with C positions of context, one JSON line),
--twolevel (instead of the benchmark: the two-level selection's source and
consumer calls at config 3's shape, top-512, one JSON line), --sweep (instead of the benchmark: fused and
dense times on the causal-tail sweep, 16384 rows x 16K..1M keys, one JSON line
per point), --copy-calibration MIB (instead of the benchmark,
run a plain 1-D device copy of MIB MiB five times: the known-size kernel that
scales rocprofv3's FETCH_SIZE / WRITE_SIZE readings to bytes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA (published)
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E (published)
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA (published)
FLOP_PER_PAIR = 2 * 32 * 128
COUNTERS = os.path.join(ROOT, "profiles", "fused_topk_cfg3_counters.json")
SOURCES = ["fp8_mqa_logits_amd/csrc/fused.hip", "fp8_mqa_logits_amd/csrc/common.h",
           "fp8_mqa_logits_amd/csrc/launch.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for s in SOURCES:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_counters(workload: str):
    """HBM bytes per fused-kernel launch from the committed counter summary,
    or None when the summary is missing, was taken on other sources or on
    another workload."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash() or c.get("workload") != workload:
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(wl, target_s: float = 15.0):
    """Time the oracle (as it stands) on a bounded sample of the workload."""
    import numpy as np

    import oracle

    host_cores = os.cpu_count() or 1
    threads = min(16, host_cores)  # the GPU machine's share of the host is 16 threads
    p = oracle.Problem(wl.q, wl.k, oracle.key_scales(wl.scale_bytes), wl.weights, wl.starts,
                       wl.ends)
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(wl.rows, size=wl.rows, replace=False))
    s = np.clip(wl.starts.astype(np.int64), 0, wl.keys)
    e = np.clip(wl.ends.astype(np.int64), s, wl.keys)
    # calibrate on a few rows per thread, then size the sample to about
    # target_s seconds
    probe = rows[:4 * threads]
    t0 = time.perf_counter()
    oracle.topk(p, probe, wl.topk, threads=threads)
    dt = time.perf_counter() - t0
    rate = float((e[probe] - s[probe]).sum()) / max(dt, 1e-6)
    per_row = float((e - s).mean())
    nrows = int(max(threads, min(wl.rows, target_s * rate / per_row)))
    nrows = (nrows + threads - 1) // threads * threads
    sample = rows[4 * threads:4 * threads + nrows]
    t0 = time.perf_counter()
    oracle.topk(p, sample, wl.topk, threads=threads)
    dt = time.perf_counter() - t0
    pairs = float((e[sample] - s[sample]).sum())
    return {"value": pairs / dt, "unit": "scores/s", "cores": threads, "kind": "oracle",
            "host_cores": host_cores, "cpu_model": cpu_model(),
            "sample": f"{len(sample)} seeded random rows of the same workload "
                      f"({int(pairs)} visible pairs), exact logits + full sort per row, "
                      f"{dt:.1f} s on {threads} threads"}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def per_call_times(step, stream, dev, n: int = 10):
    """Whole-call times (ms) of n single calls each, warm (inputs and the
    previous call's data in the caches) and flushed (512 MiB written by another
    kernel before each call); medians and minima."""
    import statistics

    import torch

    flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)

    def run(flushed):
        t = []
        for _ in range(n):
            if flushed:
                flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return t

    warm, flushed = run(False), run(True)
    return {"calls": n, "warm_median_ms": statistics.median(warm), "warm_min_ms": min(warm),
            "flushed_median_ms": statistics.median(flushed), "flushed_min_ms": min(flushed),
            "flush_bytes": flush.numel() * 4}


def time_dense(d, wl, steps: int, warmup: int, two_streams: bool = True):
    """Chunked dense path: logits for floor(2^27 / ncols) rows at a time (the
    512 MiB logits budget) over each chunk's key window, then per-row top-k.
    Timed two ways: serial (every call on one stream, one logits buffer) and
    pipelined (chunk i's pair on stream i % 2 with its own buffer, so that
    chunk i's top-k, bound by HBM latency, runs beside chunk i + 1's logits,
    bound by the MFMA; each buffer's reuse stays ordered on its stream).
    Returns (pipelined ms, serial ms, call pairs, per-kernel split, rows whose
    key sets differ between the two schedules: the top-k kernel takes ties at
    the k-th logit in the order its atomics land, so a row with such a tie can
    differ between any two runs). two_streams=False times the serial schedule
    only (pipelined ms and differing rows are then None), so that a kernel
    trace holds no overlapped dispatches."""
    import torch

    import fp8_mqa_logits_amd as mqa

    starts, ends = wl.starts.astype("int64"), wl.ends.astype("int64")
    chunks = []
    r0 = 0
    while r0 < wl.rows:
        # rows per call from the remaining rows' key window, then that chunk's own window
        nr = max(1, (1 << 27) // max(int(ends[r0:].max() - starts[r0:].min()), 1))
        r1 = min(wl.rows, r0 + nr)
        lo, hi = int(starts[r0:r1].min()), int(ends[r0:r1].max())
        chunks.append((r0, r1, lo, max(hi - lo, 1)))
        r0 = r1
    max_r = max(c[1] - c[0] for c in chunks)
    max_c = max(c[3] for c in chunks)
    bufs = [torch.empty(max_r * ((max_c + 3) // 4 * 4), dtype=torch.float32, device="cuda")
            for _ in range(2)]
    outs = [torch.empty((wl.rows, wl.topk), dtype=torch.int32, device="cuda") for _ in range(2)]
    main_s = torch.cuda.current_stream()
    side_s = torch.cuda.Stream()  # default priority, like every stream here

    def pair(i, buf, out, stream):
        r0, r1, lo, nc = chunks[i]
        ld = (nc + 3) // 4 * 4
        lg = buf[:(r1 - r0) * ld].view(r1 - r0, ld)[:, :nc]
        mqa.mqa_logits_dense(d["q"][r0:r1], d["k"], d["scales"], d["weights"][r0:r1],
                             d["starts"][r0:r1], d["ends"][r0:r1], col0=lo, ncols=nc,
                             logits=lg, stream=stream)
        mqa.mqa_topk_dense(lg, d["starts"][r0:r1], d["ends"][r0:r1], wl.topk, wl.keys,
                           col0=lo, out=out[r0:r1], stream=stream)

    def serial():
        for i in range(len(chunks)):
            pair(i, bufs[0], outs[0], main_s)

    def pipelined():
        side_s.wait_stream(main_s)
        for i in range(len(chunks)):
            pair(i, bufs[i % 2], outs[1], side_s if i % 2 else main_s)
        main_s.wait_stream(side_s)

    def timed(step):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(steps):
            step()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    serial_ms = timed(serial)
    pipe_ms, same = None, None
    if two_streams:
        pipe_ms = timed(pipelined)
        # rows whose key sets (unordered output) differ between the schedules
        same = int((torch.sort(outs[0], dim=1).values != torch.sort(outs[1], dim=1).values)
                   .any(dim=1).sum().item())
    # one more serial step with events around every call: the two kernels'
    # shares, and the bytes the logits pass writes (whole windows, -inf outside
    # ranges)
    evs = []
    for i in range(len(chunks)):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        r0, r1, lo, nc = chunks[i]
        ld = (nc + 3) // 4 * 4
        lg = bufs[0][:(r1 - r0) * ld].view(r1 - r0, ld)[:, :nc]
        e[0].record()
        mqa.mqa_logits_dense(d["q"][r0:r1], d["k"], d["scales"], d["weights"][r0:r1],
                             d["starts"][r0:r1], d["ends"][r0:r1], col0=lo, ncols=nc, logits=lg)
        e[1].record()
        mqa.mqa_topk_dense(lg, d["starts"][r0:r1], d["ends"][r0:r1], wl.topk, wl.keys,
                           col0=lo, out=outs[0][r0:r1])
        e[2].record()
        evs.append(e)
    torch.cuda.synchronize()
    split = {"logits_ms": sum(e[0].elapsed_time(e[1]) for e in evs),
             "topk_ms": sum(e[1].elapsed_time(e[2]) for e in evs),
             "logits_bytes_written": sum((r1 - r0) * nc * 4 for r0, r1, lo, nc in chunks)}
    del bufs
    return pipe_ms, serial_ms, len(chunks), split, same


def to_device(wl, dev):
    import torch

    import fp8_mqa_logits_amd as mqa
    d = {
        "q": torch.from_numpy(wl.q).to(dev),
        "k": torch.from_numpy(wl.k).to(dev),
        "weights": torch.from_numpy(wl.weights).to(dev),
        "starts": torch.from_numpy(wl.starts).to(dev),
        "ends": torch.from_numpy(wl.ends).to(dev),
    }
    d["scales"] = mqa.mqa_key_scales(torch.from_numpy(wl.scale_bytes).to(dev))
    return d


def time_fused(d, wl, steps: int, warmup: int):
    import torch

    import fp8_mqa_logits_amd as mqa
    ws = mqa.alloc_workspace(wl.rows)
    out = torch.empty((wl.rows, wl.topk), dtype=torch.int32, device="cuda")

    def step():
        mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"], d["ends"],
                             wl.topk, out=out, workspace=ws)
    mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"], d["ends"],
                         wl.topk, out=out, workspace=ws, flags=mqa.FLAG_STATS)
    stats = mqa.read_stats(ws)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, stats


def decode_bench(args):
    """The decode-shaped path: --decode REQUESTS requests of --decode-rows rows
    (speculative tokens of one request), each over --decode-ctx positions of
    its own pages (64-token pages), top-2048; inputs generated on the device.
    One JSON line: visible (row, key) scores per second, the scan kernel's
    FP8 MFMA fraction and the call's HBM fraction (each request's keys read
    once: 132 B per position)."""
    import torch

    import fp8_mqa_logits_amd as mqa
    import mqa_workloads as W
    torch.cuda.set_device(0)
    R, nreq, ctx, topk = args.decode_rows, args.decode, args.decode_ctx, 2048
    d = W.decode_device(nreq, R, ctx, topk, 64, seed=1)
    ws = torch.empty(mqa.workspace_size_decode(nreq, R), dtype=torch.uint8, device="cuda")
    out = torch.empty((d["rows"], topk), dtype=torch.int32, device="cuda")
    mode = mqa.FLAG_DETERMINISTIC if args.deterministic else 0

    def step(flags=0):
        mqa.mqa_topk_decode_paged(d["q"], d["cache"], d["table"], 64, d["weights"], d["starts"],
                                  d["ends"], topk, R, out=out, workspace=ws, flags=flags | mode)
    step(mqa.FLAG_STATS)
    torch.cuda.synchronize()
    stats = mqa.read_stats(ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step(mqa.FLAG_TIME_SCAN)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    scan_ms = mqa.scan_time_ms(args.steps) / args.steps
    pairs = d["pairs"]
    key_bytes = nreq * ctx * (128 + 4)
    achieved = pairs * FLOP_PER_PAIR / (scan_ms / 1e3) / 1e12
    print(json.dumps({
        "metric": "decode (row,key) scores/s", "value": pairs / (ms / 1e3), "unit": "scores/s",
        "ms_per_step": ms, "steps": args.steps, "warmup": args.warmup,
        "config": {"workload": f"decode_{nreq}req_x{R}rows_ctx{ctx}_k{topk}", "requests": nreq,
                   "rows_per_request": R, "context": ctx, "topk": topk, "page_size": 64,
                   "visible_pairs": pairs, "rows": d["rows"],
                   "ties": "lowest key, sorted output" if args.deterministic else "any"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP8_PEAK_TFLOPS,
                     "kernel": "fused_topk_kernel (decode)", "kernel_ms": scan_ms,
                     "call_frac": pairs * FLOP_PER_PAIR / (ms / 1e3) / 1e12 / FP8_PEAK_TFLOPS,
                     "hbm_key_bytes": key_bytes,
                     "hbm_frac_call": key_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "path_stats": stats}), flush=True)


def twolevel_bench(args):
    """DeepSeek-V4.1's two-level selection at config 3's shape (16384 rows x
    131072 keys, causal tail): the source call (top-512 keys and the 2048
    best blocks of 8 per row), the consumer call (top-512 of the keys in the
    source's blocks), and the plain top-512 call for reference. One JSON line
    of per-call times (event-timed averages)."""
    import torch

    import fp8_mqa_logits_amd as mqa
    import mqa_workloads as W
    torch.cuda.set_device(0)
    wl = W.config(3)
    d = to_device(wl, torch.device("cuda", 0))
    ws = mqa.alloc_workspace(wl.rows)
    k = 512
    out = torch.empty((wl.rows, k), dtype=torch.int32, device="cuda")
    ob = torch.empty((wl.rows, mqa.MAX_BLOCKS), dtype=torch.int32, device="cuda")
    args_ = (d["q"], d["k"], d["scales"], d["weights"], d["starts"], d["ends"])
    calls = {
        "plain_top512": lambda f=0: mqa.mqa_topk_prefill(*args_, k, out=out, workspace=ws, flags=f),
        "source_top512_blocks2048": lambda f=0: mqa.mqa_topk_prefill_blocks(
            *args_, k, out=out, out_blocks=ob, workspace=ws, flags=f),
        "consumer_top512_in_2048_blocks": lambda f=0: mqa.mqa_topk_masked(
            *args_, ob, k, out=out, workspace=ws, flags=f),
    }
    res = {}
    for name, fn in calls.items():
        fn(mqa.FLAG_STATS)
        torch.cuda.synchronize()
        st = mqa.read_stats(ws)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"ms_per_call": e0.elapsed_time(e1) / args.steps,
                     "rows_block_scan": st.get("rows_block_scan")}
    print(json.dumps({"metric": "two-level selection per-call time", "unit": "ms",
                      "config": {"workload": wl.name, "topk": k, "blocks": mqa.MAX_BLOCKS,
                                 "visible_pairs": wl.visible_pairs()},
                      "steps": args.steps, "warmup": args.warmup, "calls": res}), flush=True)


def sweep(args):
    """Fused vs dense on the causal tail of K-key contexts (16384 rows)."""
    import gc

    import torch

    import mqa_workloads as W
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    for topk in (2048, 512):
        for keys in (16384, 32768, 65536, 131072, 262144, 524288, 1048576):
            wl = W.sweep(keys, topk)
            d = to_device(wl, dev)
            fms, stats = time_fused(d, wl, 5, 2)
            pms, sms, ncalls, split, same = time_dense(d, wl, 2 if keys >= 262144 else 3, 1)
            dms = min(pms, sms)  # the faster dense schedule
            pairs = wl.visible_pairs()
            print(json.dumps({"sweep": wl.name, "keys": keys, "topk": topk, "rows": wl.rows,
                              "visible_pairs": pairs, "fused_ms": fms, "dense_ms": dms,
                              "dense_two_stream_ms": pms, "dense_serial_ms": sms,
                              "dense_rows_differing": same,
                              "dense_logits_ms": split["logits_ms"],
                              "dense_topk_ms": split["topk_ms"],
                              "dense_call_pairs": ncalls, "fused_over_dense": dms / fms,
                              "fused_tflops": pairs * FLOP_PER_PAIR / (fms / 1e3) / 1e12,
                              "path_stats": stats}),
                  flush=True)
            del d
            gc.collect()
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--dense", action="store_true")
    ap.add_argument("--dense-serial", action="store_true",
                    help="with --dense: time the serial schedule only (for kernel traces)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--paged", type=int, default=0, metavar="P")
    ap.add_argument("--heads", type=int, default=32, choices=(32, 64))
    ap.add_argument("--twolevel", action="store_true")
    ap.add_argument("--decode", type=int, default=0, metavar="REQUESTS")
    ap.add_argument("--decode-rows", type=int, default=8)
    ap.add_argument("--decode-ctx", type=int, default=131072)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this path runs on one GPU; multi-GPU runs are not supported "
              "(rows would shard across GPUs, each running the one-GPU path on its share)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return

    sys.path.insert(0, ROOT)
    import fp8_mqa_logits_amd as mqa
    import mqa_workloads as W

    if args.sweep:
        sweep(args)
        return
    if args.decode:
        decode_bench(args)
        return
    if args.twolevel:
        twolevel_bench(args)
        return

    wl = W.config(args.config)
    if args.heads == 64:
        # the same rows, keys and ranges with 64 index heads
        wl = W.heads64(wl.rows, wl.keys, wl.topk, wl.starts, wl.ends, seed=args.config,
                       name=wl.name + "_64heads")
    print(f"[bench] workload {wl.name}: {wl.visible_pairs()} visible pairs, hashes "
          f"{wl.hashes()}", file=sys.stderr, flush=True)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d = {
        "q": torch.from_numpy(wl.q).to(dev),
        "k": torch.from_numpy(wl.k).to(dev),
        "weights": torch.from_numpy(wl.weights).to(dev),
        "starts": torch.from_numpy(wl.starts).to(dev),
        "ends": torch.from_numpy(wl.ends).to(dev),
    }
    d["scales"] = mqa.mqa_key_scales(torch.from_numpy(wl.scale_bytes).to(dev))
    ws = torch.empty(mqa.workspace_size_heads(wl.rows, args.heads), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((wl.rows, wl.topk), dtype=torch.int32, device=dev)

    mode = mqa.FLAG_DETERMINISTIC if args.deterministic else 0

    if args.paged:
        ws = torch.empty(mqa.workspace_size_paged(wl.rows, wl.keys), dtype=torch.uint8,
                         device=dev)
        cache, table = W.paged_cache(wl.k, wl.scale_bytes, args.paged)
        d["cache"] = torch.from_numpy(cache).to(dev)
        d["table"] = torch.from_numpy(table).to(dev)

        def step(flags=0):
            mqa.mqa_topk_prefill_paged(d["q"], d["cache"], d["table"], args.paged, wl.keys,
                                       d["weights"], d["starts"], d["ends"], wl.topk, out=out,
                                       workspace=ws, flags=flags | mode)
    else:
        def step(flags=0):
            mqa.mqa_topk_prefill(d["q"], d["k"], d["scales"], d["weights"], d["starts"],
                                 d["ends"], wl.topk, out=out, workspace=ws, flags=flags | mode)

    # path statistics (one extra call outside the timed region)
    step(mqa.FLAG_STATS)
    torch.cuda.synchronize()
    stats = mqa.read_stats(ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step(mqa.FLAG_TIME_SCAN)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    scan_ms = mqa.scan_time_ms(args.steps) / args.steps
    timing = per_call_times(step, stream, dev)
    measured_peak = mqa.mfma_peak_tflops()
    pairs = wl.visible_pairs()
    value = pairs / (ms / 1e3)
    fpp = FLOP_PER_PAIR * args.heads // 32  # 2 * heads * 128 flop per visible pair
    achieved = pairs * fpp / (scan_ms / 1e3) / 1e12
    line = {
        "metric": "(row,key) scores/s + % FP8 MFMA peak, top-2048, 16K rows x 128K keys",
        "value": value,
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 MFMA, fp32 scores",
        "data": "synthetic (seeded N(0,1) e4m3 q/k, UE8M0 scales 2^[-4,0], N(0,1)/sqrt(32) weights)",
        "config": {"workload": wl.name, "rows": wl.rows, "keys": wl.keys, "topk": wl.topk,
                   "heads": args.heads, "visible_pairs": pairs, "parallelism": "1 GPU",
                   "ties": "lowest key, sorted output" if args.deterministic else "any",
                   "keys_from": (f"paged cache, {args.paged}-token pages" if args.paged
                                 else "gathered keys, decoded scales")},
        # the scan kernel's roofline (the dominant kernel); call_frac is the
        # whole call's FP8 fraction (all launches, the metric's own figure)
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP8_PEAK_TFLOPS,
                     "call_frac": pairs * fpp / (ms / 1e3) / 1e12 / FP8_PEAK_TFLOPS,
                     "traffic": traffic_from_counters(wl.name), "kernel": "fused_topk_kernel",
                     "kernel_ms": scan_ms, "measured_peak": measured_peak,
                     "measured_frac": achieved / measured_peak},
        "timing": timing,
        "path_stats": stats,
        "workspace_bytes": ws.numel(),
    }
    if args.dense:
        pms, sms, ncalls, split, same = time_dense(d, wl, max(1, args.steps // 4), 1,
                                                   two_streams=not args.dense_serial)
        line["dense_ms_per_step"] = min(pms, sms) if pms is not None else sms  # the faster schedule
        line["dense_two_stream_ms_per_step"] = pms  # chunk pairs overlapped
        line["dense_serial_ms_per_step"] = sms  # one stream
        # (a tie at the k-th logit makes a row differ between any two runs)
        line["dense_rows_differing"] = same
        line["dense_call_pairs"] = ncalls
        # the dense pair against its own bounds: the logits pass on the bf16
        # MFMA (the same 8192 FLOP per visible pair), its writes and the
        # top-k's reads (each visible logit once) on HBM
        lt, tt = split["logits_ms"], split["topk_ms"]
        line["dense_split"] = {
            "logits_ms": lt, "topk_ms": tt,
            "logits_bf16_tflops": FLOP_PER_PAIR * pairs / (lt * 1e-3) / 1e12,
            "logits_bf16_frac": FLOP_PER_PAIR * pairs / (lt * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "logits_write_gbs": split["logits_bytes_written"] / (lt * 1e-3) / 1e9,
            "topk_read_gbs": 4 * pairs / (tt * 1e-3) / 1e9,
            "topk_hbm_frac": 4 * pairs / (tt * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
