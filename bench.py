"""Benchmark of the per-step batched sampler on one MI355X.

One step = sample_batch (temperature -> top-k -> top-p -> draw for every
request) + write_tokens (token-pool scatter, async copy to pinned host
memory, completion ticket), on the workload the headline metric is quoted
on: B=256 requests, V=151936, fp32 logits 2*Gumbel + a rank-4 term, per-request
T ~ U[0.3, 1.5], top_k from {1, 20, 50, off}, top_p from {1, 0.95, 0.8}.
The step counter advances every step (fresh Philox counters); as in the
engine's overlapped loop, step s waits for the host copy of step s-1.
`value` is rows/s over the timed steps.  The roofline figure uses the mean
duration of sample_batch, from HIP events around a second run of the same
launches back to back on the launch stream.

Inputs are resident in HBM before timing.  The logits are copied into
several distinct device buffers used in rotation, so that repeated reads of
the same 155 MB cannot be served from the 256 MB Infinity Cache.

Prints ONE JSON line (stdout).  Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "sampled rows/sec and achieved HBM GB/s (% of peak) at B=256, V=151936"
PARAM_BYTES_PER_ROW = 4 + 4 + 4 + 8 + 4   # T, top_k, top_p, uid read; token written
C3_MIN_P_VALUES = [0.0, 0.02, 0.05, 0.1]
WRITE_BYTES_PER_ROW = 8 + 8 + 4 + 4       # row, col, token read; pool cell written
# calibration copy for the HBM byte counters: torch's elementwise negation of
# one fp32 logits buffer into another (one read and one write of each byte)
COPY_KERNEL_NEEDLE = "neg_kernel"
COPY_BYTES = 256 * 151936 * 4
# the kernel-only timing: untimed back-to-back launches first, then at least
# this many timed ones
KERNEL_WARMUP = 300
KERNEL_MIN = 300


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


# the files the sample_batch kernel is compiled from
KERNEL_SOURCES = ("device_common.hpp", "kernels.hpp", "sample_stream.hip")


def kernel_sources_digest() -> str:
    csrc = os.path.join(ROOT, "decode_step_token_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch from profiles/, if taken on the
    current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
        rec = data.get(f"{kernel}@{workload}")
        if rec and rec.get("sources_digest") == kernel_sources_digest():
            return rec.get("bytes_per_launch")
    except (OSError, ValueError):
        return None
    return None


def write_traffic(fetch_csv: str, write_csv: str, kernel: str, workload: str, command: str):
    """Turn two rocprofv3 --pmc counter files (FETCH_SIZE, then WRITE_SIZE, KiB
    per dispatch) into HBM bytes per launch of the sampler kernel, scaled by
    what the same counters read for the plain copy kernel that the
    --calibrate-copy run launches (known bytes read and written), and record
    them in profiles/traffic.json with the digest of the kernel sources."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path, newline="") as f:
            for rec in csv.DictReader(f):
                if rec.get("Counter_Name") != counter:
                    continue
                vals.setdefault(rec["Kernel_Name"], []).append(float(rec["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(vals, needle):
        names = [n for n in vals if needle in n]
        if len(names) != 1:
            raise SystemExit(f"expected one kernel matching {needle!r}, found {names}")
        v = vals[names[0]]
        return names[0], sum(v) / len(v), len(v)

    kname, kf, nf = pick(fetch, "sample_stream_kernel")
    _, kw, nw = pick(write, "sample_stream_kernel")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    if any(COPY_KERNEL_NEEDLE in n for n in fetch):
        cname, cf, _ = pick(fetch, COPY_KERNEL_NEEDLE)
        _, cw, _ = pick(write, COPY_KERNEL_NEEDLE)
    else:
        # no copy kernel in these runs: the calibration of the c3 record
        ref = data["sample_batch@c3"]
        cname, cf, cw = ref["copy_kernel"], ref["copy_fetch_kib"], ref["copy_write_kib"]
    fscale = cf * 1024.0 / COPY_BYTES
    wscale = cw * 1024.0 / COPY_BYTES
    rec = {
        "kernel_name": kname,
        "fetch_kib_per_launch": kf, "write_kib_per_launch": kw, "dispatches": [nf, nw],
        "copy_kernel": cname, "copy_bytes_each_way": COPY_BYTES,
        "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": fscale, "write_scale": wscale,
        "fetch_bytes_per_launch": kf * 1024.0 / fscale,
        "write_bytes_per_launch": kw * 1024.0 / wscale,
        "bytes_per_launch": kf * 1024.0 / fscale + kw * 1024.0 / wscale,
        "sources_digest": kernel_sources_digest(),
        "command": command,
    }
    data[f"{kernel}@{workload}"] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def _oracle_rows(task):
    """One worker task of the CPU baseline: the oracle on a few rows."""
    import oracle
    logits, dtype, T, k, p, mp, uid, step, seed = task
    oracle.sample_batch(logits, dtype, T, k, p, uid, step, seed, min_p=mp)
    return len(uid)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_single_process(w, seconds: float) -> float:
    """The oracle in this process, one row after another, for about
    ``seconds``: rows per second on one core."""
    import oracle
    t0 = time.perf_counter()
    n = 0
    while True:
        b = n % w.B
        sl = lambda a: None if a is None else a[b:b + 1]
        oracle.sample_batch(w.logits[b:b + 1], w.dtype, sl(w.temperature), sl(w.top_k), sl(w.top_p),
                            w.uid[b:b + 1], w.step, w.seed, min_p=sl(w.min_p))
        n += 1
        if time.perf_counter() - t0 > seconds:
            break
    return n / (time.perf_counter() - t0)


def percentiles_us(vals_ms):
    import numpy as np
    v = np.asarray(vals_ms) * 1e3
    return {"mean": float(v.mean()), "median": float(np.median(v)), "p10": float(np.percentile(v, 10)),
            "p90": float(np.percentile(v, 90))}


def cpu_baseline(w, seconds: float):
    """The fp64 oracle, as it is, on the host's cores (at most 16 worker
    processes, spawned: they never touch the GPU): passes over the same
    batch at steps s, s+1, ... (only the random draw differs) until about
    ``seconds`` have passed; rows per second over the timed passes."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    per = 4

    def sl(a, b0):
        return None if a is None else a[b0:b0 + per]

    def tasks(step):
        return [(w.logits[b0:b0 + per], w.dtype, sl(w.temperature, b0), sl(w.top_k, b0),
                 sl(w.top_p, b0), sl(w.min_p, b0), w.uid[b0:b0 + per], step, w.seed)
                for b0 in range(0, w.B, per)]

    with ProcessPoolExecutor(cores, mp_context=multiprocessing.get_context("spawn")) as ex:
        list(ex.map(_oracle_rows, tasks(w.step)[:cores]))     # workers started and warm
        t0 = time.perf_counter()
        n = passes = 0
        while True:
            n += sum(ex.map(_oracle_rows, tasks(w.step + passes)))
            passes += 1
            if time.perf_counter() - t0 > seconds:
                break
        dt = time.perf_counter() - t0
    single = oracle_single_process(w, min(5.0, seconds / 2))
    return {"value": n / dt, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{passes} passes over the {w.B} rows of the same batch (steps s, s+1, ...), "
                      f"fp64 NumPy oracle, {cores} worker processes, {per} rows per task",
            "single_process_rows_per_s": single, "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--buffers", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also launch the plain copy kernel the byte counters are scaled by")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="record counter-measured bytes per launch in profiles/traffic.json")
    ap.add_argument("--traffic-command", default="",
                    help="with --write-traffic: the profiling command, stored with the figures")
    ap.add_argument("--workload", choices=("c3", "c3minp", "c2", "c4loop"), default="c3",
                    help="c3: the headline sampler step (default); c3minp: the same batch with "
                         "a per-request min_p; c2: B=256 V=128256 bf16, half greedy, half T=0.7 "
                         "top-p 0.9; c4loop: the overlapped decode loop (prepare, page "
                         "table, gather, sample, write) at B=512 V=152064 bf16")
    ap.add_argument("--traffic-workload", default="c3",
                    help="with --write-traffic: the workload the counters were taken on")
    args = ap.parse_args()

    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], "sample_batch", args.traffic_workload,
                      args.traffic_command)
        return

    if args.gpus != 1:
        print(f"bench.py: this sampler runs on one GPU; --gpus {args.gpus} is not supported "
              f"(rows are independent: shard the batch, one process per GPU)", file=sys.stderr)
        sys.exit(2)

    if args.workload == "c4loop":
        bench_c4_loop(args)
        return

    import numpy as np
    import torch

    import decode_step_token_amd as dst
    import workloads as wl

    if args.workload == "c2":
        eprint("bench: generating the B=256 V=128256 bf16 workload")
        w = wl.c2()
    else:
        eprint("bench: generating the B=256 V=151936 fp32 workload")
        w = wl.c3()
    minp = None
    if args.workload == "c3minp":
        w = wl.with_min_p(w, C3_MIN_P_VALUES, 8)
        minp = torch.from_numpy(w.min_p).to("cuda:0")
    B, V = w.B, w.V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    esize = 4 if w.dtype == "f32" else 2
    host_logits = torch.from_numpy(w.logits if w.dtype == "f32" else w.logits.view(np.int16))
    bufs = [host_logits.to(dev) for _ in range(args.buffers)]
    opt = lambda a: None if a is None else torch.from_numpy(a).to(dev)
    T = opt(w.temperature)
    k = opt(w.top_k)
    p = opt(w.top_p)
    uid = torch.from_numpy(w.uid).to(dev)
    pool = torch.from_numpy(w.pool.copy()).to(dev)
    rows = torch.from_numpy(w.rows).to(dev)
    cols0 = torch.from_numpy(w.cols).to(dev)
    tokens = torch.empty(B, dtype=torch.int32, device=dev)
    host_ring = [torch.empty(B, dtype=torch.int32).pin_memory() for _ in range(2)]
    sampler = dst.Sampler(0, B, V, w.dtype, w.seed)
    stream = torch.cuda.current_stream()

    def step(s):
        sampler.sample(bufs[s % len(bufs)], temperature=T, top_k=k, top_p=p, uid=uid, step=s,
                       tokens_out=tokens, stream=stream, min_p=minp)
        return sampler.write(pool, rows, cols0, tokens, host_ring[s % 2], stream)

    eprint(f"bench: warmup {args.warmup} steps")
    prev = None
    for s in range(args.warmup):
        t = step(s)
        if prev is not None:
            sampler.wait(prev)
        prev = t
    if prev is not None:
        sampler.wait(prev)
    torch.cuda.synchronize()

    # timed region 1: whole steps (sample_batch + write_tokens with its host
    # copy); step s waits for the ticket of step s-1
    eprint(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    prev = None
    marks = []                      # host time at which each step's host copy is in
    for i in range(args.steps):
        t = step(args.warmup + i)
        if prev is not None:
            sampler.wait(prev)
            marks.append(time.perf_counter())
        prev = t
    sampler.wait(prev)
    marks.append(time.perf_counter())
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [(b_ - a_) * 1e3 for a_, b_ in zip([t0] + marks[:-1], marks)]

    # timed region 2: the sample_batch kernel alone, the same launches back to
    # back, bracketed by two HIP events on the launch stream (an event pair
    # around every launch would add its own packets to each launch); after
    # KERNEL_WARMUP untimed back-to-back launches, over at least KERNEL_MIN
    # launches, so that a short run still times the kernel in its steady state
    n_kernel = max(args.steps, KERNEL_MIN)
    for i in range(KERNEL_WARMUP):
        sampler.sample(bufs[i % len(bufs)], temperature=T, top_k=k, top_p=p, uid=uid,
                       step=args.warmup + args.steps + i, tokens_out=tokens, stream=stream,
                       min_p=minp)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(n_kernel):
        sampler.sample(bufs[i % len(bufs)], temperature=T, top_k=k, top_p=p, uid=uid,
                       step=args.warmup + args.steps + KERNEL_WARMUP + i, tokens_out=tokens, stream=stream,
                       min_p=minp)
    ev1.record(stream)
    torch.cuda.synchronize()
    kernel_ms_total = ev0.elapsed_time(ev1)
    # timed region 3 (spread only): one event after every launch, so launch i
    # spans the interval between events i and i + 1; each interval also holds
    # the event between two launches, so these read a few us above the
    # back-to-back average of region 2
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        sampler.sample(bufs[i % len(bufs)], temperature=T, top_k=k, top_p=p, uid=uid,
                       step=args.warmup + 2 * args.steps + i, tokens_out=tokens, stream=stream,
                       min_p=minp)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    launch_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    sampler.check()
    sampler.close()

    if args.calibrate_copy:
        eprint("bench: calibration copy (elementwise negation of one logits buffer)")
        dst_buf = torch.empty_like(bufs[0])
        for _ in range(3):
            torch.neg(bufs[0], out=dst_buf)
        torch.cuda.synchronize()
        del dst_buf

    ms_per_step = elapsed * 1e3 / args.steps
    avg_kernel_ms = kernel_ms_total / n_kernel
    alg_bytes = B * (V * esize + PARAM_BYTES_PER_ROW)
    achieved = alg_bytes / (avg_kernel_ms * 1e-3) / 1e9
    eprint(f"bench: {ms_per_step * 1e3:.1f} us/step, sample_batch kernel avg "
           f"{avg_kernel_ms * 1e3:.1f} us, {achieved:.0f} GB/s")

    traffic = load_traffic("sample_batch", args.workload) if args.workload in ("c3", "c2") else None
    cpu = None
    if not args.no_cpu_baseline:
        eprint(f"bench: timing the oracle on the host for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": METRIC if args.workload != "c2" else METRIC.replace("V=151936", f"V={V} bf16"),
        "value": B / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": ("c3: B=256 V=151936 fp32 2*Gumbel+rank-4 logits, per-request "
                                "T~U[0.3,1.5], top_k in {1,20,50,off}, top_p in {1,0.95,0.8}; "
                                "token pool [256,4096]"
                                + ("; min_p in {0,0.02,0.05,0.1}" if minp is not None else ""))
                   if args.workload != "c2" else
                   "c2: B=256 V=128256 bf16 N(0,3) logits, even uids greedy, odd uids T=0.7 top-p 0.9",
                   "B": B, "V": V, "logits_dtype": w.dtype, "input_buffers": len(bufs),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "sample_batch", "kernel_avg_us": avg_kernel_ms * 1e3,
                     "kernel_launches_timed": n_kernel, "kernel_warmup_launches": KERNEL_WARMUP,
                     "alg_bytes_per_launch": alg_bytes,
                     "event_interval_us": percentiles_us(launch_ms)},
        "step_us": percentiles_us(step_ms),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


GATHER_BYTES_PER_ENTRY = 8 + 8 + 4 + 4     # row, position read; pool id read; id written
PAGE_BYTES_PER_POSITION = 4 + 4            # page start read (page size 1), table cell written


def bench_c4_loop(args):
    """The scheduler's overlapped decode loop on the c4 workload: per step
    sampler_prepare (host parameters -> one upload) -> write_page_table (the
    step's new KV page per request, page size 1) -> gather_tokens (input ids
    at device_len - 1) -> sample_batch -> write_tokens (pool at device_len,
    host copy); step s waits for step s-1's ticket after enqueuing step s.
    Logits of a few distinct steps are resident and used in rotation while
    the step counter advances.  Also times gather_tokens and
    write_page_table alone, for the decode batch and for prefill-sized
    inputs."""
    import numpy as np
    import torch

    import decode_step_token_amd as dst
    import workloads as wl

    nbuf = max(1, args.buffers)
    eprint(f"bench: generating the B=512 V=152064 bf16 decode-loop workload ({nbuf} steps of logits)")
    w = wl.c4(0)
    B, V = w.B, w.V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bufs = [torch.from_numpy(wl.c4_logits(i).view(np.int16)).to(dev) for i in range(nbuf)]
    # request-level parameters on the host, prepared every step
    hT, hk, hp, hu = (torch.from_numpy(a) for a in (w.temperature, w.top_k, w.top_p, w.uid))
    blocks = [torch.empty(dst._binding.PREP_BYTES_PER_REQUEST * B, dtype=torch.uint8, device=dev)
              for _ in range(2)]
    pool = torch.from_numpy(w.pool.copy()).to(dev)
    rows = torch.from_numpy(w.rows).to(dev)
    pos0 = w.meta["pos0"]
    total = args.warmup + args.steps
    if int(pos0.max()) + total > w.pool.shape[1]:
        raise SystemExit(f"bench.py: {total} steps run past the pool's {w.pool.shape[1]} columns")
    in_pos = [torch.from_numpy(pos0 + s - 1).to(dev) for s in range(total)]
    out_pos = [torch.from_numpy(pos0 + s).to(dev) for s in range(total)]
    # page table of the same shape as the pool, page size 1: each step gives
    # every request the page for position device_len - 1, taken from the
    # front of a device free list
    page_table = torch.full(tuple(w.pool.shape), -1, dtype=torch.int32, device=dev)
    free_list = torch.arange(B * w.pool.shape[1], dtype=torch.int32, device=dev)
    req_rows = w.rows.astype(np.int64)
    cached = [pos0 + s - 1 for s in range(total)]
    devlen = [pos0 + s for s in range(total)]
    ids = torch.empty(B, dtype=torch.int32, device=dev)
    tokens = torch.empty(B, dtype=torch.int32, device=dev)
    host_ring = [torch.empty(B, dtype=torch.int32).pin_memory() for _ in range(2)]
    sampler = dst.Sampler(0, B, V, "bf16", w.seed)
    stream = torch.cuda.current_stream()

    def step(s):
        prm = sampler.prepare(B, hT, hk, hp, hu, dev_block=blocks[s % 2], stream=stream)
        off = (s * B) % (free_list.numel() - B)
        sampler.write_page_table(page_table, req_rows, cached[s], devlen[s],
                                 free_list[off:off + B], 1, stream)
        sampler.gather(pool, rows, in_pos[s], ids_out=ids, stream=stream)
        sampler.sample(bufs[s % nbuf], step=s, tokens_out=tokens, stream=stream, **prm)
        return sampler.write(pool, rows, out_pos[s], tokens, host_ring[s % 2], stream)

    def loop(first, count):
        prev = None
        for s in range(first, first + count):
            t = step(s)
            if prev is not None:
                sampler.wait(prev)
            prev = t
        if prev is not None:
            sampler.wait(prev)

    eprint(f"bench: warmup {args.warmup} steps")
    loop(0, args.warmup)
    torch.cuda.synchronize()
    eprint(f"bench: timing {args.steps} loop steps")
    t0 = time.perf_counter()
    loop(args.warmup, args.steps)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    def queued(launch, reps):
        """Mean time of `reps` launches run back to back: the stream is held
        in a spin kernel while they are enqueued."""
        for _ in range(2):
            launch()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(max(reps, 16) * 40e3))
        ev0.record(stream)
        for _ in range(reps):
            launch()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / reps

    def rate(n, nbytes, us):
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"entries": n, "avg_us": us, "achieved_GBs": gbs, "frac": gbs / PEAK_HBM_GBS}

    # host cost of one prepare call (staging, clamps and the enqueued upload)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        sampler.prepare(B, hT, hk, hp, hu, dev_block=blocks[i % 2], stream=stream)
    prep_us = (time.perf_counter() - t1) * 1e6 / args.steps
    torch.cuda.synchronize()

    # prefill-sized inputs: every request of the batch runs 1024 positions of
    # its row (spans of neighbouring columns)
    span = 1024
    pr = torch.arange(B, device=dev, dtype=torch.int64).repeat_interleave(span)
    pc = torch.arange(span, device=dev, dtype=torch.int64).repeat(B)
    out_ids = torch.empty(B * span, dtype=torch.int32, device=dev)
    g_decode = rate(B, B * GATHER_BYTES_PER_ENTRY,
                    queued(lambda: sampler.gather(pool, rows, in_pos[0], ids_out=ids, stream=stream),
                           args.steps))
    g_prefill = rate(B * span, B * span * GATHER_BYTES_PER_ENTRY,
                     queued(lambda: sampler.gather(pool, pr, pc, ids_out=out_ids, stream=stream),
                            args.steps))
    # the page-table write keeps its host records in 8 staging buffers that a
    # later call reuses only after the kernel ran, so at most 8 are queued
    zeros = np.zeros(B, dtype=np.int64)
    p_decode = rate(B, B * PAGE_BYTES_PER_POSITION,
                    queued(lambda: sampler.write_page_table(page_table, req_rows, cached[0],
                                                            devlen[0], free_list[:B], 1, stream), 8))
    p_prefill = rate(B * span, B * span * PAGE_BYTES_PER_POSITION,
                     queued(lambda: sampler.write_page_table(page_table, req_rows, zeros,
                                                             zeros + span, free_list[:B * span], 1,
                                                             stream), 8))
    sampler.check()
    sampler.close()
    eprint(f"bench: {ms_per_step * 1e3:.1f} us/loop step; gather decode {g_decode['avg_us']:.2f} us, "
           f"prefill {g_prefill['avg_us']:.2f} us; page table decode {p_decode['avg_us']:.2f} us, "
           f"prefill {p_prefill['avg_us']:.2f} us")
    out = {
        "metric": "decode-loop steps: sampled rows/sec at B=512, V=152064 "
                  "(prepare + page table + gather + sample + write)",
        "value": B / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c4 decode loop: B=512 V=152064 bf16 N(0,2.5) logits, c3 parameter "
                               "mix, token pool and page table [512,4096], per-request positions "
                               "from U[1,2048], page size 1; prepare -> page table -> gather -> "
                               "sample -> write, step s waits for step s-1's host copy",
                   "B": B, "V": V, "logits_dtype": "bf16", "input_buffers": nbuf,
                   "parallelism": "single GPU"},
        "prepare_host_us": prep_us,
        "gather_tokens": {"bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
                          "bytes_per_entry": GATHER_BYTES_PER_ENTRY,
                          "decode": g_decode, "prefill": g_prefill},
        "write_page_table": {"bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
                             "bytes_per_position": PAGE_BYTES_PER_POSITION,
                             "decode": p_decode, "prefill": p_prefill},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
