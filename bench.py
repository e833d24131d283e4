#!/usr/bin/env python3
"""Benchmark of the HiSparse decode-step swap-in path on one MI355X.

A step is one decode step of the whole path for every layer of the workload:
the forward's KV write into the hot buffer, the fused swap-in resolver
(resident / fast path / hit detection / LRU reorder / victims / plan / miss
copy from pinned host memory), the skip layers' plan replay, and the eager
backup.  Inputs (top-k rows, new KV rows) are generated and placed in HBM
before timing; host pools live in pinned host memory, as the method intends.

Prints one JSON line.  `value` = top-k entries resolved per second over the
timed steps (all layers and verify rows), wall clock between two
synchronisations; the median of --runs repetitions of the whole decode, each
after re-admitting every request, so each repeats the first exactly (one more
repetition goes first and is discarded, to warm up).  The
resolver's launch durations come from HIP events recorded in the timed runs,
spread over them so that each step's launches are timed in exactly one run
(a timed launch costs its step about 7 us of event overhead).  `roofline` describes the swap-in kernel: its miss copy is
bound by the host link (PCIe 5.0 x16 between the host and the MI355X), so
achieved = miss bytes per launch / mean launch time, against the link's
published per-direction rate; the link rate this machine measures is
reported beside it, both for a 1 GiB pinned host -> HBM DMA copy and for a
kernel streaming contiguous pinned rows with 16-byte loads (the swap-in's own
copy loop), and frac_of_measured_link is taken against the larger.  The skip layers' plan replay
and the eager backup get the same per-launch figures (rows moved x row bytes
/ mean launch time), from events on the stream each runs on in one more run
of the decode after the timed ones.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PCIE5_X16_GBPS = 64.0          # published per-direction rate of the MI355X host link
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measure_link(dev, nbytes=1 << 30, to_host=False):
    """Pinned host -> HBM (or HBM -> pinned host with to_host): one DMA copy of
    nbytes of hipHostMalloc memory, best of 3."""
    import torch
    from decode_memory_tiering_amd.hisparse import hisparse_host_alloc, hisparse_host_free, host_array
    p = hisparse_host_alloc(nbytes)
    try:
        h = torch.from_numpy(host_array(p, (nbytes,)))
        h.fill_(1)
        d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        d.copy_(h, non_blocking=True)
        torch.cuda.synchronize(dev)
        best = 0.0
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if to_host:
                h.copy_(d, non_blocking=True)
            else:
                d.copy_(h, non_blocking=True)
            e1.record()
            torch.cuda.synchronize(dev)
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        del d
        return best
    finally:
        hisparse_host_free(p)


def measure_zero_copy(dev, R=128, rows=4096, rb=1152, grids=(256, 512, 1024)):
    """Pinned host -> HBM through a kernel: the library's replay kernel with a
    plan that names every host row of every request in order, so it streams
    R * rows * rb contiguous bytes of pinned memory with 16-byte loads (the
    swap-in's own copy loop).  Best of a few grid sizes; returns (GB/s, grid)."""
    import torch
    from decode_memory_tiering_amd.hisparse import HiSparseCache, Plan
    best = (0.0, None)
    ramp = torch.arange(rows, dtype=torch.int32, device=dev).expand(R, rows).contiguous()
    plan = Plan(ramp, ramp, torch.full((R,), rows, dtype=torch.int32, device=dev))
    for grid in grids:
        c = HiSparseCache(num_layers=2, anchor_of=(0, 0), R=R, B=rows, K=rows, rb=rb, max_seq=rows,
                          device=dev, replay_grid=grid)
        try:
            c.host_np[1].fill(1)
            c.replay_plan(1, plan)
            torch.cuda.synchronize(dev)
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                c.replay_plan(1, plan)
                e1.record()
                torch.cuda.synchronize(dev)
                gbps = R * rows * rb / (e0.elapsed_time(e1) * 1e-3) / 1e9
                if gbps > best[0]:
                    best = (gbps, grid)
            if c.get_error():
                raise RuntimeError("zero-copy measurement: device error word set")
        finally:
            c.close()
    return best


def counter_bytes(workload):
    """(fetched, written) bytes per swap-in launch from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain
    copy), or None when there is none for this workload or the kernel source
    changed since the counters were taken.  Fetched bytes are the host-link
    reads of the miss rows plus the HBM metadata reads."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"swap_in_kernel_{workload}_counters.md")
    src = os.path.join(ROOT, "decode_memory_tiering_amd", "csrc", "hisparse.hip")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "rocprofv3", "`")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("src_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    try:
        return float(kv["fetch_bytes_per_launch"]), float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def counter_traffic(workload):
    """Fetched + written bytes per swap-in launch (see counter_bytes), or None."""
    fw = counter_bytes(workload)
    return None if fw is None else fw[0] + fw[1]


def tier_shares(wl, topk_all, steps, misses, block_table=None):
    """How the valid top-k entries of the given steps were served: resident
    (request or page), fast path (L <= B), newest token's own row, hot-buffer
    hit, miss.  Misses come from the run's plan counts; the other tiers follow
    from the inputs alone.  Also the hot-buffer hit rate, hits / (hits +
    misses), over the entries that reached the hot lookup."""
    from decode_memory_tiering_amd import workload as W
    res = W.resident_mask(wl).astype(bool)
    n = dict(resident=0, fast_path=0, newest=0, hit=0, miss=int(misses))
    lookup = 0
    for k in steps:
        L = W.seq_lens_at(wl, k).astype(np.int64)
        for v in topk_all[k].values():            # [S][R][K]
            for s in range(v.shape[0]):
                x = v[s].astype(np.int64)
                valid = x >= 0
                if block_table is not None:
                    P = wl.page_size
                    page = np.where(valid, x // P, 0)
                    inside = page < block_table.shape[1]
                    phys = np.where(inside, np.take_along_axis(block_table, np.minimum(page, block_table.shape[1] - 1),
                                                               1), -1)
                    is_res = valid & (phys >= 0)
                else:
                    is_res = valid & res[:, None]
                fast = valid & ~is_res & (L <= wl.B)[:, None]
                newest = valid & ~is_res & ~fast & (x == (L - 1)[:, None])
                n["resident"] += int(is_res.sum())
                n["fast_path"] += int(fast.sum())
                n["newest"] += int(newest.sum())
                lookup += int((valid & ~is_res & ~fast & ~newest).sum())
    n["hit"] = lookup - n["miss"]
    total = sum(n.values())
    return dict(entries=n, shares={k: v / total for k, v in n.items()},
                hot_hit_rate=(n["hit"] / lookup) if lookup else None)


def cpu_baseline(wl, steps, warmup, host_pools, topk_all, newkv_all, budget_s=10.0, max_threads=16):
    """The oracle, as it stands, on the same inputs and the same timed steps
    as the GPU (steps [warmup, steps) of the decode, the warmup steps run
    untimed): the decode, re-admitted between repetitions, is repeated until
    about budget_s of oracle time on one thread; then the same again with the
    requests split over the host's cores, one share per thread (requests are
    independent and the oracle keeps no global state, so the shares run side
    by side).  The oracle's hot buffers are written once beforehand, so no
    timed step pays for first-touch page faults."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle.runner import OracleRun
    o = OracleRun(wl, steps, host_pools=host_pools)
    for h in o.orc.hot:
        h.fill(0)
    per_step = [sum(int(np.count_nonzero(v >= 0)) for v in topk_all[k].values()) for k in range(steps)]

    def sweep(call):
        t_run, entries, done, reps = 0.0, 0, 0, 0
        while t_run <= budget_s and reps < 1000:
            o.readmit()
            reps += 1
            for k in range(warmup):
                call(k)
            for k in range(warmup, steps):
                t0 = time.perf_counter()
                call(k)
                t_run += time.perf_counter() - t0
                entries += per_step[k]
                done += 1
                if t_run > budget_s:
                    break
        return t_run, entries, done, reps

    t1, e1, done, reps = sweep(lambda k: o.step(k, topk_all[k], newkv_all[k]))
    threads = max(1, min(len(os.sched_getaffinity(0)), max_threads, wl.R))
    shares = [c for c in np.array_split(np.arange(wl.R, dtype=np.int32), threads) if c.size]
    with ThreadPoolExecutor(len(shares)) as pool:
        def parallel(k):
            list(pool.map(lambda req: o.step(k, topk_all[k], newkv_all[k], req), shares))
        tn, en, done_n, _ = sweep(parallel) if threads > 1 else (t1, e1, done, reps)
    what = (f"{done} timed decode steps (steps {warmup}..{steps - 1} of the same decode as the GPU run, "
            f"{reps} repetition(s), re-admitted in between, warmup steps untimed), all {wl.R} requests "
            f"and {wl.num_layers} layer(s)")
    return dict(value=e1 / t1, unit="top-k entries resolved/s", cores=1, kind="oracle",
                sample=f"{what}, single thread, oracle time {t1:.2f}s",
                threads=dict(value=en / tn, cores=len(shares),
                             sample=f"{done_n} timed decode steps, requests split over {len(shares)} "
                                    f"threads, oracle wall time {tn:.2f}s"))


def measure_page_copy(dev, W, args):
    """Spill (resident page -> host page) and host import (staging page ->
    host page, half mirrored to resident pages) on the paged decode's shape:
    64-token pages of 1152-byte rows, 4096 pages per call."""
    import torch
    from decode_memory_tiering_amd.runner import GpuRun
    wl = W.WORKLOADS["paged_decode"]
    g = GpuRun(wl, 2, fill=False)
    P, rb, n = wl.page_size, wl.rb, 4096
    rng = np.random.default_rng(0)
    max_pages = g.block_table_np.shape[1]
    n_res = g.res_cache[0].shape[0] // P
    pick = rng.choice(wl.R * max_pages, size=n, replace=False)
    spill = np.stack([rng.choice(n_res, n, replace=False), pick // max_pages, pick % max_pages,
                      -np.ones(n, np.int64)], 1).astype(np.int32)
    stg = torch.randint(0, 255, (n * P, rb), dtype=torch.uint8, device=dev)
    mirror = np.where(np.arange(n) % 2 == 0, rng.choice(n_res, n, replace=False), -1)
    imp = np.stack([np.arange(n), pick // max_pages, pick % max_pages, mirror], 1).astype(np.int32)
    spill_d, imp_d = torch.from_numpy(spill).to(dev), torch.from_numpy(imp).to(dev)
    out = {}
    for name, fn, nbytes in (("spill", lambda: g.cache.spill(0, g.res_cache[0], P, spill_d), n * P * rb),
                             ("import", lambda: g.cache.import_pages(0, stg, P, g.res_cache[0], imp_d), n * P * rb)):
        fn()
        torch.cuda.synchronize(dev)
        times = []
        for _ in range(max(args.steps, 3)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize(dev)
            times.append(e0.elapsed_time(e1) * 1e-3)
        t = float(np.mean(times))
        out[name] = dict(pages=n, bytes_to_host=nbytes, mean_us=t * 1e6, gbps=nbytes / t / 1e9)
    err = g.cache.get_error()
    g.close()
    if err:
        log(f"[bench] device error word {err:#x}")
        sys.exit(1)
    d2h = None if args.no_link else measure_link(dev, to_host=True)
    print(json.dumps({"metric": "page transfer GB/s (device -> pinned host)", "value": out["spill"]["gbps"],
                      "measured_d2h_link_gbps": d2h,
                      "unit": "GB/s", "higher_is_better": True, "n_gpus": 1, "steps": max(args.steps, 3),
                      "config": {"workload": "paged_decode pages", "page_size": P, "row_bytes": rb},
                      "spill": out["spill"], "import": out["import"],
                      "peak": PCIE5_X16_GBPS}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--runs", type=int, default=5,
                    help="repetitions of the whole timed decode (re-admitted in between); the median is reported")
    ap.add_argument("--workload", default="fastpath_mix")
    ap.add_argument("--block-size", type=int, default=0)
    ap.add_argument("--replay-grid", type=int, default=0)
    ap.add_argument("--host-flags", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fuse-backup", action="store_true",
                    help="anchor layers' eager backup as a launch of its own (A/B)")
    ap.add_argument("--no-link", action="store_true")
    ap.add_argument("--layer-compute-mib", type=int, default=0,
                    help="stand-in for each layer's other compute: a device copy of this many MiB on the "
                         "main stream after every layer (the IndexShare overlap case uses 2048)")
    ap.add_argument("--measure", default="step", choices=["step", "page_copy"],
                    help="page_copy: time spill and host import of paged_decode-shaped pages instead of decode steps")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the swap-in path is per-GPU, "
              "and sharding by request needs no exchange between GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_memory_tiering_amd import workload as W
    from decode_memory_tiering_amd.hisparse import load_library
    from decode_memory_tiering_amd.runner import GpuRun, draw_topk, new_kv_all_layers

    load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize(dev)
        print(json.dumps({"calibration_copy_bytes": n, "launches": 5}), flush=True)
        return
    if args.measure == "page_copy":
        measure_page_copy(dev, W, args)
        return
    wl = W.WORKLOADS[args.workload]
    total = args.warmup + args.steps

    t_setup = time.time()
    g = GpuRun(wl, total, block_size=args.block_size, replay_grid=args.replay_grid, host_flags=args.host_flags,
               fuse_backup=not args.no_fuse_backup)
    host_copy = None if args.no_cpu_baseline else [np.array(a, copy=True) for a in g.cache.host_np]
    streams = {a: W.TopkStream(wl, a) for a in wl.anchors}
    topk_all = [draw_topk(wl, streams, k) for k in range(total)]
    topk_dev = [{a: torch.from_numpy(v).to(dev) for a, v in t.items()} for t in topk_all]
    newkv_dev = [new_kv_all_layers(wl, k, dev) for k in range(total)]
    seq_dev = [g.seq_lens(k) for k in range(total)]
    # every step records into its own plan count (pos/slot rows are shared), so
    # nothing but the path runs inside the timed steps
    from decode_memory_tiering_amd.hisparse import Plan
    shared = {a: [Plan.empty(wl.R, wl.K, dev) for _ in range(wl.spec)] for a in wl.anchors}
    step_plans = [{a: [Plan(p.pos, p.slot, torch.zeros(wl.R, dtype=torch.int32, device=dev))
                       for p in shared[a]] for a in wl.anchors} for _ in range(total)]
    torch.cuda.synchronize(dev)
    log(f"[bench] {wl.name}: setup {time.time() - t_setup:.1f}s")

    between = None
    if args.layer_compute_mib:
        n = args.layer_compute_mib << 20
        csrc = torch.ones(n, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)

        def between(_l):
            cdst.copy_(csrc)

    # Launch events, each pair recorded on the stream its launch goes to.  A
    # timed pair costs the step about 7 us on C2 (the event's barrier keeps
    # the next launch from overlapping the previous one's tail), so the timed
    # runs share the work: run i records the resolver's launches of the
    # steps s with (s - warmup) % runs == i, and over all runs every step's
    # launches are recorded exactly once.  One more run after them, outside
    # the reported value, records every replay and backup launch.  Every
    # event is created before the first timed step.
    import inspect
    kinds = {"swap_in": "swap_in", "store_swap_in": "swap_in", "store_swap_in_backup": "swap_in",
             "swap_in_paged": "swap_in", "store_swap_in_paged_backup": "swap_in",
             "replay_plan": "replay", "backup": "backup"}
    per_step = {"swap_in": len(wl.anchors) * wl.spec, "replay": len(wl.skip_layers) * wl.spec,
                "backup": wl.num_layers}
    n_events = 2 * args.steps * (per_step["swap_in"] + sum(per_step.values()))
    pool = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    ev = {k: [] for k in per_step}      # the extra run's launches, by kind
    ev_timed = []                       # the timed runs' resolver launches
    recording = set()
    sink = {"timed": False}
    origs = {name: getattr(g.cache, name) for name in kinds}

    def timed(name, fn):
        kind = kinds[name]
        pos = list(inspect.signature(fn).parameters).index("stream")

        def call(*a, **kw):
            if kind not in recording:
                return fn(*a, **kw)
            stream = kw.get("stream") or (a[pos] if len(a) > pos else None) or torch.cuda.current_stream(dev)
            e0, e1 = pool.pop(), pool.pop()
            e0.record(stream)
            fn(*a, **kw)
            e1.record(stream)
            (ev_timed if sink["timed"] else ev[kind]).append((e0, e1))
        return call

    def run(k):
        g.step(topk_dev[k], newkv_dev[k], seq_dev[k], plans=step_plans[k], between_layers=between)

    # every run re-admits all requests and repeats the same decode exactly:
    # W untimed warmup steps, then exactly K timed steps between two
    # synchronisations.  One whole run goes first, discarded, to warm the GPU
    # and the host pool's first touches.
    for k in range(total):
        run(k)
    torch.cuda.synchronize(dev)
    walls = []
    for name in kinds:
        setattr(g.cache, name, timed(name, origs[name]))
    try:
        for i in range(args.runs + 1):
            detail = i == args.runs
            g.readmit()
            recording.clear()
            for k in range(args.warmup):
                run(k)
            torch.cuda.synchronize(dev)
            sink["timed"] = not detail
            if detail:
                recording.update(per_step)
            t0 = time.perf_counter()
            for k in range(args.warmup, total):
                if not detail:
                    recording.clear()
                    if (k - args.warmup) % args.runs == i:
                        recording.add("swap_in")
                run(k)
            torch.cuda.synchronize(dev)
            if not detail:
                walls.append(time.perf_counter() - t0)
                log(f"[bench] run {i}: {walls[-1] * 1e3:.2f} ms")
    finally:
        for name in kinds:
            setattr(g.cache, name, origs[name])
    wall = float(np.median(walls))

    entries = sum(int(np.count_nonzero(v >= 0)) for k in range(args.warmup, total) for v in topk_all[k].values())
    # plan counts hold the last run's misses; every run has the same ones
    misses = sum(int(p.count.sum().item()) for k in range(args.warmup, total)
                 for a in wl.anchors for p in step_plans[k][a])
    n_swap = len(ev_timed)              # every resolver launch of one decode, once
    assert n_swap == per_step["swap_in"] * args.steps, (n_swap, per_step["swap_in"] * args.steps)
    launch_ms = [a.elapsed_time(b) for a, b in ev_timed]
    mean_launch_s = float(np.mean(launch_ms)) * 1e-3
    miss_bytes_per_launch = misses * wl.rb / n_swap
    achieved = miss_bytes_per_launch / mean_launch_s / 1e9
    # resolve-pass metadata bytes per launch (top-k read + slot write per entry;
    # slot map read, LRU read + write per slow row; slot map write + plan pair per miss)
    slow_rows = 0
    res = W.resident_mask(wl)
    for k in range(args.warmup, total):
        L = W.seq_lens_at(wl, k)
        slow_rows += int(np.count_nonzero((L > wl.B) & (res == 0))) * len(wl.anchors) * wl.spec
    meta_bytes = entries * 8 + slow_rows * 12 * wl.B + misses * 12 + slow_rows * 4

    def kind_stats(kind, rows_per_run):
        """Host-link rate of one launch kind: rows moved x row bytes / mean launch time."""
        if not ev[kind]:
            return None
        ms = [a.elapsed_time(b) for a, b in ev[kind]]
        n = len(ev[kind])
        t = float(np.mean(ms)) * 1e-3
        return dict(launches=n, mean_launch_us=t * 1e6, rows_per_launch=rows_per_run / n,
                    gbps=rows_per_run * wl.rb / n / t / 1e9)

    # every skip layer replays each verify row's plan of its anchor
    replay_rows = sum(int(p.count.sum().item()) for k in range(args.warmup, total)
                      for x in wl.skip_layers for p in step_plans[k][wl.anchor_of[x]])
    # a separate backup launch copies one row per non-resident request (anchor
    # layers' backups ride in their swap-in launch and have no launch of their own)
    backup_rows = len(ev["backup"]) * int(np.count_nonzero(res == 0))
    err = g.cache.get_error()
    if err:
        log(f"[bench] device error word {err:#x}")
        sys.exit(1)

    link = None if args.no_link else measure_link(dev)
    zc, zc_grid = (None, None) if args.no_link else measure_zero_copy(dev)
    best_link = max(link, zc) if link else None
    cpu = None
    if not args.no_cpu_baseline:
        newkv_np = [t.cpu().numpy() for t in newkv_dev]
        g.close()
        cpu = cpu_baseline(wl, total, args.warmup, host_copy, topk_all, newkv_np)
    else:
        g.close()

    rec = {
        "metric": "top-k rows resolved/s per decode step; miss-copy GB/s as % of host-link peak",
        "value": entries / wall,
        "unit": "top-k entries resolved/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic (seeded top-k mixture, bf16/fp8 N(0,1) KV rows in pinned host memory)",
        "config": {
            "workload": wl.name, "requests": wl.R, "layers": wl.num_layers, "anchors": len(wl.anchors),
            "top_k": wl.K, "device_buffer_size": wl.B, "row_bytes": wl.rb, "verify_rows": wl.spec,
            "resident_requests": wl.n_resident, "first_seq_len": list(wl.seq_first),
            "page_size": wl.page_size or None, "resident_page_frac": wl.resident_page_frac if wl.page_size else None,
            "parallelism": "single GPU (requests are independent)",
            "prefetch": bool(g.prefetch) if wl.skip_layers else None,
            "layer_compute_mib": args.layer_compute_mib,
            "fused_launches": "store+swap-in+backup" if g.fuse_backup else
                              ("store+swap-in" if not wl.page_size else "none"),
        },
        "roofline": {
            "kernel": "swap_in_kernel",
            "bound": "host_link",
            "achieved": achieved,
            "peak": PCIE5_X16_GBPS,
            "unit": "GB/s",
            "frac": achieved / PCIE5_X16_GBPS,
            "traffic": counter_traffic(wl.name),
            # the counters' fetched bytes over the live mean launch time: the
            # miss copy's read rate as the fabric saw it (metadata included)
            "counter_fetch_gbps": (counter_bytes(wl.name)[0] / mean_launch_s / 1e9)
                                  if counter_bytes(wl.name) else None,
            "launches": n_swap,
            "mean_launch_us": mean_launch_s * 1e6,
            "miss_bytes_per_launch": miss_bytes_per_launch,
            "measured_link_gbps": link,
            "zero_copy_link_gbps": zc,
            "zero_copy_grid": zc_grid,
            "frac_of_measured_link": (achieved / best_link) if best_link else None,
            "resolve_hbm_gbps": meta_bytes / n_swap / mean_launch_s / 1e9,
            "resolve_hbm_frac": meta_bytes / n_swap / mean_launch_s / 1e9 / HBM_PEAK_GBPS,
        },
        "runs": {"n": args.runs, "ms_per_step": [w / args.steps * 1e3 for w in walls],
                 "value_min": entries / max(walls), "value_max": entries / min(walls)},
        "replay": kind_stats("replay", replay_rows),
        "backup": kind_stats("backup", backup_rows),
        "tiers": tier_shares(wl, topk_all, range(args.warmup, total), misses,
                             g.block_table_np if wl.page_size else None),
        "misses_per_step": misses / args.steps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
