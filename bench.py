#!/usr/bin/env python3
"""Benchmark of the HiSparse decode-step swap-in path on one MI355X.

A step is one decode step of the whole path for every layer of the workload:
the forward's KV write into the hot buffer, the fused swap-in resolver
(resident / fast path / hit detection / LRU reorder / victims / plan / miss
copy from pinned host memory), the skip layers' plan replay, and the eager
backup.  Inputs (top-k rows, new KV rows) are generated and placed in HBM
before timing; host pools live in pinned host memory, as the method intends.

The default workload is the DSV3.2-shaped decode: 4 layers with their own
host pools, 128 requests (32 fully resident), 40000-token sequences, top_k
2048, a 6144-slot buffer, 1152-byte bf16 rows, eager backup every step.
Prints one JSON line.  `value` = top-k entries resolved per second over the
timed steps (all layers and verify rows), wall clock between two
synchronisations; the median of --runs repetitions of the whole decode, each
after re-admitting every request, so each repeats the first exactly (one more
repetition goes first and is discarded, to warm up).  `all_steps` gives the
same rate over every step of the workload's whole decode from admission (the
first steps find an empty buffer: all misses), and per-step times.  The
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


def profile_fields(name):
    """key: value lines of a committed profiles/ summary, or {} if absent."""
    path = os.path.join(ROOT, "profiles", name)
    kv = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith(("#", "rocprofv3", "`", "|", " ")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def _src_sha256():
    import hashlib
    src = os.path.join(ROOT, "decode_memory_tiering_amd", "csrc", "hisparse.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()


def window_matches(kv, workload, steps, warmup, runs):
    """A committed summary applies only to the exact decode window it was
    taken on (workload, timed steps, warm-up steps, timed runs) and to the
    kernel source it was taken with."""
    want = dict(workload=workload, steps=str(steps), warmup=str(warmup), runs=str(runs), src_sha256=_src_sha256())
    return bool(kv) and all(kv.get(k) == v for k, v in want.items())


def counter_bytes(workload, steps, warmup, runs):
    """(fetched, written) bytes per swap-in launch of the timed window, from
    the committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each
    scaled by what it reads for a plain copy of known size); None unless the
    summary was taken on exactly this window and this kernel source.  Fetched
    bytes include the miss rows read over the host link and the HBM metadata
    reads; written bytes the hot rows and metadata written to HBM and the
    fused backup's rows written to the host pool."""
    kv = profile_fields(f"swap_in_kernel_{workload}_counters.md")
    if not window_matches(kv, workload, steps, warmup, runs):
        return None
    try:
        return float(kv["fetch_bytes_per_launch"]), float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def trace_mean_us(workload, steps, warmup, runs):
    """Mean duration of the timed window's swap-in launches in the committed
    rocprofv3 kernel trace, or None unless it was taken on exactly this
    window and kernel source."""
    kv = profile_fields(f"swap_in_kernel_{workload}_kernel_trace.md")
    if not window_matches(kv, workload, steps, warmup, runs):
        return None
    try:
        return float(kv["swap_in_timed_mean_us"])
    except (KeyError, ValueError):
        return None


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


def cpu_baseline(wl, steps, warmup, host_pools, topk_all, newkv_all, budget_s=10.0, max_threads=16,
                 pool_steps=None, rows_per_rep=None):
    """The oracle, as it stands, on the same inputs and the same timed steps
    as the GPU (steps [warmup, steps) of the decode, the warm-up steps run
    untimed), driven from C (oracle/oracle_timing.c: no Python inside the
    timed loop): the decode, re-admitted before every repetition, is
    repeated until about budget_s of timed oracle work on one thread; then
    the same with the requests split into one share per host core, a POSIX
    thread each (requests are independent and the oracle keeps no global
    state, so the shares run side by side, each through every step).  The
    oracle's hot buffers are written once beforehand, so no timed step pays
    for first-touch page faults."""
    from oracle.runner import OracleRun
    from oracle.timing import DecodeTimer
    # host pools hold pool_steps steps' rows (the GPU run's sizing)
    o = OracleRun(wl, pool_steps or steps, host_pools=host_pools)
    for h in o.orc.hot:
        h.fill(0)
    assert all(h.shape == p.shape for h, p in zip(o.orc.host, host_pools)), "host pools sized for another run"
    timer = DecodeTimer(o, topk_all[:steps], newkv_all[:steps], first_timed=warmup)
    per_rep = sum(int(np.count_nonzero(v >= 0)) for k in range(warmup, steps) for v in topk_all[k].values())

    def sweep(threads):
        t_run, reps = 0.0, 0
        while t_run <= budget_s and reps < 10000:
            t_run += timer.run(threads)
            reps += 1
        return t_run, reps

    t1, reps1 = sweep(1)
    threads = max(1, min(len(os.sched_getaffinity(0)), max_threads, wl.R))
    tn, repsn = sweep(threads) if threads > 1 else (t1, reps1)
    what = (f"steps {warmup}..{steps - 1} of the same decode as the GPU run (warm-up steps untimed), all "
            f"{wl.R} requests and {wl.num_layers} layer(s), re-admitted before each repetition")
    # rows_per_rep: the rows a repetition copies (misses and replayed rows of
    # the timed steps, the same as the GPU's); the oracle copies them from the
    # pinned pool into its host mirror of the hot buffer
    copy = (lambda reps, t: rows_per_rep * wl.rb * reps / t / 1e9) if rows_per_rep is not None else None
    return dict(value=per_rep * reps1 / t1, unit="top-k entries resolved/s", cores=1, kind="oracle",
                copy_gbps=copy(reps1, t1) if copy else None,
                sample=f"{reps1} repetition(s) of {what}; single thread, timed oracle work {t1:.2f}s",
                threads=dict(value=per_rep * repsn / tn, cores=threads,
                             copy_gbps=copy(repsn, tn) if copy else None,
                             sample=f"{repsn} repetition(s), requests split into {threads} shares on "
                                    f"{threads} threads, timed wall {tn:.2f}s"))


def measure_page_copy(dev, W, args):
    """Spill (resident page -> host page) and host import (staging page ->
    host page, half mirrored to resident pages) on the paged decode's shape:
    64-token pages of 1152-byte rows, 4096 pages per call, by the copy kernel
    and by runtime copies (one hipMemcpyAsync per run of pages contiguous on
    both sides).  Two transfer lists: pages scattered over the pool (every page its
    own copy) and whole runs of 64 consecutive pages (64 copies per call).
    Then each spill form beside a 2 GiB device-to-device copy on another
    stream (a stand-in for a layer's other work): how much the spill slows
    that work, and the spill's own rate meanwhile."""
    import torch
    from decode_memory_tiering_amd.runner import GpuRun
    wl = W.WORKLOADS["paged_decode"]
    g = GpuRun(wl, 2, fill=False)
    P, rb, n = wl.page_size, wl.rb, 4096
    rng = np.random.default_rng(0)
    max_pages = g.block_table_np.shape[1]
    n_res = g.res_cache[0].shape[0] // P
    assert n_res >= n
    pick = rng.choice(wl.R * max_pages, size=n, replace=False)
    spill = np.stack([rng.choice(n_res, n, replace=False), pick // max_pages, pick % max_pages,
                      -np.ones(n, np.int64)], 1).astype(np.int32)
    stg = torch.randint(0, 255, (n * P, rb), dtype=torch.uint8, device=dev)
    mirror = np.where(np.arange(n) % 2 == 0, rng.choice(n_res, n, replace=False), -1)
    imp = np.stack([np.arange(n), pick // max_pages, pick % max_pages, mirror], 1).astype(np.int32)
    # runs: request q's host pages 0..63 from resident pages 64q..64q+63 (import: staging
    # likewise, no mirror), so every run of 64 transfers is contiguous on both sides
    q = np.arange(n)
    spill_runs = np.stack([q, q // 64, q % 64, -np.ones(n, np.int64)], 1).astype(np.int32)
    imp_runs = spill_runs.copy()
    lists = {"scattered": (spill, imp), "runs64": (spill_runs, imp_runs)}
    res0 = g.res_cache[0]

    def timeit(fn, reps):
        fn()
        torch.cuda.synchronize(dev)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize(dev)
            times.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.mean(times))

    out = {}
    reps = max(args.steps, 3)
    nbytes = n * P * rb
    for lname, (sp, im) in lists.items():
        sp_d, im_d = torch.from_numpy(sp).to(dev), torch.from_numpy(im).to(dev)
        forms = {
            "spill_kernel": lambda: g.cache.spill(0, res0, P, sp_d),
            "spill_dma": lambda: g.cache.spill_dma(0, res0, P, sp),
            "import_kernel": lambda: g.cache.import_pages(0, stg, P, res0, im_d),
            "import_dma": lambda: g.cache.import_pages_dma(0, stg, P, res0, im),
        }
        for fname, fn in forms.items():
            t0 = time.perf_counter()
            fn()
            host_us = (time.perf_counter() - t0) * 1e6          # the call's own (enqueue) time
            torch.cuda.synchronize(dev)
            t = timeit(fn, reps)
            out[f"{lname}/{fname}"] = dict(pages=n, bytes_to_host=nbytes, mean_us=t * 1e6,
                                           gbps=nbytes / t / 1e9, enqueue_us=host_us)
            log(f"[bench] {lname}/{fname}: {nbytes / t / 1e9:.1f} GB/s, enqueue {host_us:.0f} us")
    # beside a 2 GiB device copy on the main stream
    m = 2048 << 20
    csrc = torch.ones(m, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    side = torch.cuda.Stream(device=dev)
    t_alone = timeit(lambda: cdst.copy_(csrc), reps)
    overlap = {"compute_alone_us": t_alone * 1e6}
    for lname, (sp, _) in lists.items():
        sp_d = torch.from_numpy(sp).to(dev)
        for fname, fn in (("spill_kernel", lambda s: g.cache.spill(0, res0, P, sp_d, s)),
                          ("spill_dma", lambda s: g.cache.spill_dma(0, res0, P, sp, s))):
            c_ms, s_ms = [], []
            for _ in range(reps):
                torch.cuda.synchronize(dev)
                e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                main = torch.cuda.current_stream(dev)
                # the compute is enqueued first, so the spill's own enqueue
                # time on the host cannot delay it; both start together
                e[0].record(main)
                cdst.copy_(csrc)
                e[1].record(main)
                side.wait_event(e[0])
                e[2].record(side)
                fn(side)
                e[3].record(side)
                torch.cuda.synchronize(dev)
                c_ms.append(e[0].elapsed_time(e[1]))
                s_ms.append(e[2].elapsed_time(e[3]))
            tc, ts = float(np.mean(c_ms)) * 1e-3, float(np.mean(s_ms)) * 1e-3
            overlap[f"{lname}/{fname}"] = dict(compute_us=tc * 1e6, compute_slowdown=tc / t_alone,
                                               spill_us=ts * 1e6, spill_gbps=nbytes / ts / 1e9)
            log(f"[bench] beside 2 GiB copy, {lname}/{fname}: compute x{tc / t_alone:.3f}, "
                f"spill {nbytes / ts / 1e9:.1f} GB/s")
    err = g.cache.get_error()
    g.close()
    if err:
        log(f"[bench] device error word {err:#x}")
        sys.exit(1)
    d2h = None if args.no_link else measure_link(dev, to_host=True)
    print(json.dumps({"metric": "page transfer GB/s (device -> pinned host)",
                      "value": out["scattered/spill_kernel"]["gbps"],
                      "measured_d2h_link_gbps": d2h,
                      "unit": "GB/s", "higher_is_better": True, "n_gpus": 1, "steps": reps,
                      "config": {"workload": "paged_decode pages", "page_size": P, "row_bytes": rb, "pages": n},
                      "forms": out, "beside_2gib_copy": overlap,
                      "peak": PCIE5_X16_GBPS}), flush=True)


def algorithmic_bytes(wl, topk_all, steps, misses, fused_rows):
    """Bytes the swap-in launches of the given steps must move, by where they
    go: host-link reads (miss rows), host-link writes (rows the fused eager
    backup writes), HBM reads (top-k rows, slot maps and LRU lists of slow
    rows, new KV rows of a fused store) and HBM writes (miss rows landing in
    the hot buffer, slot ids, LRU lists, slot-map updates, plan pairs and
    counts, fused new rows)."""
    from decode_memory_tiering_amd import workload as W
    res = W.resident_mask(wl)
    entries = slow = 0
    for k in steps:
        for v in topk_all[k].values():
            entries += int(np.count_nonzero(v >= 0))
        L = W.seq_lens_at(wl, k)
        slow += int(np.count_nonzero((L > wl.B) & (res == 0))) * len(wl.anchors) * wl.spec
    rb, B = wl.rb, wl.B
    return dict(
        host_link_read=misses * rb,
        host_link_write=fused_rows * rb,
        hbm_read=entries * 4 + slow * 8 * B + fused_rows * rb,
        hbm_write=misses * rb + entries * 4 + slow * (4 * B + 4) + misses * 12 + fused_rows * rb,
        entries=entries, slow_rows=slow)


def measure_indexshare_overlap(dev, W, args):
    """The IndexShare decode (one anchor + 3 skip layers replaying its miss
    plan) with a 2 GiB device copy after every layer standing in for that
    layer's other compute: the step time with the skip layers' replays
    pre-issued on the side stream against the same decode with every replay
    inline on the main stream, alternating, plus each replay launch's rate."""
    import torch
    from decode_memory_tiering_amd.hisparse import Plan
    from decode_memory_tiering_amd.runner import GpuRun, draw_topk, new_kv_all_layers
    wl = W.WORKLOADS["indexshare"]
    total = args.warmup + args.steps
    g = GpuRun(wl, total, prefetch=True)
    streams = {a: W.TopkStream(wl, a) for a in wl.anchors}
    topk_all = [draw_topk(wl, streams, k) for k in range(total)]
    topk_dev = [{a: torch.from_numpy(v).to(dev) for a, v in t.items()} for t in topk_all]
    newkv_dev = [new_kv_all_layers(wl, k, dev) for k in range(total)]
    seq_dev = [g.seq_lens(k) for k in range(total)]
    shared = {a: [Plan.empty(wl.R, wl.K, dev) for _ in range(wl.spec)] for a in wl.anchors}
    step_plans = [{a: [Plan(p.pos, p.slot, torch.zeros(wl.R, dtype=torch.int32, device=dev))
                       for p in shared[a]] for a in wl.anchors} for _ in range(total)]
    n = (args.layer_compute_mib or 2048) << 20
    csrc = torch.ones(n, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)

    def decode(prefetch, replay_events=None):
        g.prefetch = prefetch
        g.readmit()
        for k in range(args.warmup):
            g.step(topk_dev[k], newkv_dev[k], seq_dev[k], plans=step_plans[k], between_layers=lambda l: cdst.copy_(csrc))
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for k in range(args.warmup, total):
            g.step(topk_dev[k], newkv_dev[k], seq_dev[k], plans=step_plans[k], between_layers=lambda l: cdst.copy_(csrc))
        torch.cuda.synchronize(dev)
        return (time.perf_counter() - t0) / args.steps

    decode(True)
    times = {True: [], False: []}
    for _ in range(args.runs):
        for pf in (True, False):
            times[pf].append(decode(pf))
    # one more prefetched decode with an event pair around every replay launch
    orig = g.cache.replay_plan
    ev = []

    def timed_replay(skip, plan, req_idx=None, stream=None):
        s = stream or torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        orig(skip, plan, req_idx, s)
        e1.record(s)
        ev.append((e0, e1))
    g.cache.replay_plan = timed_replay
    try:
        decode(True)
    finally:
        g.cache.replay_plan = orig
    rows = sum(int(p.count.sum().item()) for k in range(args.warmup, total) for x in wl.skip_layers
               for p in step_plans[k][wl.anchor_of[x]])
    ms = [a.elapsed_time(b) for a, b in ev[len(wl.skip_layers) * wl.spec * args.warmup:]]
    err = g.cache.get_error()
    g.close()
    if err:
        log(f"[bench] device error word {err:#x}")
        sys.exit(1)
    t_pf, t_in = float(np.median(times[True])), float(np.median(times[False]))
    replay_t = float(np.mean(ms)) * 1e-3
    print(json.dumps({
        "metric": "IndexShare decode step time, skip-layer replays prefetched on a side stream vs inline",
        "value": t_pf * 1e3, "unit": "ms/step", "higher_is_better": False, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "runs": args.runs,
        "config": {"workload": wl.name, "requests": wl.R, "layers": wl.num_layers, "top_k": wl.K,
                   "device_buffer_size": wl.B, "row_bytes": wl.rb, "layer_compute_mib": n >> 20},
        "prefetch_ms_per_step": t_pf * 1e3, "inline_ms_per_step": t_in * 1e3,
        "overlap_saving": 1.0 - t_pf / t_in,
        "runs_ms": {"prefetch": [t * 1e3 for t in times[True]], "inline": [t * 1e3 for t in times[False]]},
        "replay": {"launches": len(ms), "mean_launch_us": replay_t * 1e6, "rows_per_launch": rows / len(ms),
                   "gbps": rows * wl.rb / len(ms) / replay_t / 1e9, "grid": "default (12 workgroups)"},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--runs", type=int, default=5,
                    help="repetitions of the whole timed decode (re-admitted in between); the median is reported")
    ap.add_argument("--workload", default="dsv32_decode")
    ap.add_argument("--all-steps-runs", type=int, default=3,
                    help="repetitions of the workload's whole decode from admission for the all_steps figure "
                         "(0: skip it)")
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
    ap.add_argument("--measure", default="step", choices=["step", "page_copy", "indexshare_overlap"],
                    help="page_copy: time spill and host import of paged_decode-shaped pages; "
                         "indexshare_overlap: the IndexShare step with side-stream replays against inline ones")
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
    if args.measure == "indexshare_overlap":
        measure_indexshare_overlap(dev, W, args)
        return
    wl = W.WORKLOADS[args.workload]
    total = args.warmup + args.steps
    n_all = wl.steps if args.all_steps_runs > 0 else 0
    n_gen = max(total, n_all)

    t_setup = time.time()
    g = GpuRun(wl, n_gen, block_size=args.block_size, replay_grid=args.replay_grid, host_flags=args.host_flags,
               fuse_backup=not args.no_fuse_backup)
    host_copy = None if args.no_cpu_baseline else [np.array(a, copy=True) for a in g.cache.host_np]
    streams = {a: W.TopkStream(wl, a) for a in wl.anchors}
    topk_all = [draw_topk(wl, streams, k) for k in range(n_gen)]
    topk_dev = [{a: torch.from_numpy(v).to(dev) for a, v in t.items()} for t in topk_all]
    newkv_dev = [new_kv_all_layers(wl, k, dev) for k in range(n_gen)]
    seq_dev = [g.seq_lens(k) for k in range(n_gen)]
    # every step records into its own plan count (pos/slot rows are shared), so
    # nothing but the path runs inside the timed steps
    from decode_memory_tiering_amd.hisparse import Plan
    shared = {a: [Plan.empty(wl.R, wl.K, dev) for _ in range(wl.spec)] for a in wl.anchors}
    step_plans = [{a: [Plan(p.pos, p.slot, torch.zeros(wl.R, dtype=torch.int32, device=dev))
                       for p in shared[a]] for a in wl.anchors} for _ in range(n_gen)]
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
    # the detail run also keeps the kernel's per-request counters
    # (hisparse_set_stats) over its timed steps, to cross-check the tiers
    kstats = torch.zeros(wl.R, 6, dtype=torch.int64, device=dev)
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
                g.cache.set_stats(kstats)
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
        g.cache.set_stats(None)
    kcount = kstats.sum(0).cpu().numpy()
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
    res = W.resident_mask(wl)
    # rows a fused store + backup launch writes to the hot buffer and the host pool
    fused_rows = args.steps * len(wl.anchors) * int(np.count_nonzero(res == 0)) if g.fuse_backup else 0
    alg = algorithmic_bytes(wl, topk_all, range(args.warmup, total), misses, fused_rows)
    meta_bytes = alg["hbm_read"] + alg["hbm_write"] - misses * wl.rb - 2 * fused_rows * wl.rb
    alg_total = alg["host_link_read"] + alg["host_link_write"] + alg["hbm_read"] + alg["hbm_write"]

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

    # The workload's whole decode from admission: the first step finds every
    # long request's buffer empty (all misses).  Wall clock over all steps,
    # median of the repetitions; then one more repetition with an event on
    # the main stream at every step boundary for the per-step times.
    all_steps = None
    if n_all:
        all_walls = []
        for _ in range(args.all_steps_runs):
            g.readmit()
            t0 = time.perf_counter()
            for k in range(n_all):
                run(k)
            torch.cuda.synchronize(dev)
            all_walls.append(time.perf_counter() - t0)
        g.readmit()
        main_s = torch.cuda.current_stream(dev)
        bounds = [torch.cuda.Event(enable_timing=True) for _ in range(n_all + 1)]
        bounds[0].record(main_s)
        for k in range(n_all):
            run(k)
            bounds[k + 1].record(main_s)
        torch.cuda.synchronize(dev)
        step_ms = [bounds[k].elapsed_time(bounds[k + 1]) for k in range(n_all)]
        per_k = [sum(int(np.count_nonzero(v >= 0)) for v in topk_all[k].values()) for k in range(n_all)]
        all_misses = [sum(int(p.count.sum().item()) for a in wl.anchors for p in step_plans[k][a])
                      for k in range(n_all)]
        w_all = float(np.median(all_walls))
        all_steps = dict(
            steps=n_all, value=sum(per_k) / w_all, ms_per_step=w_all / n_all * 1e3,
            runs_ms_per_step=[w / n_all * 1e3 for w in all_walls],
            first_steps_ms=[round(x, 4) for x in step_ms[:4]],
            first_steps_misses=all_misses[:4],
            steady_value=sum(per_k[2:]) / (sum(step_ms[2:]) * 1e-3) if n_all > 2 else None,
            steady_ms_per_step=float(np.mean(step_ms[2:])) if n_all > 2 else None,
            miss_gbps=sum(all_misses) * wl.rb / w_all / 1e9,
            note="steps 0..{} of the workload's decode from admission; value by wall clock (median of {} runs); "
                 "per-step times from events at step boundaries in one more run; steady = steps 2 on"
                 .format(n_all - 1, args.all_steps_runs))
        log(f"[bench] all {n_all} steps: {w_all * 1e3:.2f} ms, first step {step_ms[0]:.3f} ms")

    err = g.cache.get_error()
    if err:
        log(f"[bench] device error word {err:#x}")
        sys.exit(1)

    link = None if args.no_link else measure_link(dev)
    zc, zc_grid = (None, None) if args.no_link else measure_zero_copy(dev)
    best_link = max(link, zc) if link else None
    cpu = None
    if not args.no_cpu_baseline:
        newkv_np = [t.cpu().numpy() for t in newkv_dev[:total]]
        g.close()
        cpu = cpu_baseline(wl, total, args.warmup, host_copy, topk_all, newkv_np, pool_steps=n_gen,
                           rows_per_rep=misses + replay_rows)
    else:
        g.close()

    cb = counter_bytes(wl.name, args.steps, args.warmup, args.runs)
    traffic = None if cb is None else cb[0] + cb[1]
    tr_us = trace_mean_us(wl.name, args.steps, args.warmup, args.runs)
    step_s = wall / args.steps
    tiers = tier_shares(wl, topk_all, range(args.warmup, total), misses,
                        g.block_table_np if wl.page_size else None)
    # the same split from the kernel's own counters (entries, resident, fast
    # path, newest, hit, miss), counted in the detail run's timed steps
    tiers_kernel = dict(zip(("entries", "resident", "fast_path", "newest", "hit", "miss"), map(int, kcount)))
    tiers["kernel_counters"] = tiers_kernel
    tiers["kernel_counters_agree"] = all(tiers_kernel[k] == tiers["entries"][k] for k in tiers["entries"]) and \
        tiers_kernel["entries"] == entries
    rec = {
        "metric": "top-k rows resolved/s per decode step; miss-copy GB/s as % of host-link peak",
        "value": entries / wall,
        "unit": "top-k entries resolved/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
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
            "traffic": traffic,
            # counters over the algorithmic bytes of the same launches (1.0 =
            # no byte moved that the method does not need)
            "traffic_ratio": traffic / (alg_total / n_swap) if traffic else None,
            "counter_fetch_bytes": cb[0] if cb else None,
            "counter_write_bytes": cb[1] if cb else None,
            "algorithmic_bytes_per_launch": {k: alg[k] / n_swap for k in
                                             ("host_link_read", "host_link_write", "hbm_read", "hbm_write")},
            "launches": n_swap,
            "mean_launch_us": mean_launch_s * 1e6,
            "trace_mean_launch_us": tr_us,
            "achieved_from_trace": miss_bytes_per_launch / (tr_us * 1e-6) / 1e9 if tr_us else None,
            # a lower bound that needs no per-launch timing: every row a step
            # reads over the host link (misses and skip-layer replays) over
            # the whole step's wall time
            "achieved_from_step_time": (misses + replay_rows) * wl.rb / args.steps / step_s / 1e9,
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
        "all_steps": all_steps,
        "replay": kind_stats("replay", replay_rows),
        "backup": kind_stats("backup", backup_rows),
        "tiers": tiers,
        "misses_per_step": misses / args.steps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
