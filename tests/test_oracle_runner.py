"""The oracle's decode driver on request subsets.

Requests are independent in the method (each has its own LRU list, slot map,
hot rows and host rows), so stepping disjoint request subsets, in any order
and from several threads, must leave every buffer exactly as one full-batch
step does.  The CPU baseline of the benchmark relies on this when it splits
the requests over threads."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from decode_memory_tiering_amd import workload as W
from decode_memory_tiering_amd.runner import draw_topk, new_kv_all_layers
from oracle.runner import OracleRun

CASES = [
    W.Workload("subset_mix", 3, (0, 0, 2), R=7, B=200, K=64, rb=32, steps=6, spec=2, n_resident=2,
               seq_first=("uniform", 100, 400), seed=11),
    W.Workload("subset_paged", 2, (0, 0), R=6, B=150, K=50, rb=48, steps=5, page_size=16,
               resident_page_frac=0.3, seq_first=("uniform", 120, 500), seed=12),
]


def inputs(wl):
    streams = {a: W.TopkStream(wl, a) for a in wl.anchors}
    topk = [draw_topk(wl, streams, k) for k in range(wl.steps)]
    newkv = [new_kv_all_layers(wl, k, "cpu").numpy() for k in range(wl.steps)]
    return topk, newkv


def snapshot(o):
    orc = o.orc
    return ([h.copy() for h in orc.host], [h.copy() for h in orc.hot],
            {g: a.copy() for g, a in orc.lru.items()}, {g: a.copy() for g, a in orc.tok.items()})


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_subsets_match_full_batch(wl):
    topk, newkv = inputs(wl)
    full, part = OracleRun(wl), OracleRun(wl)
    shares = [np.array([5, 0, 3], np.int32), np.array([1, 4], np.int32), np.array([2] + ([6] if wl.R > 6 else []),
                                                                                     np.int32)]
    for k in range(wl.steps):
        outs, plans = full.step(k, topk[k], newkv[k])
        with ThreadPoolExecutor(len(shares)) as pool:
            got = list(pool.map(lambda r: part.step(k, topk[k], newkv[k], r), shares))
        for req, (o2, p2) in zip(shares, got):
            for g in wl.anchors:
                np.testing.assert_array_equal(o2[g], outs[g][:, req])
                for s in range(wl.spec):
                    np.testing.assert_array_equal(p2[g][s].count, plans[g][s].count[req])
                    for j, r in enumerate(req):
                        n = int(plans[g][s].count[r])
                        np.testing.assert_array_equal(p2[g][s].pos[j, :n], plans[g][s].pos[r, :n])
                        np.testing.assert_array_equal(p2[g][s].slot[j, :n], plans[g][s].slot[r, :n])
    a, b = snapshot(full), snapshot(part)
    for x, y in zip(a[0] + a[1], b[0] + b[1]):
        np.testing.assert_array_equal(x, y)
    for g in wl.anchors:
        np.testing.assert_array_equal(a[2][g], b[2][g])
        np.testing.assert_array_equal(a[3][g], b[3][g])


def test_readmit_repeats_the_decode():
    wl = CASES[0]
    topk, newkv = inputs(wl)
    o = OracleRun(wl)
    first = [o.step(k, topk[k], newkv[k])[0] for k in range(wl.steps)]
    o.readmit()
    again = [o.step(k, topk[k], newkv[k])[0] for k in range(wl.steps)]
    for x, y in zip(first, again):
        for g in wl.anchors:
            np.testing.assert_array_equal(x[g], y[g])


@pytest.mark.parametrize("threads", [1, 3, 16])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_threaded_timing_driver_runs_the_same_decode(wl, threads):
    # the CPU baseline's C driver (admission, warm-up steps, timed steps over
    # request shares on threads) leaves every buffer as the step-by-step
    # decode does; a second call (re-admitted) repeats it
    from oracle.timing import DecodeTimer
    topk, newkv = inputs(wl)
    ref = OracleRun(wl)
    for k in range(wl.steps):
        ref.step(k, topk[k], newkv[k])
    timed = OracleRun(wl)
    timer = DecodeTimer(timed, topk, newkv, first_timed=2)
    for _ in range(2):
        assert timer.run(threads) >= 0.0
        a, b = snapshot(ref), snapshot(timed)
        for x, y in zip(a[0] + a[1], b[0] + b[1]):
            np.testing.assert_array_equal(x, y)
        for g in wl.anchors:
            np.testing.assert_array_equal(a[2][g], b[2][g])
            np.testing.assert_array_equal(a[3][g], b[3][g])
