"""The benchmark's tier breakdown, checked against what the oracle actually
returned: every valid top-k entry is counted in exactly one tier, and the
hot-buffer hits it derives from the inputs and the miss count equal the hits
in the oracle's outputs."""
import numpy as np
import pytest

import bench
from decode_memory_tiering_amd import workload as W
from decode_memory_tiering_amd.runner import draw_topk, new_kv_all_layers
from oracle.runner import OracleRun

CASES = [
    W.Workload("tiers_mix", 2, (0, 0), R=8, B=200, K=64, rb=32, steps=6, spec=2, n_resident=2,
               seq_first=("uniform", 100, 400), seed=21),
    W.Workload("tiers_paged", 1, (0,), R=6, B=150, K=50, rb=48, steps=5, page_size=16,
               resident_page_frac=0.3, seq_first=("uniform", 120, 500), seed=22),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_tier_shares_match_oracle_outputs(wl):
    o = OracleRun(wl)
    streams = {a: W.TopkStream(wl, a) for a in wl.anchors}
    topk_all, misses, hits, resident, newest = [], 0, 0, 0, 0
    res_mask = W.resident_mask(wl).astype(bool)
    for k in range(wl.steps):
        topk = draw_topk(wl, streams, k)
        topk_all.append(topk)
        outs, plans = o.step(k, topk, new_kv_all_layers(wl, k, "cpu").numpy())
        L = W.seq_lens_at(wl, k)
        for a in wl.anchors:
            for s in range(wl.spec):
                misses += int(plans[a][s].count.sum())
                out, x = outs[a][s], topk[a][s]
                for r in range(wl.R):
                    if L[r] <= wl.B or (not wl.page_size and res_mask[r]):
                        continue
                    v = out[r][x[r] >= 0]
                    if wl.page_size:
                        resident += int((v < o.hot_row_base).sum())
                        v = v[v >= o.hot_row_base] - (o.hot_row_base + r * (wl.B + 1))
                    newest += int((v == wl.B).sum())
                    hits += int(((v >= 0) & (v < wl.B)).sum())
    hits -= misses
    got = bench.tier_shares(wl, topk_all, range(wl.steps), misses, o.block_table if wl.page_size else None)
    assert got["entries"]["hit"] == hits
    assert got["entries"]["newest"] == newest
    if wl.page_size:
        # resident-page entries of long rows; short rows' resident entries count there too
        assert got["entries"]["resident"] >= resident
    valid = sum(int((v >= 0).sum()) for t in topk_all for v in t.values())
    assert sum(got["entries"].values()) == valid
    assert 0 < got["hot_hit_rate"] < 1


def test_committed_counters_apply_only_to_their_window(tmp_path, monkeypatch):
    # a counter summary is attached only to the exact decode window (workload,
    # timed steps, warm-up steps, runs) and kernel source it was taken on
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "swap_in_kernel_wl_counters.md").write_text(
        "# counters\n\nrocprofv3 --pmc FETCH_SIZE -- python bench.py\n\nsrc_sha256: abc\nworkload: wl\n"
        "steps: 20\nwarmup: 5\nruns: 5\nfetch_bytes_per_launch: 100\nwrite_bytes_per_launch: 50\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_src_sha256", lambda: "abc")
    assert bench.counter_bytes("wl", 20, 5, 5) == (100.0, 50.0)
    assert bench.counter_bytes("wl", 30, 2, 5) is None        # another window
    assert bench.counter_bytes("wl", 20, 5, 3) is None
    assert bench.counter_bytes("other", 20, 5, 5) is None
    monkeypatch.setattr(bench, "_src_sha256", lambda: "changed")
    assert bench.counter_bytes("wl", 20, 5, 5) is None        # kernel changed since


def test_algorithmic_bytes_split():
    wl = CASES[0]
    streams = {a: W.TopkStream(wl, a) for a in wl.anchors}
    topk_all = [draw_topk(wl, streams, k) for k in range(3)]
    alg = bench.algorithmic_bytes(wl, topk_all, range(3), misses=10, fused_rows=4)
    assert alg["host_link_read"] == 10 * wl.rb and alg["host_link_write"] == 4 * wl.rb
    entries = sum(int((v >= 0).sum()) for t in topk_all for v in t.values())
    assert alg["entries"] == entries
    assert alg["hbm_read"] == entries * 4 + alg["slow_rows"] * 8 * wl.B + 4 * wl.rb


def test_cpu_baseline_reports_entries_and_copy_rate():
    # the benchmark's CPU-baseline leg on a small decode: the oracle timed
    # from C over the timed steps, on one thread and on request shares;
    # entries/s and copy GB/s come from the same repetitions, so their ratio
    # is the rows copied per entry resolved
    wl = CASES[0]
    steps, warmup = wl.steps, 2
    streams = {a: W.TopkStream(wl, a) for a in wl.anchors}
    topk_all = [draw_topk(wl, streams, k) for k in range(steps)]
    newkv = [new_kv_all_layers(wl, k, "cpu").numpy() for k in range(steps)]
    o = OracleRun(wl, steps)
    rows = 0
    for k in range(steps):
        _, plans = o.step(k, topk_all[k], newkv[k])
        if k >= warmup:   # misses, and every skip layer's replay of its anchor's plans
            rows += sum(int(p.count.sum()) for a in wl.anchors for p in plans[a])
            rows += sum(int(p.count.sum()) for x in wl.skip_layers for p in plans[wl.anchor_of[x]])
    pools = [np.array(h, copy=True) for h in OracleRun(wl, steps).orc.host]
    got = bench.cpu_baseline(wl, steps, warmup, pools, topk_all, newkv, budget_s=0.05, max_threads=2,
                             rows_per_rep=rows)
    entries = sum(int((v >= 0).sum()) for t in topk_all[warmup:] for v in t.values())
    assert got["kind"] == "oracle" and got["cores"] == 1 and got["value"] > 0
    assert got["threads"]["cores"] == min(2, len(__import__("os").sched_getaffinity(0)))
    assert got["copy_gbps"] == pytest.approx(got["value"] / entries * rows * wl.rb / 1e9)
    assert got["threads"]["copy_gbps"] == pytest.approx(got["threads"]["value"] / entries * rows * wl.rb / 1e9)


def test_more_than_one_gpu_is_refused():
    # one GPU only: asked for more, the benchmark says so and exits before
    # touching any device
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=root)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr and res.stdout == ""
