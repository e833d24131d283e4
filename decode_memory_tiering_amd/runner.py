"""Drive a decode workload through the HIP path (tests and benchmark).

One decode step, for every layer in order (SGLang guide "HiSparse:
Hierarchical Sparse Attention", "Decode Workflow" and "Shared-index
prefetch"; vLLM design note "HiSparse local KV offload architecture",
"Resident device pages" for the verify rows):

  store_newest(l)                        the forward's KV write (on an anchor layer
                                         it rides in the first swap-in's launch)
  anchor layer:  swap_in(l), once per verify row s, each with its own plan row
                 then, with prefetch on, the replays of verify row 0's plan
                 on its skip layers are issued on the side stream after an
                 event
  skip layer:    per verify row s, in order: the replay of plan row s (row 0
                 from the side stream when prefetched, else inline), then
                 that row's consumer.  Row s+1's misses take victims from
                 slots row s resolved to, so row s+1 is replayed only after
                 row s was consumed; this is why only row 0 is prefetched.
  backup(l)                              eager backup of the newest token (on an
                                         anchor layer it rides in that launch too)

Every launch goes through the C ABI; this module only allocates tensors,
moves seeded inputs to the device and orders streams.
"""
from __future__ import annotations

import os
from typing import Dict, List, Optional

import numpy as np

from . import workload as W
from .hisparse import HISPARSE_HOST_DEFAULT, HiSparseCache, Plan


def prefetch_enabled() -> bool:
    """Skip-layer replays run on a side stream unless HISPARSE_DISABLE_PREFETCH=1
    (A/B switch; the SGLang guide's "Shared-index prefetch" has the same one)."""
    return os.environ.get("HISPARSE_DISABLE_PREFETCH", "0") != "1"


class GpuRun:
    def __init__(self, wl: W.Workload, steps: Optional[int] = None, device: str = "cuda",
                 block_size: int = 0, replay_grid: int = 0, host_flags: int = HISPARSE_HOST_DEFAULT,
                 prefetch: Optional[bool] = None, fill: bool = True, fuse_store: bool = True,
                 fuse_backup: bool = True, static_state: bool = False):
        import torch
        self.torch = torch
        self.wl = wl
        self.steps = wl.steps if steps is None else steps
        self.dev = torch.device(device)
        self.max_seq = W.max_seq(wl, self.steps)
        self.L0 = W.prompt_lens(wl)
        self.cache = HiSparseCache(num_layers=wl.num_layers, anchor_of=wl.anchor_of, R=wl.R, B=wl.B,
                                   K=wl.K, rb=wl.rb, max_seq=self.max_seq, device=device,
                                   host_flags=host_flags, block_size=block_size,
                                   replay_grid=replay_grid, static_state=static_state)
        self.prefetch = prefetch_enabled() if prefetch is None else prefetch
        # an anchor layer's KV write rides in its swap-in launch
        # (store_swap_in), and so does its eager backup (store_swap_in_backup)
        self.fuse_store = fuse_store
        self.fuse_backup = fuse_store and fuse_backup
        res = W.resident_mask(wl)
        self.resident = torch.from_numpy(res).to(self.dev) if res.any() else None
        self.resident_np = res
        self.out = {g: torch.zeros(wl.spec, wl.R, wl.K, dtype=torch.int32, device=self.dev)
                    for g in wl.anchors}
        self.plans = {g: [Plan.empty(wl.R, wl.K, self.dev) for _ in range(wl.spec)] for g in wl.anchors}
        self.side = torch.cuda.Stream(device=self.dev)
        self.events: Dict[int, "torch.cuda.Event"] = {}
        # per-page residency: the block table, and per layer a resident cache
        # [n_phys * P][rb] holding the resident pages' KV; the caller's row
        # view is the resident cache's rows, then the hot buffer's rows.
        self.paged = wl.page_size > 0
        if self.paged:
            assert wl.n_resident == 0, "per-page residency replaces the per-request mask"
            bt, n_phys = W.block_table(wl, self.steps)
            self.block_table_np = bt
            self.block_table = torch.from_numpy(bt).to(self.dev)
            self.hot_row_base = n_phys * wl.page_size
            self.res_cache = [torch.zeros(n_phys * wl.page_size, wl.rb, dtype=torch.uint8, device=self.dev)
                              for _ in range(wl.num_layers)]
            self._resident_newest = {}
            for k in range(self.steps):          # every step's pairs, ahead of any timing
                self._resident_pairs(W.seq_lens_at(wl, k))
        if fill:
            self.fill_and_admit()

    # -- set-up ----------------------------------------------------------------
    def fill_and_admit(self):
        wl = self.wl
        for l in range(wl.num_layers):
            W.fill_host_pool(self.cache.host[l], wl, l, self.L0, self.dev)
        if self.paged:
            self._fill_resident()
        self.readmit()

    def readmit(self):
        """Admit every request again on every anchor layer (state reset, and
        the hot rows of short requests refilled from the host pool).  Host
        rows past the prefill hold what the previous run's backups wrote,
        which a new run writes again with the same values, so a run after
        readmit() repeats the previous one exactly."""
        torch, wl = self.torch, self.wl
        req = torch.arange(wl.R, dtype=torch.int32, device=self.dev)
        L0 = torch.from_numpy(self.L0.astype(np.int32)).to(self.dev)
        for g in wl.anchors:
            self.cache.admit(g, req, L0)
        torch.cuda.synchronize(self.dev)

    def _fill_resident(self):
        """Resident pages hold the same KV as the host pool (prefill's rows)."""
        torch, wl, P = self.torch, self.wl, self.wl.page_size
        r_idx, p_idx = np.nonzero(self.block_table_np >= 0)
        phys = self.block_table_np[r_idx, p_idx]
        for l in range(wl.num_layers):
            host = self.cache.host[l]
            for r, pg, ph in zip(r_idx.tolist(), p_idx.tolist(), phys.tolist()):
                lo, hi = pg * P, min((pg + 1) * P, self.max_seq)
                self.res_cache[l][ph * P: ph * P + (hi - lo)].copy_(host[r, lo:hi], non_blocking=False)

    def _resident_pairs(self, seq_lens_np):
        """(request, resident row) of every request whose newest token's page
        is resident, as device index tensors (None if there is none).  They
        depend only on the sequence lengths (the block table is fixed for the
        run), so they are computed once per distinct lengths; __init__ does
        it for every step of the decode."""
        key = seq_lens_np.tobytes()
        if key not in self._resident_newest:
            P, bt = self.wl.page_size, self.block_table_np
            pg = (seq_lens_np.astype(np.int64) - 1) // P
            inside = pg < bt.shape[1]
            phys = np.where(inside, bt[np.arange(self.wl.R), np.minimum(pg, bt.shape[1] - 1)], -1)
            rows = np.nonzero(phys >= 0)[0]
            dst = phys[rows].astype(np.int64) * P + (seq_lens_np[rows].astype(np.int64) - 1) % P
            self._resident_newest[key] = (self.torch.from_numpy(rows.astype(np.int64)).to(self.dev),
                                          self.torch.from_numpy(dst).to(self.dev)) if rows.size else None
        return self._resident_newest[key]

    def store_newest_resident(self, layer: int, new_kv_l, seq_lens_np):
        """The forward's KV write for requests whose newest page is resident."""
        idx = self._resident_pairs(seq_lens_np)
        if idx is not None:
            src, dst = idx
            self.res_cache[layer].index_copy_(0, dst, new_kv_l.index_select(0, src))

    def row_view(self, layer: int):
        """The caller's row view of one layer: resident cache rows, then hot rows."""
        wl = self.wl
        return self.torch.cat([self.res_cache[layer], self.cache.hot[layer].view(wl.R * (wl.B + 1), wl.rb)])

    def seq_lens(self, step: int):
        return self.torch.from_numpy(W.seq_lens_at(self.wl, step).astype(np.int32)).to(self.dev)

    # -- one decode step ------------------------------------------------------
    def step(self, topk: Dict[int, "torch.Tensor"], new_kv: "torch.Tensor", seq_lens,
             between_layers=None, after_swap_in=None, plans: Optional[Dict[int, List[Plan]]] = None,
             seq_lens_np=None, after_replay=None):
        """topk[g]: [S][R][K] int32 (device) for every anchor g; new_kv:
        [layers][R][rb] uint8 (device); seq_lens: [R] int32 (device).
        between_layers(l) runs on the main stream after layer l (a stand-in for
        the layer's other compute); after_swap_in(g, s) runs right after each
        swap-in (the consumer of that verify row); after_replay(l, s) runs on
        the main stream once skip layer l's rows of verify row s are in place
        (that layer's consumer of the row); plans replaces the plan rows
        this step records into (default: self.plans); seq_lens_np (host copy
        of seq_lens) lets a paged run write the newest token into a resident
        page, as the forward would."""
        torch, wl, c = self.torch, self.wl, self.cache
        plans = self.plans if plans is None else plans
        main = torch.cuda.current_stream(self.dev)
        for l in range(wl.num_layers):
            g = wl.anchor_of[l]
            # the paged path fuses the KV write only together with the backup
            fused = self.fuse_store and g == l and (not self.paged or self.fuse_backup)
            if not fused:
                c.store_newest(l, new_kv[l], seq_lens, self.resident)
            if self.paged and seq_lens_np is not None:
                self.store_newest_resident(l, new_kv[l], seq_lens_np)
            if g == l:
                for s in range(wl.spec):
                    if self.paged and fused and s == 0:
                        c.store_swap_in_paged_backup(l, new_kv[l], topk[l][s], seq_lens, self.block_table,
                                                     wl.page_size, self.hot_row_base, None, self.out[l][s],
                                                     plans[l][s])
                    elif self.paged:
                        c.swap_in_paged(l, topk[l][s], seq_lens, self.block_table, wl.page_size,
                                        self.hot_row_base, None, self.out[l][s], plans[l][s])
                    elif fused and s == 0:
                        fn = c.store_swap_in_backup if self.fuse_backup else c.store_swap_in
                        fn(l, new_kv[l], topk[l][s], seq_lens, self.resident, None, self.out[l][s], plans[l][s])
                    else:
                        c.swap_in(l, topk[l][s], seq_lens, self.resident, None, self.out[l][s], plans[l][s])
                    if after_swap_in is not None:
                        after_swap_in(l, s)
                skips = [x for x in wl.skip_layers if wl.anchor_of[x] == l]
                if skips and self.prefetch:
                    ev = torch.cuda.Event()
                    ev.record(main)
                    self.side.wait_event(ev)
                    with torch.cuda.stream(self.side):
                        for x in skips:
                            c.replay_plan(x, plans[l][0], None, self.side)
                            e2 = torch.cuda.Event()
                            e2.record(self.side)
                            self.events[x] = e2
            else:
                for s in range(wl.spec):
                    if self.prefetch and s == 0:
                        main.wait_event(self.events.pop(l))
                    else:
                        c.replay_plan(l, plans[g][s], None, main)
                    if after_replay is not None:
                        after_replay(l, s)
            if not (fused and self.fuse_backup):
                c.backup(l, seq_lens, self.resident)
            if between_layers is not None:
                between_layers(l)

    def close(self):
        self.cache.close()


def valid_entries(topk_np: np.ndarray) -> int:
    return int(np.count_nonzero(topk_np >= 0))


def new_kv_all_layers(wl: W.Workload, step: int, device) -> "torch.Tensor":
    import torch
    return torch.stack([W.new_kv_rows(wl, step, l, device) for l in range(wl.num_layers)])


def draw_topk(wl: W.Workload, streams: Dict[int, W.TopkStream], step: int) -> Dict[int, np.ndarray]:
    """Top-k rows of one decode step for every anchor: [S][R][K] int32."""
    L = W.seq_lens_at(wl, step)
    return {g: np.stack([streams[g].rows(step, L, s) for s in range(wl.spec)]) for g in wl.anchors}
