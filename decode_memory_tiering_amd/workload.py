"""Seeded synthetic inputs for the HiSparse decode-step swap-in resolver.

This module only draws inputs: workload shapes, per-step top-k rows, sequence
lengths, resident masks and KV payload rows.  It holds none of the resolver's
arithmetic, and both the HIP path and the CPU oracle take their inputs from it.

Shapes follow the pages' deployment and benchmark parameters (SGLang guide
"HiSparse: Hierarchical Sparse Attention": top_k 2048, device_buffer_size 6144
in "HiSparse Config Parameters"; a 40000-token random input in "Benchmark";
576-wide bf16 MLA rows and fp8_e4m3 rows in the KV-dtype note).  No dataset is
used: every top-k row is drawn from a seeded mixture that stands in for an
indexer's selections (half from the previous step's selection, a quarter from
the most recent 2048 positions, the rest uniform), or uniformly for the
low-locality long-context case.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

RECENT_WINDOW = 2048
POISON = 0xA5


@dataclass(frozen=True)
class Workload:
    name: str
    num_layers: int
    anchor_of: Tuple[int, ...]      # anchor layer of each layer (== itself for anchors)
    R: int                           # requests in the batch
    B: int                           # device_buffer_size (token slots per request)
    K: int                           # top_k
    rb: int                          # KV row bytes
    steps: int                       # decode steps
    spec: int = 1                    # verify rows per decode step (speculative decoding)
    n_resident: int = 0              # requests whose KV is fully resident
    topk_kind: str = "mixture"       # "mixture" | "uniform"
    seq_first: Tuple = ("fixed", 8192)   # ("fixed", L) | ("uniform", lo, hi) | ("list", L_0, ..., L_R-1): L at step 0
    row_format: str = "bf16"         # "bf16" (576 x bf16) | "fp8_656"
    seed: int = 1
    page_size: int = 0               # > 0: per-page residency with this page size
    resident_page_frac: float = 0.0  # share of (request, page) pairs that are resident

    @property
    def anchors(self) -> Tuple[int, ...]:
        return tuple(sorted(set(self.anchor_of)))

    @property
    def skip_layers(self) -> Tuple[int, ...]:
        return tuple(l for l in range(self.num_layers) if self.anchor_of[l] != l)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, with the shapes of the pages' deployment (top_k 2048,
# buffer 6144) and benchmark (40000-token inputs); the first is small enough
# for the oracle to finish in seconds.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, (0,), R=4, B=1024, K=256, rb=1152, steps=16,
                     seq_first=("fixed", 8192), seed=1),
    "fastpath_mix": Workload("fastpath_mix", 1, (0,), R=64, B=6144, K=2048, rb=1152,
                             steps=32, seq_first=("uniform", 512, 12288), seed=2),
    "dsv32_decode": Workload("dsv32_decode", 4, (0, 1, 2, 3), R=128, B=6144, K=2048,
                             rb=1152, steps=64, n_resident=32,
                             seq_first=("fixed", 40000), seed=3),
    "indexshare": Workload("indexshare", 4, (0, 0, 0, 0), R=128, B=6144, K=2048,
                           rb=1152, steps=64, seq_first=("fixed", 40000), seed=4),
    "long_context": Workload("long_context", 1, (0,), R=32, B=4096, K=2048, rb=656,
                             steps=16, spec=3, topk_kind="uniform",
                             seq_first=("fixed", 131072), row_format="fp8_656", seed=5),
    # per-page residency: a quarter of the 64-token pages of each request are
    # resident, the rest host-backed holes (vLLM design note, "Resident device
    # pages"); otherwise the DSV3.2-shaped decode of one layer
    "paged_decode": Workload("paged_decode", 1, (0,), R=128, B=6144, K=2048, rb=1152, steps=32,
                             seq_first=("fixed", 40000), seed=6, page_size=64, resident_page_frac=0.25),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def first_seq_lens(wl: Workload) -> np.ndarray:
    """Sequence length (tokens with KV, newest included) of every request at
    decode step 0; it grows by one per step."""
    kind = wl.seq_first[0]
    if kind == "fixed":
        return np.full(wl.R, int(wl.seq_first[1]), np.int32)
    if kind == "uniform":
        lo, hi = int(wl.seq_first[1]), int(wl.seq_first[2])
        return _rng(wl.seed, 7001).integers(lo, hi + 1, size=wl.R).astype(np.int32)
    if kind == "list":
        vals = np.asarray(wl.seq_first[1:], dtype=np.int32)
        assert vals.size == wl.R
        return vals
    raise ValueError(kind)


def prompt_lens(wl: Workload) -> np.ndarray:
    """Host rows valid at admission (the prefill's KV): L0 = L(step 0) - 1."""
    return first_seq_lens(wl) - 1


def seq_lens_at(wl: Workload, step: int) -> np.ndarray:
    return first_seq_lens(wl) + np.int32(step)


def max_seq(wl: Workload, steps: Optional[int] = None) -> int:
    """Host-pool rows per request that hold every position the run writes."""
    steps = wl.steps if steps is None else steps
    return int(first_seq_lens(wl).max()) + steps - 1


def resident_mask(wl: Workload) -> np.ndarray:
    """Exactly n_resident requests, picked by a seeded permutation."""
    m = np.zeros(wl.R, np.uint8)
    if wl.n_resident:
        m[_rng(wl.seed, 7002).permutation(wl.R)[: wl.n_resident]] = 1
    return m


def block_table(wl: Workload, steps: Optional[int] = None) -> Tuple[np.ndarray, int]:
    """Per-page residency: [R][max_pages] physical page of each page, or -1
    (host-backed).  A seeded share resident_page_frac of all (request, page)
    pairs is resident, on distinct physical pages in a shuffled order.
    Returns the table and the number of physical pages."""
    assert wl.page_size > 0
    ms = max_seq(wl, steps)
    max_pages = (ms + wl.page_size - 1) // wl.page_size
    rng = _rng(wl.seed, 7003)
    n = wl.R * max_pages
    n_res = int(round(wl.resident_page_frac * n))
    flat = np.full(n, -1, np.int32)
    flat[rng.choice(n, size=n_res, replace=False)] = rng.permutation(n_res).astype(np.int32)
    return flat.reshape(wl.R, max_pages), n_res


# ---------------------------------------------------------------------------
# top-k rows
# ---------------------------------------------------------------------------
def _distinct_excluding(rng: np.random.Generator, lo: int, hi: int, n: int,
                        taken: np.ndarray) -> np.ndarray:
    """Up to n distinct values of [lo, hi) not yet taken; marks them taken."""
    if n <= 0 or hi <= lo:
        return np.empty(0, np.int64)
    avail = (hi - lo) - int(np.count_nonzero(taken[lo:hi]))
    n = min(n, avail)
    if n <= 0:
        return np.empty(0, np.int64)
    if 4 * n >= avail:
        pool = np.flatnonzero(~taken[lo:hi]) + lo
        pick = rng.choice(pool, size=n, replace=False)
    else:
        parts = []
        got = 0
        while got < n:
            cand = rng.integers(lo, hi, size=2 * (n - got) + 8)
            cand = cand[~taken[cand]]
            _, first = np.unique(cand, return_index=True)
            cand = cand[np.sort(first)][: n - got]
            taken[cand] = True
            parts.append(cand)
            got += cand.size
        pick = np.concatenate(parts)
    taken[pick] = True
    return pick


def draw_topk_row(rng: np.random.Generator, L: int, K: int, prev: Optional[np.ndarray],
                  kind: str = "mixture") -> np.ndarray:
    """One request's top-k row: K distinct positions in [0, L), in a random
    order; when L <= K, a permutation of [0, L) padded with -1."""
    row = np.full(K, -1, np.int32)
    if L <= K:
        row[:L] = rng.permutation(L)
        return row
    taken = np.zeros(L, bool)
    parts = []
    if kind == "mixture":
        kp, kr = K // 2, K // 4
        if prev is not None:
            pv = prev[(prev >= 0) & (prev < L)]
            if pv.size > kp:
                pv = rng.choice(pv, size=kp, replace=False)
            taken[pv] = True
            parts.append(pv.astype(np.int64))
        parts.append(_distinct_excluding(rng, max(0, L - RECENT_WINDOW), L, kr, taken))
    elif kind != "uniform":
        raise ValueError(kind)
    have = sum(p.size for p in parts)
    parts.append(_distinct_excluding(rng, 0, L, K - have, taken))
    sel = np.concatenate(parts)
    assert sel.size == K
    row[:] = rng.permutation(sel)
    return row


class TopkStream:
    """Per-(stream, request) top-k rows, step after step.  A stream is an
    anchor layer (skip layers reuse their anchor's rows)."""

    def __init__(self, wl: Workload, stream: int):
        self.wl = wl
        self.stream = stream
        self.prev: Dict[int, np.ndarray] = {}

    def rows(self, step: int, seq_lens: np.ndarray, s: int = 0) -> np.ndarray:
        wl = self.wl
        out = np.empty((wl.R, wl.K), np.int32)
        for r in range(wl.R):
            rng = _rng(wl.seed, self.stream, r, step, s)
            row = draw_topk_row(rng, int(seq_lens[r]), wl.K, self.prev.get(r), wl.topk_kind)
            out[r] = row
            self.prev[r] = row
        return out


# ---------------------------------------------------------------------------
# KV payload rows (opaque bytes to the resolver)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def payload_rows(n: int, wl: Workload, gen, device) -> "torch.Tensor":
    """n KV rows of wl.rb bytes: bf16 N(0,1) for 576-wide MLA rows; for the
    656-byte fp8 rows, 512 e4m3 values of N(0,1), four fp32 scales of 1.0 and
    64 bf16 N(0,1) values (the row's contents never affect the resolver)."""
    torch = _torch()
    if wl.row_format == "bf16":
        assert wl.rb % 2 == 0
        x = torch.randn(n, wl.rb // 2, generator=gen, device=device)
        return x.to(torch.bfloat16).view(torch.uint8).reshape(n, wl.rb)
    if wl.row_format == "fp8_656":
        assert wl.rb == 656
        q = torch.randn(n, 512, generator=gen, device=device).to(torch.float8_e4m3fn)
        sc = torch.ones(n, 4, device=device, dtype=torch.float32)
        rope = torch.randn(n, 64, generator=gen, device=device).to(torch.bfloat16)
        return torch.cat([q.view(torch.uint8), sc.view(torch.uint8).reshape(n, 16),
                          rope.view(torch.uint8).reshape(n, 128)], dim=1)
    raise ValueError(wl.row_format)


def fill_host_pool(pool, wl: Workload, layer: int, L0: Sequence[int], device) -> None:
    """Write a layer's host pool [R][max_seq][rb] (a CPU uint8 tensor): rows
    [0, L0[r]) get seeded payload, rows from L0[r] on get the poison byte."""
    torch = _torch()
    gen = torch.Generator(device=device)
    R, ms, rb = pool.shape
    for r in range(R):
        gen.manual_seed(int(wl.seed) * 1_000_003 + layer * 10_007 + r)
        n = int(L0[r])
        if n:
            pool[r, :n].copy_(payload_rows(n, wl, gen, device))
        pool[r, n:].fill_(POISON)


def new_kv_rows(wl: Workload, step: int, layer: int, device) -> "torch.Tensor":
    """The forward's new KV row of every request at one decode step: [R][rb]."""
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(int(wl.seed) * 7_919 + step * 104_729 + layer * 15_485_863 + 1)
    return payload_rows(wl.R, wl, gen, device)
