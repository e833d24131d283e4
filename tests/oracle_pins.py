"""Checks that pin the CPU oracle to facts fixed outside itself.

Each ``pin_*`` function runs the oracle (any build of ``hisparse_oracle.c``,
passed in as a loaded library) and returns a list of failure strings; an
empty list means the pin holds.  ``test_oracle_pins.py`` asserts that every
pin holds for the real oracle, and that every planted mistake in a mutated
copy of the oracle is caught by at least one pin.

What each pin rests on:
  * pin_closed_forms: the short-sequence fast path gives slot = position and
    copies nothing (SGLang guide, "Decode Workflow"); a resident request
    returns its own positions before any hot lookup or host copy (vLLM design
    note, "Resident device pages" and "Performance invariants").
  * pin_textbook_lru_*: state and slots equal a textbook LRU cache
    (``collections.OrderedDict``) fed each step's accesses -- brute force
    over every top-k sequence of tiny sizes, and random larger ones.
  * pin_invariants: a hit never moves its row; the slot map stays injective;
    every resolved slot holds the bytes of the position asked for (the
    pages' correctness statement for the hot lookup and the host copy);
    the plan row lists exactly the misses; backup writes the newest token.
  * pin_hand_trace: a trace worked out by hand (tests/golden).
  * pin_replay: a skip layer that replays the plan ends up byte-identical to
    one resolved directly (SGLang guide, "Shared-index prefetch").
  * pin_paged_*: per-page residency (vLLM design note, "Resident device
    pages"): a hand-worked trace; every page resident gives page*P + t%P
    and moves nothing; no page resident gives the per-request resolver's
    result; and in the caller's combined row view every resolved row holds
    the position's KV while resident positions never reach the hot tiers.
  * pin_spill_round_trip / pin_import_mirror: page transfers (vLLM design
    note, "Spill transaction" and "P/D import target"): the copied pages
    equal their sources, nothing else changes, a page past the pool is cut,
    and after the table entry is replaced the resolver still returns every
    position's KV.
"""
from __future__ import annotations

import itertools
import json
import os
from typing import List, Sequence

import numpy as np

from oracle.oracle import ORC_EPRECOND, Oracle, OracleError
from textbook_lru import TextbookLRU

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RB = 16  # tiny payload rows: (request, position) as two int64


def _row(r: int, t: int, tag: int = 0) -> np.ndarray:
    return np.array([r, t + tag], dtype=np.int64).view(np.uint8)


def _tiny_oracle(lib, R, B, K, max_seq, layers=1, anchor_of=(0,)):
    return Oracle(num_layers=layers, anchor_of=anchor_of, R=R, B=B, K=K, rb=RB,
                  max_seq=max_seq, lib=lib)


def _fill_host(orc: Oracle, L0s: Sequence[int], layer: int = 0, tag: int = 0):
    for r in range(orc.R):
        orc.host[layer][r, :, :] = 0xA5
        for t in range(int(L0s[r])):
            orc.host[layer][r, t] = _row(r, t, tag)


def _new_kv(R: int, L: Sequence[int], tag: int = 10_000_000) -> np.ndarray:
    return np.stack([_row(r, int(L[r]) - 1, tag) for r in range(R)])


# ---------------------------------------------------------------------------
def pin_closed_forms(lib) -> List[str]:
    fails = []
    rng = np.random.default_rng(11)
    R, B, K = 6, 16, 8
    max_seq = 40
    orc = _tiny_oracle(lib, R, B, K, max_seq)
    L0 = np.array([3, 10, 15, 16, 20, 30], np.int32)
    _fill_host(orc, L0)
    orc.admit(0, np.arange(R), L0)
    resident = np.array([0, 0, 0, 0, 1, 1], np.uint8)
    for step in range(4):
        L = L0 + 1 + step
        topk = np.full((R, K), -1, np.int32)
        for r in range(R):
            n = min(K, int(L[r]))
            topk[r, :n] = rng.choice(int(L[r]), size=n, replace=False)
        orc.store_newest(0, _new_kv(R, L), L, resident)
        lru0, tok0, hot0 = orc.lru[0].copy(), orc.tok[0].copy(), orc.hot[0].copy()
        host0 = orc.host[0].copy()
        out, plan = orc.swap_in(0, topk, L, resident)
        for r in range(R):
            if resident[r] or L[r] <= B:
                if not np.array_equal(out[r], topk[r]):
                    fails.append(f"closed form: step {step} r {r}: out != topk")
                if plan.count[r] != 0:
                    fails.append(f"closed form: step {step} r {r}: plan count {plan.count[r]}")
                if not (np.array_equal(orc.lru[0][r], lru0[r]) and np.array_equal(orc.tok[0][r], tok0[r])):
                    fails.append(f"closed form: step {step} r {r}: state changed")
                if not np.array_equal(orc.hot[0][r], hot0[r]):
                    fails.append(f"closed form: step {step} r {r}: hot bytes changed")
        orc.backup(0, L, resident)
        for r in range(R):
            if resident[r] and not np.array_equal(orc.host[0][r], host0[r]):
                fails.append(f"closed form: resident request {r} host pool written by backup")
            if not resident[r] and L[r] <= B:
                # fast path: the newest token sits at its own position and is
                # backed up from there
                if not np.array_equal(orc.host[0][r, L[r] - 1], _row(r, int(L[r]) - 1, 10_000_000)):
                    fails.append(f"closed form: fast-path backup of r {r} wrong")
                for i in range(K):
                    t = int(topk[r, i])
                    if t >= 0 and not np.array_equal(orc.hot[0][r, t], orc.host[0][r, t]):
                        fails.append(f"closed form: fast path slot {t} of r {r} does not hold position {t}")
                        break
    return fails


# ---------------------------------------------------------------------------
def _textbook_compare(lib, B, K, L0, seqs: np.ndarray, label: str) -> List[str]:
    """seqs: [n][steps][K] top-k rows; request n runs sequence n."""
    fails = []
    n, steps, _ = seqs.shape
    max_seq = L0 + steps
    orc = _tiny_oracle(lib, n, B, K, max_seq)
    L0s = np.full(n, L0, np.int32)
    _fill_host(orc, L0s)
    orc.admit(0, np.arange(n), L0s)
    books = [TextbookLRU(B, L0) for _ in range(n)]
    for k in range(steps):
        L = L0s + 1 + k
        orc.store_newest(0, _new_kv(n, L), L)
        out, plan = orc.swap_in(0, seqs[:, k, :], L)
        orc.backup(0, L)
        for r in range(n):
            exp_out = books[r].step(seqs[r, k].tolist(), int(L[r]))
            exp_lru, exp_tok = books[r].state()
            if out[r].tolist() != exp_out:
                fails.append(f"{label}: seq {r} step {k}: out {out[r].tolist()} != textbook {exp_out}")
            elif orc.lru[0][r].tolist() != exp_lru or orc.tok[0][r].tolist() != exp_tok:
                fails.append(f"{label}: seq {r} step {k}: state lru={orc.lru[0][r].tolist()} "
                             f"tok={orc.tok[0][r].tolist()} != textbook {exp_lru} {exp_tok}")
            if len(fails) > 5:
                return fails
    return fails


def _all_rows(L: int, K: int, with_pad: bool) -> List[tuple]:
    syms = list(range(L))
    rows = list(itertools.permutations(syms, K))
    if with_pad:
        for npad in range(1, K + 1):
            for pos in itertools.combinations(range(K), npad):
                for vals in itertools.permutations(syms, K - npad):
                    row, it = [], iter(vals)
                    for i in range(K):
                        row.append(-1 if i in pos else next(it))
                    rows.append(tuple(row))
    return rows


def pin_textbook_lru_exhaustive(lib) -> List[str]:
    """Every top-k sequence over tiny spaces: B <= 4, L <= 12, up to 3 steps."""
    fails = []
    cases = [  # (B, K, L0, steps, padding)
        (1, 1, 1, 3, True), (1, 1, 3, 3, True),
        (2, 1, 2, 3, True), (2, 2, 2, 3, True), (2, 2, 4, 3, False),
        (3, 2, 3, 3, False), (3, 3, 3, 2, False), (3, 2, 5, 3, False),
        (4, 2, 4, 3, False), (4, 3, 6, 2, False), (4, 4, 9, 1, False),
    ]
    for B, K, L0, steps, pad in cases:
        per_step = [_all_rows(L0 + 1 + k, K, pad) for k in range(steps)]
        seqs = np.array(list(itertools.product(*per_step)), dtype=np.int32)  # [n][steps][K]
        fails += _textbook_compare(lib, B, K, L0, seqs, f"exhaustive B={B} K={K} L0={L0}")
        if fails:
            return fails
    return fails


def pin_textbook_lru_random(lib, n_seq: int = 64, steps: int = 12) -> List[str]:
    fails = []
    rng = np.random.default_rng(5)
    for B, K, L0 in [(8, 8, 12), (16, 5, 16), (16, 12, 40), (32, 16, 33), (64, 48, 200)]:
        seqs = np.empty((n_seq, steps, K), np.int32)
        for r in range(n_seq):
            for k in range(steps):
                L = L0 + 1 + k
                # bias towards recent positions so hits are common
                hi = min(L, rng.integers(K + 1, L + 1))
                seqs[r, k] = rng.choice(hi, size=K, replace=False) if hi >= K else \
                    rng.choice(L, size=K, replace=False)
        fails += _textbook_compare(lib, B, K, L0, seqs, f"random B={B} K={K}")
        if fails:
            return fails
    return fails


# ---------------------------------------------------------------------------
def pin_invariants(lib, steps: int = 10) -> List[str]:
    fails = []
    rng = np.random.default_rng(3)
    R, B, K = 8, 32, 12
    L0 = np.array([20, 31, 32, 33, 50, 90, 200, 300], np.int32)
    max_seq = int(L0.max()) + steps
    orc = _tiny_oracle(lib, R, B, K, max_seq)
    _fill_host(orc, L0)
    orc.admit(0, np.arange(R), L0)
    prev = [None] * R
    for k in range(steps):
        L = L0 + 1 + k
        topk = np.full((R, K), -1, np.int32)
        for r in range(R):
            Lr = int(L[r])
            cand = []
            if prev[r] is not None:
                cand = [t for t in prev[r] if t >= 0][: K // 2]
            rest = [t for t in rng.permutation(Lr).tolist() if t not in cand]
            row = (cand + rest)[:K]
            if Lr - 1 not in row and rng.random() < 0.5:
                row[-1] = Lr - 1
            rng.shuffle(row)
            topk[r, : len(row)] = row
            prev[r] = row
        orc.store_newest(0, _new_kv(R, L), L)
        tok0 = orc.tok[0].copy()
        hot0 = orc.hot[0].copy()
        out, plan = orc.swap_in(0, topk, L)
        orc.backup(0, L)
        for r in range(R):
            Lr = int(L[r])
            o, t_row = out[r], topk[r]
            valid = o[t_row >= 0]
            if len(set(valid.tolist())) != len(valid):
                fails.append(f"invariant: step {k} r {r}: resolved slots not distinct")
            if Lr > B and np.count_nonzero(o == B) != np.count_nonzero(t_row == Lr - 1):
                fails.append(f"invariant: step {k} r {r}: newest row misuse")
            for i in range(K):
                t = int(t_row[i])
                if t < 0:
                    if o[i] != -1:
                        fails.append(f"invariant: padding not -1")
                    continue
                # the pages' correctness statement: the resolved row holds t's KV
                if not np.array_equal(orc.hot[0][r, o[i]], orc.host[0][r, t]):
                    fails.append(f"invariant: step {k} r {r} i {i}: slot {o[i]} does not hold position {t}")
                if Lr > B and t != Lr - 1 and t in tok0[r]:
                    s = int(np.flatnonzero(tok0[r] == t)[0])
                    if o[i] != s:
                        fails.append(f"invariant: step {k} r {r}: hit on {t} moved from {s} to {o[i]}")
                    if not np.array_equal(orc.hot[0][r, s], hot0[r, s]):
                        fails.append(f"invariant: step {k} r {r}: hit row {s} rewritten")
            tk = orc.tok[0][r]
            pos = tk[tk >= 0]
            if len(set(pos.tolist())) != len(pos):
                fails.append(f"invariant: step {k} r {r}: slot map not injective")
            if sorted(orc.lru[0][r].tolist()) != list(range(B)):
                fails.append(f"invariant: step {k} r {r}: lru not a permutation")
            if Lr > B:
                for s in range(B):
                    if tk[s] >= 0 and not np.array_equal(orc.hot[0][r, s], orc.host[0][r, tk[s]]):
                        fails.append(f"invariant: step {k} r {r}: slot {s} dirty")
                        break
                miss_i = [i for i in range(K) if t_row[i] >= 0 and t_row[i] != Lr - 1
                          and t_row[i] not in tok0[r]]
                if plan.count[r] != len(miss_i):
                    fails.append(f"invariant: step {k} r {r}: plan count {plan.count[r]} != {len(miss_i)}")
                else:
                    m = plan.count[r]
                    if plan.pos[r, :m].tolist() != [int(t_row[i]) for i in miss_i] or \
                            plan.slot[r, :m].tolist() != [int(o[i]) for i in miss_i]:
                        fails.append(f"invariant: step {k} r {r}: plan pairs wrong")
            elif plan.count[r] != 0:
                fails.append(f"invariant: fast path recorded a plan")
            if not np.array_equal(orc.host[0][r, Lr - 1], _row(r, Lr - 1, 10_000_000)):
                fails.append(f"invariant: step {k} r {r}: backup did not write newest token")
            if len(fails) > 5:
                return fails
    return fails


# ---------------------------------------------------------------------------
def pin_hand_trace(lib) -> List[str]:
    with open(os.path.join(GOLDEN, "hand_worked_trace.json")) as f:
        g = json.load(f)
    fails = []
    for tr in g["traces"]:
        B, K, L0 = tr["B"], tr["K"], tr["L0"]
        orc = _tiny_oracle(lib, 1, B, K, L0 + len(tr["steps"]) + 1)
        _fill_host(orc, [L0])
        orc.admit(0, [0], [L0])
        for k, st in enumerate(tr["steps"]):
            L = np.array([st["L"]], np.int32)
            orc.store_newest(0, _new_kv(1, L), L)
            out, plan = orc.swap_in(0, np.array([st["topk"]], np.int32), L)
            orc.backup(0, L)
            got = dict(out=out[0].tolist(), lru=orc.lru[0][0].tolist(), tok=orc.tok[0][0].tolist(),
                       plan_pos=plan.pos[0, : plan.count[0]].tolist(),
                       plan_slot=plan.slot[0, : plan.count[0]].tolist())
            for key in got:
                if got[key] != st[key]:
                    fails.append(f"hand trace '{tr['name']}' step {k}: {key} {got[key]} != {st[key]}")
    return fails


# ---------------------------------------------------------------------------
def pin_replay(lib, steps: int = 6) -> List[str]:
    """Layer 1 replays layer 0's plan; layer 2 is a second anchor fed the same
    top-k (its own LRU).  Layers 1 and 2 must end byte-identical."""
    fails = []
    rng = np.random.default_rng(9)
    R, B, K = 4, 16, 6
    L0 = np.array([10, 20, 40, 80], np.int32)
    max_seq = int(L0.max()) + steps
    orc = Oracle(num_layers=3, anchor_of=(0, 0, 2), R=R, B=B, K=K, rb=RB, max_seq=max_seq, lib=lib)
    for l in range(3):
        _fill_host(orc, L0, layer=l, tag=1000 if l else 0)   # layers 1 and 2 share contents
    orc.admit(0, np.arange(R), L0)
    orc.admit(2, np.arange(R), L0)
    for k in range(steps):
        L = L0 + 1 + k
        topk = np.stack([rng.choice(int(L[r]), size=K, replace=False) for r in range(R)]).astype(np.int32)
        for l in range(3):
            orc.store_newest(l, _new_kv(R, L, tag=5000), L)
        out0, plan0 = orc.swap_in(0, topk, L)
        orc.replay(1, plan0)
        out2, _ = orc.swap_in(2, topk, L)
        if not np.array_equal(out0, out2):
            fails.append(f"replay: step {k}: anchors with the same history disagree")
        for l in range(3):
            orc.backup(l, L)
        for r in range(R):
            for i in range(K):
                if not np.array_equal(orc.hot[1][r, out0[r, i]], orc.host[1][r, topk[r, i]]):
                    fails.append(f"replay: step {k} r {r}: replayed slot does not hold its position")
                    break
    for r in range(R):
        if not np.array_equal(orc.hot[1][r], orc.hot[2][r]):
            fails.append(f"replay: request {r}: replayed buffer differs from directly resolved one")
    return fails


def pin_preconditions(lib) -> List[str]:
    fails = []
    B, K = 8, 4
    orc = _tiny_oracle(lib, 1, B, K, 40)
    _fill_host(orc, [20])
    orc.admit(0, [0], [20])
    L = np.array([21], np.int32)
    for bad in ([1, 1, 2, 3], [1, 2, 3, 21], [1, 2, 3, -2], [40, 1, 2, 3]):
        try:
            orc.swap_in(0, np.array([bad], np.int32), L)
            fails.append(f"precondition: {bad} accepted")
        except OracleError as e:
            if e.rc != ORC_EPRECOND:
                fails.append(f"precondition: {bad} gave {e.rc}")
    try:
        orc.swap_in(0, np.array([[1, 2, 3, 4]], np.int32), np.array([41], np.int32))
        fails.append("precondition: L beyond the host pool accepted")
    except OracleError:
        pass
    orc.tok[0][0, :2] = 5
    try:
        orc.swap_in(0, np.array([[1, 2, 3, 4]], np.int32), L)
        fails.append("precondition: non-injective slot map accepted")
    except OracleError:
        pass
    try:
        orc.admit(0, [0], [41])
        fails.append("precondition: a prompt longer than the host pool admitted")
    except OracleError:
        pass
    return fails


# ---------------------------------------------------------------------------
# per-page residency
# ---------------------------------------------------------------------------
def pin_paged_hand_trace(lib) -> List[str]:
    with open(os.path.join(GOLDEN, "hand_worked_trace.json")) as f:
        g = json.load(f)
    fails = []
    for tr in g["paged_traces"]:
        B, K, L0, P = tr["B"], tr["K"], tr["L0"], tr["page_size"]
        orc = _tiny_oracle(lib, 1, B, K, L0 + len(tr["steps"]) + 1)
        _fill_host(orc, [L0])
        orc.admit(0, [0], [L0])
        bt = np.array([tr["block_row"]], np.int32)
        for k, st in enumerate(tr["steps"]):
            L = np.array([st["L"]], np.int32)
            orc.store_newest(0, _new_kv(1, L), L)
            out, plan = orc.swap_in_paged(0, np.array([st["topk"]], np.int32), L, bt, P, tr["hot_base"])
            orc.backup(0, L)
            got = dict(out=out[0].tolist(), lru=orc.lru[0][0].tolist(), tok=orc.tok[0][0].tolist(),
                       plan_pos=plan.pos[0, : plan.count[0]].tolist(),
                       plan_slot=plan.slot[0, : plan.count[0]].tolist())
            for key in got:
                if got[key] != st[key]:
                    fails.append(f"paged hand trace step {k}: {key} {got[key]} != {st[key]}")
    return fails


def _paged_setup(lib, R, B, K, P, L0, steps, frac, seed, n_phys_extra=7):
    """A cache, a block table with a seeded share `frac` of resident pages
    (distinct physical pages in a shuffled order), and a resident cache
    [n_phys*P][RB] holding the same KV as the host pool for resident pages."""
    rng = np.random.default_rng(seed)
    max_seq = int(L0.max()) + steps + 1
    max_pages = (max_seq + P - 1) // P
    orc = _tiny_oracle(lib, R, B, K, max_seq)
    _fill_host(orc, L0)
    orc.admit(0, np.arange(R), L0)
    n_res = int(round(frac * R * max_pages))
    flat = np.full(R * max_pages, -1, np.int32)
    chosen = rng.choice(R * max_pages, size=n_res, replace=False)
    n_phys = n_res + n_phys_extra
    flat[chosen] = rng.choice(n_phys, size=n_res, replace=False)
    bt = flat.reshape(R, max_pages)
    res_cache = np.zeros((n_phys * P, RB), np.uint8)
    for r in range(R):
        for pg in range(max_pages):
            if bt[r, pg] >= 0:
                for off in range(P):
                    t = pg * P + off
                    if t < max_seq:
                        res_cache[bt[r, pg] * P + off] = orc.host[0][r, t]
    return orc, bt, res_cache, rng, max_seq


def pin_paged_closed_forms(lib) -> List[str]:
    fails = []
    R, B, K, P = 3, 16, 6, 4
    L0 = np.array([10, 30, 60], np.int32)
    # every page resident: tier 0 answers everything, nothing else moves
    orc, _, _, rng, max_seq = _paged_setup(lib, R, B, K, P, L0, 3, 0.0, 1)
    max_pages = (max_seq + P - 1) // P
    bt = np.arange(R * max_pages, dtype=np.int32)[::-1].copy().reshape(R, max_pages)
    for k in range(3):
        L = L0 + 1 + k
        topk = np.stack([rng.choice(int(L[r]), K, replace=False) for r in range(R)]).astype(np.int32)
        lru0, tok0, hot0 = orc.lru[0].copy(), orc.tok[0].copy(), orc.hot[0].copy()
        out, plan = orc.swap_in_paged(0, topk, L, bt, P, 1000)
        exp = bt[np.arange(R)[:, None], topk // P] * P + topk % P
        if not np.array_equal(out, exp):
            fails.append(f"paged closed form: all-resident step {k}: out != page*P + t%P")
        if plan.count.any() or not np.array_equal(orc.lru[0], lru0) or not np.array_equal(orc.tok[0], tok0) \
                or not np.array_equal(orc.hot[0], hot0):
            fails.append(f"paged closed form: all-resident step {k}: state, plan or bytes changed")
    # no page resident: the per-request resolver, shifted into the caller's row view
    a, _, _, rng, _ = _paged_setup(lib, R, B, K, P, L0, 5, 0.0, 2)
    b, _, _, _, _ = _paged_setup(lib, R, B, K, P, L0, 5, 0.0, 2)
    base = 77
    for k in range(5):
        L = L0 + 1 + k
        topk = np.stack([rng.choice(int(L[r]), K, replace=False) for r in range(R)]).astype(np.int32)
        for o in (a, b):
            o.store_newest(0, _new_kv(R, L), L)
        oa, pa = a.swap_in_paged(0, topk, L, None, P, base)
        ob, pb = b.swap_in(0, topk, L)
        exp = np.where(ob >= 0, base + np.arange(R)[:, None] * (B + 1) + ob, -1)
        if not np.array_equal(oa, exp) or not np.array_equal(pa.count, pb.count):
            fails.append(f"paged closed form: no-resident step {k}: differs from the per-request resolver")
        if not (np.array_equal(a.lru[0], b.lru[0]) and np.array_equal(a.tok[0], b.tok[0])):
            fails.append(f"paged closed form: no-resident step {k}: state differs")
        for o in (a, b):
            o.backup(0, L)
    return fails


def pin_paged_bytes(lib, steps: int = 10) -> List[str]:
    """The pages' correctness statement in the caller's combined row view
    (resident cache rows, then the hot rows): every resolved row holds the KV
    of the position asked for; resident positions never enter the slot map or
    the plan."""
    fails = []
    R, B, K, P = 5, 24, 10, 4
    L0 = np.array([15, 24, 40, 90, 200], np.int32)
    for frac in (0.2, 0.5, 0.8):
        orc, bt, res_cache, rng, max_seq = _paged_setup(lib, R, B, K, P, L0, steps, frac, 7)
        base = res_cache.shape[0]
        for k in range(steps):
            L = L0 + 1 + k
            topk = np.full((R, K), -1, np.int32)
            for r in range(R):
                n = min(K, int(L[r]))
                hi = int(L[r])
                lo = max(0, hi - 3 * K)
                topk[r, :n] = rng.choice(np.arange(lo, hi), n, replace=False) if hi - lo >= n else \
                    rng.choice(hi, n, replace=False)
            nk = _new_kv(R, L)
            orc.store_newest(0, nk, L)
            for r in range(R):          # the forward also writes a resident newest page
                pg = (int(L[r]) - 1) // P
                if bt[r, pg] >= 0:
                    res_cache[bt[r, pg] * P + (int(L[r]) - 1) % P] = nk[r]
            tok0 = orc.tok[0].copy()
            out, plan = orc.swap_in_paged(0, topk, L, bt, P, base)
            view = np.concatenate([res_cache, orc.hot[0].reshape(R * (B + 1), RB)])
            for r in range(R):
                for i in range(K):
                    t = int(topk[r, i])
                    if t < 0:
                        if out[r, i] != -1:
                            fails.append("paged bytes: padding not -1")
                        continue
                    want = nk[r] if t == L[r] - 1 else orc.host[0][r, t]
                    if not (0 <= out[r, i] < view.shape[0]) or not np.array_equal(view[out[r, i]], want):
                        fails.append(f"paged bytes frac {frac} step {k} r {r} i {i}: row {out[r, i]} "
                                     f"does not hold position {t}")
                        break
                    resident = bt[r, t // P] >= 0
                    if resident != (out[r, i] < base):
                        fails.append(f"paged bytes: position {t} resolved in the wrong tier")
                        break
                c = int(plan.count[r])
                if any(bt[r, int(t) // P] >= 0 for t in plan.pos[r, :c]):
                    fails.append(f"paged bytes: a resident position was copied")
                changed = orc.tok[0][r][orc.tok[0][r] != tok0[r]]
                if any(bt[r, int(t) // P] >= 0 for t in changed):
                    fails.append(f"paged bytes: a resident position entered the slot map")
            orc.backup(0, L)
            if len(fails) > 5:
                return fails
    return fails


# ---------------------------------------------------------------------------
# page transfers: spill and host import
# ---------------------------------------------------------------------------
def _paged_steps(orc, bt, res_cache, rng, L0, k0, steps, P, fails, label):
    """Paged resolve steps with the combined-view byte check."""
    R, K, B = orc.R, orc.K, orc.B
    base = res_cache.shape[0]
    for k in range(k0, k0 + steps):
        L = L0 + 1 + k
        topk = np.stack([rng.choice(int(L[r]), min(K, int(L[r])), replace=False) for r in range(R)]).astype(np.int32)
        nk = _new_kv(R, L)
        orc.store_newest(0, nk, L)
        for r in range(R):
            pg = (int(L[r]) - 1) // P
            if bt[r, pg] >= 0:
                res_cache[bt[r, pg] * P + (int(L[r]) - 1) % P] = nk[r]
        out, _ = orc.swap_in_paged(0, topk, L, bt, P, base)
        view = np.concatenate([res_cache, orc.hot[0].reshape(R * (B + 1), RB)])
        for r in range(R):
            for i in range(K):
                t = int(topk[r, i])
                want = nk[r] if t == L[r] - 1 else orc.host[0][r, t]
                if not np.array_equal(view[out[r, i]], want):
                    fails.append(f"{label}: step {k} r {r}: row {out[r, i]} does not hold position {t}")
                    return
        orc.backup(0, L)


def pin_spill_round_trip(lib) -> List[str]:
    """Spill resident pages to their host pages (whose old contents are
    poisoned first), mark them host-backed, keep resolving: every position
    still resolves to its KV, now through the hot tiers."""
    fails = []
    R, B, K, P, steps = 4, 24, 10, 4, 4
    L0 = np.array([30, 45, 70, 100], np.int32)
    orc, bt, res_cache, rng, max_seq = _paged_setup(lib, R, B, K, P, L0, 2 * steps + 1, 0.5, 21)
    _paged_steps(orc, bt, res_cache, rng, L0, 0, steps, P, fails, "spill (before)")
    rr, pp = np.nonzero(bt >= 0)
    pick = rng.choice(rr.size, size=rr.size // 2, replace=False)
    transfers = []
    for q in pick:
        r, pg = int(rr[q]), int(pp[q])
        lo, hi = pg * P, min(pg * P + P, max_seq)
        orc.host[0][r, lo:hi] = 0x5A                      # stale host page
        transfers.append((int(bt[r, pg]), r, pg, -1))
    before = orc.host[0].copy()
    orc.page_copy(0, P, res_cache, transfers)
    for sp, r, pg, _ in transfers:
        lo, hi = pg * P, min(pg * P + P, max_seq)
        if not np.array_equal(orc.host[0][r, lo:hi], res_cache[sp * P: sp * P + hi - lo]):
            fails.append(f"spill: host page {pg} of request {r} != resident page {sp}")
        before[r, lo:hi] = orc.host[0][r, lo:hi]
    if not np.array_equal(before, orc.host[0]):
        fails.append("spill: rows outside the spilled pages changed")
    for sp, r, pg, _ in transfers:
        bt[r, pg] = -1                                    # the table entry is replaced
    _paged_steps(orc, bt, res_cache, rng, L0, steps, steps, P, fails, "spill (after)")
    return fails


def pin_import_mirror(lib) -> List[str]:
    """Import staging pages into host pages (the last one past max_seq is cut),
    mirroring some into resident pages; mark the mirrored pages resident and
    keep resolving."""
    fails = []
    R, B, K, P, steps = 3, 16, 8, 8, 3
    L0 = np.array([20, 40, 60], np.int32)
    orc, bt, res_cache, rng, max_seq = _paged_setup(lib, R, B, K, P, L0, steps + 1, 0.0, 22, n_phys_extra=12)
    max_pages = bt.shape[1]
    staging = rng.integers(0, 256, size=(10 * P, RB), dtype=np.uint8)
    transfers, mirrored = [], []
    for x, (r, pg) in enumerate([(0, 0), (0, 2), (1, 1), (1, 3), (2, 0), (2, max_pages - 1), (0, 1)]):
        mp = x if x % 2 == 0 else -1
        transfers.append((x, r, pg, mp))
        if mp >= 0:
            mirrored.append((r, pg, mp))
    before = orc.host[0].copy()
    orc.page_copy(0, P, staging, transfers, mirror=res_cache)
    for sp, r, pg, mp in transfers:
        lo, hi = pg * P, min(pg * P + P, max_seq)
        want = staging[sp * P: sp * P + hi - lo]
        if not np.array_equal(orc.host[0][r, lo:hi], want):
            fails.append(f"import: host page {pg} of request {r} != staging page {sp}")
        if mp >= 0 and not np.array_equal(res_cache[mp * P: mp * P + hi - lo], want):
            fails.append(f"import: mirror page {mp} != staging page {sp}")
        before[r, lo:hi] = orc.host[0][r, lo:hi]
    if not np.array_equal(before, orc.host[0]):
        fails.append("import: rows outside the imported pages changed")
    for r, pg, mp in mirrored:
        bt[r, pg] = mp
    _paged_steps(orc, bt, res_cache, rng, L0, 0, steps, P, fails, "import")
    try:
        orc.page_copy(0, P, staging, [(0, R, 0, -1)])
        fails.append("import: request out of range accepted")
    except OracleError:
        pass
    try:
        orc.page_copy(0, P, staging, [(0, 0, max_pages, -1)])
        fails.append("import: host page past the pool accepted")
    except OracleError:
        pass
    return fails


# cheapest first: a planted mistake is usually caught within milliseconds
ALL_PINS = {
    "hand_trace": pin_hand_trace,
    "closed_forms": pin_closed_forms,
    "invariants": pin_invariants,
    "replay": pin_replay,
    "preconditions": pin_preconditions,
    "paged_hand_trace": pin_paged_hand_trace,
    "paged_closed_forms": pin_paged_closed_forms,
    "paged_bytes": pin_paged_bytes,
    "spill_round_trip": pin_spill_round_trip,
    "import_mirror": pin_import_mirror,
    "textbook_lru_random": pin_textbook_lru_random,
    "textbook_lru_exhaustive": pin_textbook_lru_exhaustive,
}
