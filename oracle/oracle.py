"""CPU oracle of the HiSparse decode-step swap-in resolver (Python side).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the product path never imports it.  It loads
``liboracle.so`` built from ``hisparse_oracle.c`` with gcc, and keeps the
oracle's own copies of every buffer in plain numpy host arrays, so nothing it
computes passes through the HIP library.

The method it follows is stated on two pages:
  * SGLang guide "HiSparse: Hierarchical Sparse Attention", sections
    "Decode Workflow" and "Shared-index prefetch";
  * vLLM design note "HiSparse local KV offload architecture", sections
    "Resident device pages", "Hot lookup and LRU" and "Performance invariants".
The C source lists each reading taken where those pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hisparse_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

ORC_OK = 0
ORC_EINVAL = -22
ORC_ENOMEM = -12
ORC_EPRECOND = -2001


class OracleError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what}: oracle returned {rc}")
        self.rc = rc


def build_oracle(src: str = SRC, out: str = LIB, extra_flags: Sequence[str] = ()) -> str:
    """Compile the C oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           "-I", HERE, *extra_flags, src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def load_oracle(path: str = LIB) -> ctypes.CDLL:
    if not os.path.exists(path):
        build_oracle(out=path)
    lib = ctypes.CDLL(path)
    lib.orc_newest_row.argtypes = [_I32, _I32]
    lib.orc_newest_row.restype = _I32
    lib.orc_admit_state.argtypes = [_I32, _I32, _P, _P]
    lib.orc_admit_fill.argtypes = [_I32, _I32, _I64, _P, _P]
    lib.orc_store_newest.argtypes = [_I32, _I32, _I64, _P, _P]
    lib.orc_swap_in_row.argtypes = [_I32, _I32, _I64, _I32, _I32, _I32,
                                    _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.orc_swap_in.argtypes = [_I32, _I32, _I32, _I64, _I32, _I32, _P,
                                _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.orc_swap_in_paged.argtypes = [_I32, _I32, _I32, _I64, _I32, _I32, _P,
                                      _P, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.orc_page_copy.argtypes = [_I32, _I32, _I64, _I32, _P, _I32, _P, _P, _I32, _I32, _P]
    lib.orc_replay.argtypes = [_I32, _I32, _I32, _I64, _I32, _I32, _P,
                               _P, _P, _P, _P, _P]
    lib.orc_backup.argtypes = [_I32, _I32, _I64, _I32, _I32, _P, _P, _P, _P, _P]
    for fn in ("orc_admit_state", "orc_admit_fill", "orc_store_newest",
               "orc_swap_in_row", "orc_swap_in", "orc_swap_in_paged", "orc_page_copy", "orc_replay", "orc_backup"):
        getattr(lib, fn).restype = ctypes.c_int
    return lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


@dataclass
class Plan:
    """One plan row: pairs (host position, device slot) in ascending top-k
    index; entries at or beyond count[b] are unspecified."""
    pos: np.ndarray    # [nb][K] int32
    slot: np.ndarray   # [nb][K] int32
    count: np.ndarray  # [nb] int32


class Oracle:
    """Host-memory model of one HiSparse cache with ``num_layers`` layers.

    host[l]  : [R][max_seq][rb] uint8   (full KV, the pinned pool's stand-in)
    hot[l]   : [R][B+1][rb] uint8       (per-request device buffer + newest row)
    lru[g], tok[g] : [R][B] int32, only for anchor layers g (anchor_of[g] == g)
    """

    def __init__(self, *, num_layers: int, anchor_of: Sequence[int], R: int, B: int,
                 K: int, rb: int, max_seq: int, lib: Optional[ctypes.CDLL] = None,
                 allocate_host: bool = True):
        if len(anchor_of) != num_layers:
            raise ValueError("anchor_of needs one entry per layer")
        self.lib = lib if lib is not None else load_oracle()
        self.L, self.R, self.B, self.K, self.rb, self.max_seq = num_layers, R, B, K, rb, max_seq
        self.anchor_of = [int(a) for a in anchor_of]
        self.host: List[np.ndarray] = [
            np.zeros((R, max_seq, rb), np.uint8) if allocate_host else None
            for _ in range(num_layers)]
        self.hot: List[np.ndarray] = [np.zeros((R, B + 1, rb), np.uint8)
                                      for _ in range(num_layers)]
        self.lru: Dict[int, np.ndarray] = {}
        self.tok: Dict[int, np.ndarray] = {}
        for g in sorted(set(self.anchor_of)):
            if self.anchor_of[g] != g:
                raise ValueError(f"layer {g} is named as an anchor but is not its own anchor")
            self.lru[g] = np.tile(np.arange(B, dtype=np.int32), (R, 1))
            self.tok[g] = np.full((R, B), -1, np.int32)

    # -- helpers -----------------------------------------------------------
    def _check(self, rc: int, what: str):
        if rc != ORC_OK:
            raise OracleError(rc, what)

    def newest_row(self, L: int) -> int:
        return int(self.lib.orc_newest_row(self.B, int(L)))

    # -- admission ---------------------------------------------------------
    def admit(self, anchor: int, req_ids, seq_len0):
        req_ids = _i32(req_ids)
        seq_len0 = _i32(seq_len0)
        for r, L0 in zip(req_ids.tolist(), seq_len0.tolist()):
            if L0 > self.max_seq:    # the prefill's rows must lie in the host pool
                raise OracleError(ORC_EPRECOND, "admit: prompt longer than the host pool")
            lru = np.empty(self.B, np.int32)
            tok = np.empty(self.B, np.int32)
            self._check(self.lib.orc_admit_state(self.B, L0, _ptr(lru), _ptr(tok)), "admit_state")
            self.lru[anchor][r] = lru
            self.tok[anchor][r] = tok
            for l in range(self.L):
                if self.anchor_of[l] != anchor:
                    continue
                self._check(self.lib.orc_admit_fill(
                    self.B, L0, self.rb, _ptr(self.host[l][r]), _ptr(self.hot[l][r])),
                    "admit_fill")

    # -- forward's KV write -------------------------------------------------
    def store_newest(self, layer: int, new_rows, seq_lens, resident=None, req_idx=None):
        new_rows = _u8(new_rows)
        seq_lens = _i32(seq_lens)
        nb = seq_lens.shape[0]
        for b in range(nb):
            if resident is not None and resident[b]:
                continue
            r = b if req_idx is None else int(req_idx[b])
            self._check(self.lib.orc_store_newest(
                self.B, int(seq_lens[b]), self.rb, _ptr(new_rows[b]), _ptr(self.hot[layer][r])),
                "store_newest")

    # -- the resolver --------------------------------------------------------
    def swap_in(self, anchor: int, topk, seq_lens, resident=None, req_idx=None):
        topk = _i32(topk)
        seq_lens = _i32(seq_lens)
        nb = topk.shape[0]
        assert topk.shape == (nb, self.K)
        res = _u8(resident) if resident is not None else None
        ridx = _i32(req_idx) if req_idx is not None else None
        out = np.empty((nb, self.K), np.int32)
        plan = Plan(np.full((nb, self.K), -7, np.int32), np.full((nb, self.K), -7, np.int32),
                    np.zeros(nb, np.int32))
        rc = self.lib.orc_swap_in(
            self.R, self.B, self.K, self.rb, self.max_seq, nb, _ptr(ridx),
            _ptr(topk), _ptr(seq_lens), _ptr(res), _ptr(out),
            _ptr(self.lru[anchor]), _ptr(self.tok[anchor]),
            _ptr(self.host[anchor]), _ptr(self.hot[anchor]),
            _ptr(plan.pos), _ptr(plan.slot), _ptr(plan.count))
        self._check(rc, "swap_in")
        return out, plan

    def swap_in_paged(self, anchor: int, topk, seq_lens, block_table, page_size: int,
                      hot_row_base: int = 0, req_idx=None):
        """Per-page residency: block_table [nb][max_pages] int32 (physical page
        or -1 for a host-backed page).  Returns physical rows in the caller's
        view: resident rows page*P + t%P, hot rows hot_row_base + r*(B+1) + slot."""
        topk = _i32(topk)
        seq_lens = _i32(seq_lens)
        nb = topk.shape[0]
        bt = _i32(block_table) if block_table is not None else None
        max_pages = 0 if bt is None else int(bt.shape[1])
        ridx = _i32(req_idx) if req_idx is not None else None
        out = np.empty((nb, self.K), np.int32)
        plan = Plan(np.full((nb, self.K), -7, np.int32), np.full((nb, self.K), -7, np.int32),
                    np.zeros(nb, np.int32))
        rc = self.lib.orc_swap_in_paged(
            self.R, self.B, self.K, self.rb, self.max_seq, nb, _ptr(ridx),
            _ptr(topk), _ptr(seq_lens), _ptr(bt), max_pages, int(page_size), int(hot_row_base), _ptr(out),
            _ptr(self.lru[anchor]), _ptr(self.tok[anchor]),
            _ptr(self.host[anchor]), _ptr(self.hot[anchor]),
            _ptr(plan.pos), _ptr(plan.slot), _ptr(plan.count))
        self._check(rc, "swap_in_paged")
        return out, plan

    def page_copy(self, layer: int, page_size: int, src: np.ndarray, transfers, mirror: Optional[np.ndarray] = None):
        """Spill / host import: src [src_pages*P][rb] (resident cache or
        staging pool) -> host pool pages, optionally mirrored into mirror
        [mirror_pages*P][rb].  transfers [n][4] = (src page, request, host
        page, mirror page or -1)."""
        tr = _i32(transfers).reshape(-1, 4)
        src = _u8(src)
        rc = self.lib.orc_page_copy(
            self.R, self.max_seq, self.rb, int(page_size), _ptr(src), src.shape[0] // page_size,
            _ptr(self.host[layer]), _ptr(mirror), 0 if mirror is None else mirror.shape[0] // page_size,
            tr.shape[0], _ptr(tr))
        self._check(rc, "page_copy")

    def replay(self, skip_layer: int, plan: Plan, req_idx=None):
        ridx = _i32(req_idx) if req_idx is not None else None
        nb = plan.count.shape[0]
        rc = self.lib.orc_replay(
            self.R, self.B, self.K, self.rb, self.max_seq, nb, _ptr(ridx),
            _ptr(_i32(plan.pos)), _ptr(_i32(plan.slot)), _ptr(_i32(plan.count)),
            _ptr(self.host[skip_layer]), _ptr(self.hot[skip_layer]))
        self._check(rc, "replay")

    def backup(self, layer: int, seq_lens, resident=None, req_idx=None):
        seq_lens = _i32(seq_lens)
        nb = seq_lens.shape[0]
        res = _u8(resident) if resident is not None else None
        ridx = _i32(req_idx) if req_idx is not None else None
        rc = self.lib.orc_backup(
            self.R, self.B, self.rb, self.max_seq, nb, _ptr(ridx), _ptr(seq_lens), _ptr(res),
            _ptr(self.hot[layer]), _ptr(self.host[layer]))
        self._check(rc, "backup")
