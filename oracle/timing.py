"""CPU-baseline timing of the oracle: a whole decode run, in C, over disjoint
request shares on POSIX threads.

TEST INFRASTRUCTURE ONLY (the benchmark's CPU-baseline leg and its test).
``liboracle_timing.so`` holds ``oracle_timing.c`` with its own build of the
unchanged ``hisparse_oracle.c``; the timed loop calls the oracle's functions
in the order of one decode step and never returns to Python between steps.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Sequence

import numpy as np

from oracle.runner import OracleRun

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_timing.so")
SRCS = (os.path.join(HERE, "hisparse_oracle.c"), os.path.join(HERE, "oracle_timing.c"))


def build_timing(out: str = LIB) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread", "-I", HERE,
           *SRCS, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class orc_decode(ctypes.Structure):
    _fields_ = [
        ("layers", _I32), ("R", _I32), ("B", _I32), ("K", _I32), ("max_seq", _I32), ("spec", _I32),
        ("rb", _I64),
        ("anchor_of", _P), ("host", _P), ("hot", _P), ("lru", _P), ("tok", _P),
        ("L0", _P), ("resident", _P), ("block_table", _P),
        ("max_pages", _I32), ("page_size", _I32),
        ("hot_row_base", _I64),
        ("n_steps", _I32), ("first_timed", _I32),
        ("topk", _P), ("new_kv", _P), ("seq_lens", _P),
    ]


def load_timing(path: str = LIB) -> ctypes.CDLL:
    if not os.path.exists(path):
        build_timing(path)
    lib = ctypes.CDLL(path)
    lib.orc_time_decode.argtypes = [ctypes.POINTER(orc_decode), _I32, ctypes.POINTER(ctypes.c_double)]
    lib.orc_time_decode.restype = ctypes.c_int
    return lib


class DecodeTimer:
    """Times steps [first_timed, n_steps) of a decode on an OracleRun's
    buffers (its host pools, hot buffers and LRU state), each call re-admitting
    every request first, so each call repeats the same decode.

    topk_all[k]: {anchor: [S][R][K] int32}; newkv_all[k]: [layers][R][rb]."""

    def __init__(self, run: OracleRun, topk_all: Sequence[Dict[int, np.ndarray]],
                 newkv_all: Sequence[np.ndarray], first_timed: int, lib=None):
        from decode_memory_tiering_amd import workload as W
        wl, orc = run.wl, run.orc
        self.lib = lib if lib is not None else load_timing()
        n = len(topk_all)
        S, R, K = wl.spec, wl.R, wl.K
        topk = np.zeros((n, wl.num_layers, S, R, K), np.int32)
        for k, t in enumerate(topk_all):
            for a, v in t.items():
                topk[k, a] = v
        self._keep: List[object] = []
        self.topk = topk
        self.new_kv = np.ascontiguousarray(np.stack([np.asarray(x, np.uint8) for x in newkv_all]))
        assert self.new_kv.shape == (n, wl.num_layers, R, wl.rb)
        self.seq_lens = np.ascontiguousarray(np.stack([W.seq_lens_at(wl, k) for k in range(n)]).astype(np.int32))
        self.L0 = np.ascontiguousarray(run.L0.astype(np.int32))
        self.anchor_of = np.asarray(wl.anchor_of, np.int32)
        L = wl.num_layers
        self.host = (_P * L)(*[h.ctypes.data for h in orc.host])
        self.hot = (_P * L)(*[h.ctypes.data for h in orc.hot])
        self.lru = (_P * L)(*[orc.lru[l].ctypes.data if l in orc.lru else None for l in range(L)])
        self.tok = (_P * L)(*[orc.tok[l].ctypes.data if l in orc.tok else None for l in range(L)])
        res = run.resident if run.resident.any() else None
        self.resident = None if res is None else np.ascontiguousarray(res.astype(np.uint8))
        paged = wl.page_size > 0
        self.block_table = np.ascontiguousarray(run.block_table.astype(np.int32)) if paged else None
        d = orc_decode()
        d.layers, d.R, d.B, d.K, d.max_seq, d.spec, d.rb = L, R, wl.B, K, orc.max_seq, S, wl.rb
        d.anchor_of = self.anchor_of.ctypes.data
        d.host, d.hot, d.lru, d.tok = (ctypes.cast(x, _P) for x in (self.host, self.hot, self.lru, self.tok))
        d.L0 = self.L0.ctypes.data
        d.resident = None if self.resident is None else self.resident.ctypes.data
        d.block_table = None if self.block_table is None else self.block_table.ctypes.data
        d.max_pages = 0 if self.block_table is None else self.block_table.shape[1]
        d.page_size = wl.page_size if paged else 0
        d.hot_row_base = run.hot_row_base if paged else 0
        d.n_steps, d.first_timed = n, first_timed
        d.topk, d.new_kv, d.seq_lens = self.topk.ctypes.data, self.new_kv.ctypes.data, self.seq_lens.ctypes.data
        self.d = d

    def run(self, threads: int) -> float:
        """One repetition on `threads` shares; returns the timed seconds."""
        sec = ctypes.c_double()
        rc = self.lib.orc_time_decode(ctypes.byref(self.d), int(threads), ctypes.byref(sec))
        if rc != 0:
            raise RuntimeError(f"orc_time_decode returned {rc}")
        return float(sec.value)
