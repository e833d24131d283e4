"""Python binding of ``libhisparse.so`` (the C ABI declared in include/hisparse.h).

Argument marshalling only: every step of the swap-in path runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and streams.  The
library must be built (``python -m decode_memory_tiering_amd.build``); if it
is missing, loading fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhisparse.so")

HISPARSE_OK = 0
HISPARSE_EINVAL = -22
HISPARSE_ENOMEM = -12
HISPARSE_EBUSY = -16
HISPARSE_ENOSPC = -28

HISPARSE_DERR_TOPK_RANGE = 0x1
HISPARSE_DERR_TOPK_DUP = 0x2
HISPARSE_DERR_SEQ_LEN = 0x4
HISPARSE_DERR_REQ_IDX = 0x8
HISPARSE_DERR_STATE = 0x10
HISPARSE_DERR_PLAN = 0x20
HISPARSE_DERR_PAGE = 0x40

HISPARSE_STAT_ENTRIES, HISPARSE_STAT_RESIDENT, HISPARSE_STAT_FAST = 0, 1, 2
HISPARSE_STAT_NEWEST, HISPARSE_STAT_HIT, HISPARSE_STAT_MISS = 3, 4, 5
HISPARSE_STAT_COUNT = 6

HISPARSE_HOST_DEFAULT = 0
HISPARSE_HOST_COHERENT = 1
HISPARSE_HOST_NONCOHERENT = 2

# every entry point include/hisparse.h declares
EXPORTS = (
    "hisparse_init", "hisparse_init_static", "hisparse_static_scratch_bytes", "hisparse_destroy",
    "hisparse_admit", "hisparse_store_newest",
    "hisparse_swap_in", "hisparse_store_swap_in", "hisparse_store_swap_in_backup", "hisparse_swap_in_paged",
    "hisparse_store_swap_in_paged_backup",
    "hisparse_replay_plan", "hisparse_backup", "hisparse_spill", "hisparse_import", "hisparse_spill_dma",
    "hisparse_import_dma", "hisparse_get_state",
    "hisparse_set_state", "hisparse_set_stats", "hisparse_get_error", "hisparse_host_alloc", "hisparse_host_free",
    "hisparse_swap_in_lds_bytes", "hisparse_strerror", "hisparse_version",
)


class HisparseError(RuntimeError):
    def __init__(self, rc: int, what: str):
        self.rc = rc
        msg = _lib().hisparse_strerror(rc).decode() if _LIB is not None else str(rc)
        super().__init__(f"{what} failed: {rc} ({msg})")


class hisparse_config(ctypes.Structure):
    _fields_ = [
        ("top_k", ctypes.c_int32),
        ("device_buffer_size", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("max_requests", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("row_bytes", ctypes.c_int32),
        ("host_pool", ctypes.POINTER(ctypes.c_void_p)),
        ("hot_buffer", ctypes.POINTER(ctypes.c_void_p)),
        ("anchor_of", ctypes.POINTER(ctypes.c_int32)),
        ("block_size", ctypes.c_int32),
        ("replay_grid", ctypes.c_int32),
    ]


class hisparse_plan(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_void_p), ("slot", ctypes.c_void_p), ("count", ctypes.c_void_p)]


_LIB: Optional[ctypes.CDLL] = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m decode_memory_tiering_amd.build` "
                           "(the HiSparse path has no fallback)")
    # torch first: its HIP runtime must be the one the library binds to (both
    # carry the same soname, and the first one loaded serves the process)
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I32, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
    lib.hisparse_init.argtypes = [ctypes.POINTER(hisparse_config), ctypes.POINTER(ctypes.c_void_p)]
    lib.hisparse_init_static.argtypes = [ctypes.POINTER(hisparse_config), ctypes.POINTER(ctypes.c_void_p)]
    lib.hisparse_static_scratch_bytes.argtypes = []
    lib.hisparse_static_scratch_bytes.restype = ctypes.c_size_t
    lib.hisparse_destroy.argtypes = [P]
    lib.hisparse_destroy.restype = None
    lib.hisparse_admit.argtypes = [P, I32, P, P, I32, P]
    lib.hisparse_store_newest.argtypes = [P, I32, P, P, P, P, I32, P]
    lib.hisparse_swap_in.argtypes = [P, I32, P, P, P, P, I32, P, hisparse_plan, P]
    lib.hisparse_store_swap_in.argtypes = [P, I32, P, P, P, P, P, I32, P, hisparse_plan, P]
    lib.hisparse_store_swap_in_backup.argtypes = [P, I32, P, P, P, P, P, I32, P, hisparse_plan, P]
    lib.hisparse_swap_in_paged.argtypes = [P, I32, P, P, P, I32, I32, I32, P, I32, P, hisparse_plan, P]
    lib.hisparse_store_swap_in_paged_backup.argtypes = [P, I32, P, P, P, P, I32, I32, I32, P, I32, P,
                                                        hisparse_plan, P]
    lib.hisparse_replay_plan.argtypes = [P, I32, hisparse_plan, P, I32, P]
    lib.hisparse_backup.argtypes = [P, I32, P, P, P, I32, P]
    lib.hisparse_spill.argtypes = [P, I32, P, I32, I32, P, I32, P]
    lib.hisparse_import.argtypes = [P, I32, P, I32, I32, P, I32, P, I32, P]
    lib.hisparse_spill_dma.argtypes = [P, I32, P, I32, I32, P, I32, P]
    lib.hisparse_import_dma.argtypes = [P, I32, P, I32, I32, P, I32, P, I32, P]
    lib.hisparse_get_state.argtypes = [P, I32, P, P, P]
    lib.hisparse_set_state.argtypes = [P, I32, P, P, P]
    lib.hisparse_set_stats.argtypes = [P, P]
    lib.hisparse_get_error.argtypes = [P, ctypes.POINTER(U32), ctypes.c_int, P]
    lib.hisparse_host_alloc.argtypes = [ctypes.c_size_t, U32, ctypes.POINTER(ctypes.c_void_p)]
    lib.hisparse_host_free.argtypes = [P]
    lib.hisparse_swap_in_lds_bytes.argtypes = [I32, I32]
    lib.hisparse_swap_in_lds_bytes.restype = ctypes.c_size_t
    lib.hisparse_strerror.argtypes = [ctypes.c_int]
    lib.hisparse_strerror.restype = ctypes.c_char_p
    lib.hisparse_version.argtypes = []
    for name in EXPORTS:
        fn = getattr(lib, name)
        if name not in ("hisparse_destroy", "hisparse_strerror", "hisparse_swap_in_lds_bytes",
                        "hisparse_static_scratch_bytes"):
            fn.restype = ctypes.c_int
    return lib


def _check(rc: int, what: str):
    if rc != HISPARSE_OK:
        raise HisparseError(rc, what)


def _ptr(t) -> Optional[int]:
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_contiguous(), "HiSparse buffers must be contiguous"
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class Plan:
    """One plan row on the device: pos / slot [nb][K], count [nb] (int32)."""
    pos: "torch.Tensor"
    slot: "torch.Tensor"
    count: "torch.Tensor"

    @classmethod
    def empty(cls, nb: int, K: int, device="cuda") -> "Plan":
        import torch
        return cls(torch.zeros(nb, K, dtype=torch.int32, device=device),
                   torch.zeros(nb, K, dtype=torch.int32, device=device),
                   torch.zeros(nb, dtype=torch.int32, device=device))

    def c(self) -> hisparse_plan:
        return hisparse_plan(_ptr(self.pos), _ptr(self.slot), _ptr(self.count))


# ---------------------------------------------------------------------------
# the C ABI, name for name
# ---------------------------------------------------------------------------
def hisparse_host_alloc(nbytes: int, flags: int = HISPARSE_HOST_DEFAULT) -> int:
    p = ctypes.c_void_p()
    _check(_lib().hisparse_host_alloc(nbytes, flags, ctypes.byref(p)), "hisparse_host_alloc")
    return int(p.value)


def hisparse_host_free(ptr: int) -> None:
    _check(_lib().hisparse_host_free(ptr), "hisparse_host_free")


def hisparse_init(*, top_k: int, device_buffer_size: int, num_layers: int, max_requests: int,
                  max_seq_len: int, row_bytes: int, host_pool: Sequence[int], hot_buffer: Sequence,
                  anchor_of: Sequence[int], block_size: int = 0, replay_grid: int = 0,
                  static_state: bool = False) -> int:
    """static_state: hisparse_init_static (state in the library's static
    scratch array, no allocation) instead of hisparse_init."""
    hp = (ctypes.c_void_p * len(host_pool))(*[int(p) for p in host_pool])
    hb = (ctypes.c_void_p * len(hot_buffer))(*[_ptr(t) for t in hot_buffer])
    an = (ctypes.c_int32 * len(anchor_of))(*[int(a) for a in anchor_of])
    cfg = hisparse_config(top_k, device_buffer_size, num_layers, max_requests, max_seq_len, row_bytes,
                          ctypes.cast(hp, ctypes.POINTER(ctypes.c_void_p)),
                          ctypes.cast(hb, ctypes.POINTER(ctypes.c_void_p)),
                          ctypes.cast(an, ctypes.POINTER(ctypes.c_int32)), block_size, replay_grid)
    ctx = ctypes.c_void_p()
    name = "hisparse_init_static" if static_state else "hisparse_init"
    _check(getattr(_lib(), name)(ctypes.byref(cfg), ctypes.byref(ctx)), name)
    return int(ctx.value)


def hisparse_static_scratch_bytes() -> int:
    return int(_lib().hisparse_static_scratch_bytes())


def hisparse_destroy(ctx: int) -> None:
    _lib().hisparse_destroy(ctx)


def hisparse_admit(ctx: int, anchor_layer: int, req_ids, seq_len0, stream=None) -> None:
    _check(_lib().hisparse_admit(ctx, anchor_layer, _ptr(req_ids), _ptr(seq_len0), int(req_ids.shape[0]),
                                 _stream(stream)), "hisparse_admit")


def hisparse_store_newest(ctx: int, layer: int, new_rows, seq_lens, resident_mask=None, req_idx=None,
                          stream=None) -> None:
    _check(_lib().hisparse_store_newest(ctx, layer, _ptr(new_rows), _ptr(seq_lens), _ptr(resident_mask),
                                        _ptr(req_idx), int(seq_lens.shape[0]), _stream(stream)),
           "hisparse_store_newest")


def hisparse_swap_in(ctx: int, anchor_layer: int, topk_idx, seq_lens, resident_mask, req_idx, out_slots,
                     plan: Plan, stream=None) -> None:
    _check(_lib().hisparse_swap_in(ctx, anchor_layer, _ptr(topk_idx), _ptr(seq_lens), _ptr(resident_mask),
                                   _ptr(req_idx), int(topk_idx.shape[0]), _ptr(out_slots), plan.c(),
                                   _stream(stream)), "hisparse_swap_in")


def hisparse_store_swap_in(ctx: int, anchor_layer: int, new_rows, topk_idx, seq_lens, resident_mask, req_idx,
                           out_slots, plan: Plan, stream=None) -> None:
    _check(_lib().hisparse_store_swap_in(ctx, anchor_layer, _ptr(new_rows), _ptr(topk_idx), _ptr(seq_lens),
                                         _ptr(resident_mask), _ptr(req_idx), int(topk_idx.shape[0]),
                                         _ptr(out_slots), plan.c(), _stream(stream)), "hisparse_store_swap_in")


def hisparse_store_swap_in_backup(ctx: int, anchor_layer: int, new_rows, topk_idx, seq_lens, resident_mask,
                                  req_idx, out_slots, plan: Plan, stream=None) -> None:
    _check(_lib().hisparse_store_swap_in_backup(ctx, anchor_layer, _ptr(new_rows), _ptr(topk_idx), _ptr(seq_lens),
                                                _ptr(resident_mask), _ptr(req_idx), int(topk_idx.shape[0]),
                                                _ptr(out_slots), plan.c(), _stream(stream)),
           "hisparse_store_swap_in_backup")


def hisparse_swap_in_paged(ctx: int, anchor_layer: int, topk_idx, seq_lens, block_table, page_size: int,
                           hot_row_base: int, req_idx, out_rows, plan: Plan, stream=None) -> None:
    max_pages = 0 if block_table is None else int(block_table.shape[1])
    _check(_lib().hisparse_swap_in_paged(ctx, anchor_layer, _ptr(topk_idx), _ptr(seq_lens), _ptr(block_table),
                                         max_pages, page_size, hot_row_base, _ptr(req_idx),
                                         int(topk_idx.shape[0]), _ptr(out_rows), plan.c(), _stream(stream)),
           "hisparse_swap_in_paged")


def hisparse_store_swap_in_paged_backup(ctx: int, anchor_layer: int, new_rows, topk_idx, seq_lens, block_table,
                                        page_size: int, hot_row_base: int, req_idx, out_rows, plan: Plan,
                                        stream=None) -> None:
    max_pages = 0 if block_table is None else int(block_table.shape[1])
    _check(_lib().hisparse_store_swap_in_paged_backup(ctx, anchor_layer, _ptr(new_rows), _ptr(topk_idx),
                                                      _ptr(seq_lens), _ptr(block_table), max_pages, page_size,
                                                      hot_row_base, _ptr(req_idx), int(topk_idx.shape[0]),
                                                      _ptr(out_rows), plan.c(), _stream(stream)),
           "hisparse_store_swap_in_paged_backup")


def hisparse_replay_plan(ctx: int, skip_layer: int, plan: Plan, req_idx=None, stream=None) -> None:
    _check(_lib().hisparse_replay_plan(ctx, skip_layer, plan.c(), _ptr(req_idx), int(plan.count.shape[0]),
                                       _stream(stream)), "hisparse_replay_plan")


def hisparse_backup(ctx: int, layer: int, seq_lens, resident_mask=None, req_idx=None, stream=None) -> None:
    _check(_lib().hisparse_backup(ctx, layer, _ptr(seq_lens), _ptr(resident_mask), _ptr(req_idx),
                                  int(seq_lens.shape[0]), _stream(stream)), "hisparse_backup")


def hisparse_spill(ctx: int, layer: int, resident_cache, page_size: int, transfers, stream=None) -> None:
    pages = int(resident_cache.shape[0]) // page_size
    _check(_lib().hisparse_spill(ctx, layer, _ptr(resident_cache), pages, page_size, _ptr(transfers),
                                 int(transfers.shape[0]), _stream(stream)), "hisparse_spill")


def hisparse_import(ctx: int, layer: int, staging, page_size: int, resident_cache, transfers, stream=None) -> None:
    rpages = 0 if resident_cache is None else int(resident_cache.shape[0]) // page_size
    _check(_lib().hisparse_import(ctx, layer, _ptr(staging), int(staging.shape[0]) // page_size, page_size,
                                  _ptr(resident_cache), rpages, _ptr(transfers), int(transfers.shape[0]),
                                  _stream(stream)), "hisparse_import")


def _host_transfers(transfers) -> np.ndarray:
    t = np.ascontiguousarray(np.asarray(transfers, dtype=np.int32).reshape(-1, 4))
    return t


def hisparse_spill_dma(ctx: int, layer: int, resident_cache, page_size: int, transfers, stream=None) -> None:
    """transfers: host array [n][4] (numpy or CPU tensor)."""
    pages = int(resident_cache.shape[0]) // page_size
    t = _host_transfers(transfers)
    _check(_lib().hisparse_spill_dma(ctx, layer, _ptr(resident_cache), pages, page_size, t.ctypes.data,
                                     int(t.shape[0]), _stream(stream)), "hisparse_spill_dma")


def hisparse_import_dma(ctx: int, layer: int, staging, page_size: int, resident_cache, transfers,
                        stream=None) -> None:
    """transfers: host array [n][4] (numpy or CPU tensor)."""
    rpages = 0 if resident_cache is None else int(resident_cache.shape[0]) // page_size
    t = _host_transfers(transfers)
    _check(_lib().hisparse_import_dma(ctx, layer, _ptr(staging), int(staging.shape[0]) // page_size, page_size,
                                      _ptr(resident_cache), rpages, t.ctypes.data, int(t.shape[0]),
                                      _stream(stream)), "hisparse_import_dma")


def hisparse_get_state(ctx: int, anchor_layer: int, lru, slot_tok, stream=None) -> None:
    _check(_lib().hisparse_get_state(ctx, anchor_layer, _ptr(lru), _ptr(slot_tok), _stream(stream)),
           "hisparse_get_state")


def hisparse_set_state(ctx: int, anchor_layer: int, lru, slot_tok, stream=None) -> None:
    _check(_lib().hisparse_set_state(ctx, anchor_layer, _ptr(lru), _ptr(slot_tok), _stream(stream)),
           "hisparse_set_state")


def hisparse_set_stats(ctx: int, stats) -> None:
    """stats: device tensor [R][HISPARSE_STAT_COUNT] int64 (read as uint64), or None."""
    _check(_lib().hisparse_set_stats(ctx, _ptr(stats)), "hisparse_set_stats")


def hisparse_get_error(ctx: int, clear: bool = True, stream=None) -> int:
    v = ctypes.c_uint32()
    _check(_lib().hisparse_get_error(ctx, ctypes.byref(v), int(clear), _stream(stream)), "hisparse_get_error")
    return int(v.value)


def hisparse_swap_in_lds_bytes(top_k: int, device_buffer_size: int) -> int:
    return int(_lib().hisparse_swap_in_lds_bytes(top_k, device_buffer_size))


def hisparse_strerror(code: int) -> str:
    return _lib().hisparse_strerror(code).decode()


def hisparse_version() -> int:
    return int(_lib().hisparse_version())


# ---------------------------------------------------------------------------
# the serving config's JSON keys
# ---------------------------------------------------------------------------
def parse_hisparse_config(text_or_dict) -> dict:
    """Keyword arguments for HiSparseCache from the JSON keys of SGLang's
    --hisparse-config (SGLang guide "HiSparse: Hierarchical Sparse
    Attention", "HiSparse Config Parameters"): top_k -> K,
    device_buffer_size -> B, swap_in_block_size -> the swap-in workgroup
    size (a multiple of 64 in [128, 1024]; the guide's 960 is one).
    host_to_device_ratio sizes the host pool in a serving system; here the
    caller sizes it through max_seq, so the key is accepted and ignored."""
    import json
    cfg = json.loads(text_or_dict) if isinstance(text_or_dict, str) else dict(text_or_dict)
    known = {"top_k", "device_buffer_size", "host_to_device_ratio", "swap_in_block_size"}
    unknown = set(cfg) - known
    if unknown:
        raise ValueError(f"unknown hisparse-config keys: {sorted(unknown)}")
    if "top_k" not in cfg or "device_buffer_size" not in cfg:
        raise ValueError("hisparse-config needs top_k and device_buffer_size")
    out = dict(K=int(cfg["top_k"]), B=int(cfg["device_buffer_size"]))
    bs = int(cfg.get("swap_in_block_size", 0))
    if bs and (bs % 64 or not 128 <= bs <= 1024):
        raise ValueError(f"swap_in_block_size {bs}: needs a multiple of 64 in [128, 1024] (wave64)")
    if bs:
        out["block_size"] = bs
    if int(out["K"]) > int(out["B"]):
        raise ValueError("top_k must not exceed device_buffer_size")
    return out


# ---------------------------------------------------------------------------
# a cache object: pinned host pools + device hot buffers + a context
# ---------------------------------------------------------------------------
def host_array(ptr: int, shape) -> np.ndarray:
    """numpy view of pinned host memory (no copy)."""
    n = int(np.prod(shape))
    buf = (ctypes.c_uint8 * n).from_address(ptr)
    return np.ctypeslib.as_array(buf).reshape(shape)


class HiSparseCache:
    """One HiSparse cache: per-layer pinned host pools [R][max_seq][rb] (owned,
    allocated with hisparse_host_alloc), per-layer device hot buffers
    [R][B+1][rb] (torch), and the library context."""

    def __init__(self, *, num_layers: int, anchor_of: Sequence[int], R: int, B: int, K: int, rb: int,
                 max_seq: int, device="cuda", host_flags: int = HISPARSE_HOST_DEFAULT,
                 block_size: int = 0, replay_grid: int = 0, static_state: bool = False):
        import torch
        self.num_layers, self.R, self.B, self.K, self.rb, self.max_seq = num_layers, R, B, K, rb, max_seq
        self.anchor_of = [int(a) for a in anchor_of]
        self.device = torch.device(device)
        self._host_ptrs: List[int] = []
        self.ctx = 0
        nbytes = R * max_seq * rb
        for _ in range(num_layers):
            self._host_ptrs.append(hisparse_host_alloc(nbytes, host_flags))
        self.host_np = [host_array(p, (R, max_seq, rb)) for p in self._host_ptrs]
        self.host = [torch.from_numpy(a) for a in self.host_np]          # CPU views, same memory
        self.hot = [torch.zeros(R, B + 1, rb, dtype=torch.uint8, device=self.device)
                    for _ in range(num_layers)]
        self.ctx = hisparse_init(top_k=K, device_buffer_size=B, num_layers=num_layers, max_requests=R,
                                 max_seq_len=max_seq, row_bytes=rb, host_pool=self._host_ptrs,
                                 hot_buffer=self.hot, anchor_of=self.anchor_of, block_size=block_size,
                                 replay_grid=replay_grid, static_state=static_state)

    def close(self):
        if self.ctx:
            hisparse_destroy(self.ctx)
            self.ctx = 0
        self.host, self.host_np = [], []
        for p in self._host_ptrs:
            hisparse_host_free(p)
        self._host_ptrs = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # thin forwards
    def admit(self, anchor, req_ids, seq_len0, stream=None):
        hisparse_admit(self.ctx, anchor, req_ids, seq_len0, stream)

    def store_newest(self, layer, new_rows, seq_lens, resident_mask=None, req_idx=None, stream=None):
        hisparse_store_newest(self.ctx, layer, new_rows, seq_lens, resident_mask, req_idx, stream)

    def swap_in(self, anchor, topk_idx, seq_lens, resident_mask, req_idx, out_slots, plan, stream=None):
        hisparse_swap_in(self.ctx, anchor, topk_idx, seq_lens, resident_mask, req_idx, out_slots, plan, stream)

    def store_swap_in(self, anchor, new_rows, topk_idx, seq_lens, resident_mask, req_idx, out_slots, plan,
                      stream=None):
        hisparse_store_swap_in(self.ctx, anchor, new_rows, topk_idx, seq_lens, resident_mask, req_idx, out_slots,
                               plan, stream)

    def store_swap_in_backup(self, anchor, new_rows, topk_idx, seq_lens, resident_mask, req_idx, out_slots, plan,
                             stream=None):
        hisparse_store_swap_in_backup(self.ctx, anchor, new_rows, topk_idx, seq_lens, resident_mask, req_idx,
                                      out_slots, plan, stream)

    def swap_in_paged(self, anchor, topk_idx, seq_lens, block_table, page_size, hot_row_base, req_idx, out_rows,
                      plan, stream=None):
        hisparse_swap_in_paged(self.ctx, anchor, topk_idx, seq_lens, block_table, page_size, hot_row_base,
                               req_idx, out_rows, plan, stream)

    def store_swap_in_paged_backup(self, anchor, new_rows, topk_idx, seq_lens, block_table, page_size,
                                   hot_row_base, req_idx, out_rows, plan, stream=None):
        hisparse_store_swap_in_paged_backup(self.ctx, anchor, new_rows, topk_idx, seq_lens, block_table, page_size,
                                            hot_row_base, req_idx, out_rows, plan, stream)

    def replay_plan(self, skip_layer, plan, req_idx=None, stream=None):
        hisparse_replay_plan(self.ctx, skip_layer, plan, req_idx, stream)

    def backup(self, layer, seq_lens, resident_mask=None, req_idx=None, stream=None):
        hisparse_backup(self.ctx, layer, seq_lens, resident_mask, req_idx, stream)

    def spill(self, layer, resident_cache, page_size, transfers, stream=None):
        hisparse_spill(self.ctx, layer, resident_cache, page_size, transfers, stream)

    def import_pages(self, layer, staging, page_size, resident_cache, transfers, stream=None):
        hisparse_import(self.ctx, layer, staging, page_size, resident_cache, transfers, stream)

    def spill_dma(self, layer, resident_cache, page_size, transfers, stream=None):
        hisparse_spill_dma(self.ctx, layer, resident_cache, page_size, transfers, stream)

    def import_pages_dma(self, layer, staging, page_size, resident_cache, transfers, stream=None):
        hisparse_import_dma(self.ctx, layer, staging, page_size, resident_cache, transfers, stream)

    def get_state(self, anchor, stream=None):
        import torch
        lru = torch.empty(self.R, self.B, dtype=torch.int32, device=self.device)
        tok = torch.empty_like(lru)
        hisparse_get_state(self.ctx, anchor, lru, tok, stream)
        return lru, tok

    def set_state(self, anchor, lru, tok, stream=None):
        hisparse_set_state(self.ctx, anchor, lru, tok, stream)

    def set_stats(self, stats):
        hisparse_set_stats(self.ctx, stats)

    def get_error(self, clear=True, stream=None) -> int:
        return hisparse_get_error(self.ctx, clear, stream)
