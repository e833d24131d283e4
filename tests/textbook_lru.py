"""Independent brute-force models that pin the oracle.

``TextbookLRU`` is a textbook LRU cache built on ``collections.OrderedDict``:
keys are token positions, values are device-buffer slots, iteration order is
recency (least recent first).  It knows nothing of the oracle's partition
formula; a decode step is fed to it as a reference string of accesses:

  * the entries already cached (hits) are touched in their prior recency
    order (``move_to_end``), then
  * the remaining entries (misses) are inserted in ascending top-k index, each
    evicting the least recent key (``popitem(last=False)``) and taking over
    its slot.

Under the readings the oracle takes (victims from the LRU end in order,
misses in ascending top-k index, a stable reorder), its state after every
step must equal this cache's.  The fast path (sequence not longer than the
buffer), the resident tier, padding (-1) and the newest token (row B) are
outside the cache, as the SGLang guide's "Decode Workflow" and the vLLM
design note's "Hot lookup and LRU" describe.

``BytesModel`` tracks KV rows as a dict position -> bytes and is used for the
pages' own correctness statement: every resolved slot must hold the bytes of
the position it was asked for.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import List, Sequence, Tuple


class TextbookLRU:
    def __init__(self, B: int, L0: int):
        self.B = B
        self.od: "OrderedDict[object, int]" = OrderedDict()
        for s in range(B):
            key = s if L0 <= B else ("empty", s)   # placeholder keys never equal a token
            self.od[key] = s

    def step(self, topk: Sequence[int], L: int) -> List[int]:
        B = self.B
        if L <= B:
            return [int(t) for t in topk]          # slot = position; cache untouched
        out: List = [None] * len(topk)
        hit_keys = set()
        for i, t in enumerate(topk):
            t = int(t)
            if t < 0:
                out[i] = -1
            elif t == L - 1:
                out[i] = B
            elif t in self.od:
                out[i] = self.od[t]
                hit_keys.add(t)
        for key in [k for k in self.od if k in hit_keys]:
            self.od.move_to_end(key)
        for i, t in enumerate(topk):
            if out[i] is None:
                _, slot = self.od.popitem(last=False)
                self.od[int(t)] = slot
                out[i] = slot
        return out

    def state(self) -> Tuple[List[int], List[int]]:
        lru = list(self.od.values())
        tok = [-1] * self.B
        for key, slot in self.od.items():
            if isinstance(key, int):
                tok[slot] = key
        return lru, tok
