"""The allocation-free entry point hisparse_init_static against hisparse_init
(MI355X only).

A context from hisparse_init_static keeps its device state in the library's
static scratch array.  Two decodes in a row are run through it, the second on
a smaller configuration (so stale contents of the array from the first would
show), each against the same decode through a context from hisparse_init and
against the CPU oracle, bit for bit: slot ids, plan rows, LRU state and slot
maps after every step, every hot-buffer and host-pool byte at the end."""
import numpy as np
import pytest

from decode_memory_tiering_amd import workload as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_memory_tiering_amd.hisparse import load_library
    load_library()


FIRST = W.Workload("static_a", 3, (0, 0, 2), R=12, B=1024, K=256, rb=96, steps=8, n_resident=2,
                   seq_first=("uniform", 500, 6000), seed=51)
SECOND = W.Workload("static_b", 2, (0, 0), R=5, B=300, K=120, rb=48, steps=6, spec=2,
                    seq_first=("uniform", 100, 2000), seed=52)


def _same(a, b):
    assert a.keys() == b.keys()
    for key in a:
        for x, y in zip(a[key], b[key]):
            if isinstance(x, tuple):
                for u, v in zip(x, y):
                    np.testing.assert_array_equal(u, v, err_msg=key)
            else:
                np.testing.assert_array_equal(x, y, err_msg=key)


def test_static_init_matches_init_on_two_decodes_in_a_row():
    from lockstep import run_lockstep
    for wl in (FIRST, SECOND):
        print(f"\n[no-alloc] {wl.name} R={wl.R} B={wl.B} K={wl.K} layers={wl.num_layers}", flush=True)
        heap, static = {}, {}
        run_lockstep(wl, keep=heap)
        run_lockstep(wl, static_state=True, keep=static)
        _same(heap, static)
        print(f"[no-alloc] {wl.name} ok", flush=True)


def test_static_init_limits():
    from decode_memory_tiering_amd.hisparse import (HISPARSE_EBUSY, HISPARSE_ENOSPC, HiSparseCache, HisparseError,
                                                    hisparse_static_scratch_bytes)
    cap = hisparse_static_scratch_bytes()
    assert cap == 32 << 20
    small = dict(num_layers=1, anchor_of=(0,), R=4, B=64, K=16, rb=32, max_seq=200)
    a = HiSparseCache(**small, static_state=True)
    try:
        # one static context per device at a time
        with pytest.raises(HisparseError) as e:
            HiSparseCache(**small, static_state=True)
        assert e.value.rc == HISPARSE_EBUSY
        b = HiSparseCache(**small)            # heap contexts are unaffected
        b.close()
    finally:
        a.close()
    # state of 2 anchors x 2 x R x B x 4 bytes beyond the array
    big = dict(num_layers=2, anchor_of=(0, 1), R=160, B=16384, K=16, rb=16, max_seq=16)
    assert 2 * 2 * 160 * 16384 * 4 > cap
    with pytest.raises(HisparseError) as e:
        HiSparseCache(**big, static_state=True)
    assert e.value.rc == HISPARSE_ENOSPC
    # a failed call leaves the slot free
    c = HiSparseCache(**small, static_state=True)
    c.close()
