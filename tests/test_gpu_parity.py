"""GPU parity: the HIP path against the CPU oracle, bit-exact (MI355X only).

Every test calls the HIP kernels through the C ABI (the Python binding only
marshals arguments) and compares with the oracle on the same seeded inputs:
slot ids, plan rows, LRU state and slot map after every step, the pages'
correctness statement on the gathered rows, and every byte of the hot
buffers and host pools at the end.  There is no floating point on the path,
so the bar is exact equality everywhere.
"""
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
    load_library()  # fails loudly when the HIP library is not built


def _lockstep(wl, **kw):
    from lockstep import run_lockstep
    print(f"\n[parity] {wl.name} R={wl.R} B={wl.B} K={wl.K} rb={wl.rb} layers={wl.num_layers} "
          f"steps={kw.get('steps', wl.steps)} block={kw.get('block_size', 0)}", flush=True)
    st = run_lockstep(wl, **kw)
    print(f"[parity] {wl.name} ok: {st}", flush=True)
    return st


# -- the five workloads at their full sizes --------------------------------------
def test_tiny_full():
    st = _lockstep(W.WORKLOADS["tiny"])
    assert st["misses"] > 0


def test_fastpath_mix_full():
    st = _lockstep(W.WORKLOADS["fastpath_mix"], progress=True)
    assert 0 < st["slow_rows"] < 64 * 32


@pytest.mark.timeout(900)
def test_dsv32_decode_full():
    _lockstep(W.WORKLOADS["dsv32_decode"], progress=True, compare_state_every=4)


@pytest.mark.timeout(900)
def test_indexshare_full_prefetch():
    _lockstep(W.WORKLOADS["indexshare"], progress=True, prefetch=True, compare_state_every=4)


@pytest.mark.timeout(600)
def test_indexshare_inline_replay():
    _lockstep(W.WORKLOADS["indexshare"], steps=8, prefetch=False, progress=True)


@pytest.mark.timeout(600)
def test_long_context_full():
    st = _lockstep(W.WORKLOADS["long_context"], progress=True)
    assert st["misses"] > 0


# -- geometries spanning several tiles with ragged tails, launch shapes --------------
RAGGED = [
    W.Workload("ragged_a", 2, (0, 1), R=7, B=1000, K=333, rb=48, steps=12, n_resident=2,
               seq_first=("uniform", 200, 3000), seed=11),
    W.Workload("ragged_b", 3, (0, 0, 2), R=5, B=777, K=777, rb=16, steps=10,
               seq_first=("uniform", 700, 2000), seed=12),
    W.Workload("ragged_c", 1, (0,), R=9, B=130, K=65, rb=656, steps=20, spec=2,
               seq_first=("uniform", 60, 600), row_format="fp8_656", seed=13),
    W.Workload("ragged_d", 1, (0,), R=3, B=4100, K=4096, rb=32, steps=6, topk_kind="uniform",
               seq_first=("uniform", 4000, 9000), seed=14),
]


def _cdiv(a, b):
    return (a + b - 1) // b


def _launch_shape_fits(wl, block):
    # 64-entry chunks of the LRU list / top-k row each wave holds in registers
    waves = block // 64
    return _cdiv(_cdiv(wl.B, 64), waves) <= 16 and _cdiv(_cdiv(wl.K, 64), waves) <= 4


def _assert_init_rejects(wl, block):
    """A workgroup too narrow for the buffer (more 64-entry chunks per wave
    than the kernel holds in registers): init refuses it on the host."""
    from decode_memory_tiering_amd.hisparse import HISPARSE_EINVAL, HiSparseCache, HisparseError
    print(f"\n[parity] {wl.name} B={wl.B} K={wl.K} block={block}: init must return EINVAL", flush=True)
    with pytest.raises(HisparseError) as e:
        c = HiSparseCache(num_layers=wl.num_layers, anchor_of=wl.anchor_of, R=wl.R, B=wl.B, K=wl.K, rb=wl.rb,
                          max_seq=W.max_seq(wl), block_size=block)
        c.close()
    assert e.value.rc == HISPARSE_EINVAL


@pytest.mark.parametrize("block", [128, 256, 1024])
@pytest.mark.parametrize("wl", RAGGED, ids=[w.name for w in RAGGED])
def test_ragged_geometries(wl, block):
    if not _launch_shape_fits(wl, block):
        _assert_init_rejects(wl, block)
        return
    _lockstep(wl, block_size=block)


@pytest.mark.parametrize("fuse", ["none", "store"])
@pytest.mark.parametrize("wl", [W.WORKLOADS["tiny"], RAGGED[0], RAGGED[2]], ids=["tiny", "ragged_a", "ragged_c"])
def test_separate_store_and_backup_launches(wl, fuse):
    # the forward's KV write and the eager backup as launches of their own
    # ("none"), or only the backup ("store": store_swap_in + backup)
    _lockstep(wl, fuse_store=fuse == "store", fuse_backup=False)


def test_fast_to_slow_transition():
    B = 512
    wl = W.Workload("transition", 1, (0,), R=6, B=B, K=128, rb=64, steps=8,
                    seq_first=("list", B - 3, B - 1, B, B + 1, B + 2, 2 * B), seed=21)
    _lockstep(wl)


def test_topk_equals_buffer_size():
    wl = W.Workload("k_eq_b", 1, (0,), R=4, B=256, K=256, rb=32, steps=10,
                    seq_first=("list", 200, 257, 300, 5000), seed=22)
    _lockstep(wl)


def test_single_slot_buffer():
    wl = W.Workload("b1", 1, (0,), R=3, B=1, K=1, rb=16, steps=8, topk_kind="uniform",
                    seq_first=("list", 1, 2, 9), seed=23)
    _lockstep(wl)


@pytest.mark.parametrize("flags", [1, 2])
def test_host_memory_kinds(flags):
    _lockstep(W.WORKLOADS["tiny"], steps=6, host_flags=flags)


def test_replay_grid_sizes():
    wl = W.Workload("replay_grid", 4, (0, 0, 0, 0), R=12, B=300, K=100, rb=80, steps=6,
                    seq_first=("uniform", 200, 5000), seed=24)
    for g in (1, 5, 64):
        _lockstep(wl, replay_grid=g, prefetch=True)


# -- per-page residency ----------------------------------------------------------
PAGED = [
    W.Workload("paged_a", 2, (0, 0), R=6, B=300, K=100, rb=48, steps=10, page_size=16,
               resident_page_frac=0.3, seq_first=("uniform", 100, 3000), seed=31),
    W.Workload("paged_none", 1, (0,), R=5, B=256, K=64, rb=32, steps=8, page_size=8,
               resident_page_frac=0.0, seq_first=("uniform", 100, 2000), seed=32),
    W.Workload("paged_all", 1, (0,), R=4, B=256, K=64, rb=32, steps=6, page_size=32,
               resident_page_frac=1.0, seq_first=("uniform", 100, 2000), seed=33),
    W.Workload("paged_spec", 1, (0,), R=5, B=512, K=200, rb=656, steps=6, spec=3, page_size=7,
               resident_page_frac=0.5, seq_first=("uniform", 300, 5000), topk_kind="uniform",
               row_format="fp8_656", seed=34),
]


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("wl", PAGED, ids=[w.name for w in PAGED])
def test_paged_geometries(wl, fused):
    # fused: store + paged swap-in + backup in one launch; separate: three launches
    _lockstep(wl, fuse_store=fused)


@pytest.mark.timeout(600)
def test_paged_decode_full():
    _lockstep(W.WORKLOADS["paged_decode"], progress=True, compare_state_every=4)


# -- randomized small geometries mixing every feature ------------------------------
def _random_workload(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 1500))
    K = int(rng.integers(1, min(B, 4096) + 1))
    R = int(rng.integers(1, 9))
    layers = int(rng.integers(1, 4))
    anchor_of = [0]
    for l in range(1, layers):
        anchor_of.append(l if rng.random() < 0.5 else anchor_of[int(rng.integers(0, l))])
    anchor_of = tuple(anchor_of[a] if anchor_of[anchor_of[a]] == anchor_of[a] else a for a in anchor_of)
    paged = rng.random() < 0.4
    kw = dict(page_size=int(rng.integers(1, 65)), resident_page_frac=float(rng.random())) if paged else \
        dict(n_resident=int(rng.integers(0, R + 1)) if rng.random() < 0.3 else 0)
    return W.Workload(f"fuzz{seed}", layers, anchor_of, R=R, B=B, K=K, rb=16 * int(rng.integers(1, 17)),
                      steps=int(rng.integers(2, 7)), spec=int(rng.integers(1, 4)),
                      topk_kind="mixture" if rng.random() < 0.7 else "uniform",
                      seq_first=("uniform", 1, 3 * B + 10), seed=2000 + seed, **kw)


@pytest.mark.parametrize("seed", range(64))
def test_random_geometries(seed):
    wl = _random_workload(seed)
    blocks = [b for b in (128, 256, 512, 768, 1024) if _launch_shape_fits(wl, b)]
    block = blocks[seed % len(blocks)]
    _lockstep(wl, block_size=block, prefetch=bool(seed % 2), fuse_store=seed % 4 != 3)


def _random_wide_workload(seed):
    # larger batches and buffers than _random_workload: more requests per
    # launch, wider rows of the LRU list per wave, long contexts, and the
    # serving guide's 960-thread workgroup among the sizes
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(512, 8193))
    K = int(rng.integers(1, min(B, 4096) + 1))
    R = int(rng.integers(9, 65))
    layers = int(rng.integers(1, 4))
    anchor_of = tuple([0] + [0 if rng.random() < 0.5 else l for l in range(1, layers)])
    paged = rng.random() < 0.3
    kw = dict(page_size=int(rng.integers(8, 129)), resident_page_frac=float(rng.random() * 0.5)) if paged else \
        dict(n_resident=int(rng.integers(0, R // 2 + 1)))
    return W.Workload(f"fuzzwide{seed}", layers, anchor_of, R=R, B=B, K=K, rb=16 * int(rng.integers(1, 37)),
                      steps=int(rng.integers(2, 5)), spec=int(rng.integers(1, 3)),
                      topk_kind="mixture" if rng.random() < 0.6 else "uniform",
                      seq_first=("uniform", B // 2, 3 * B), seed=6000 + seed, **kw)


@pytest.mark.parametrize("seed", range(48))
def test_random_wide_geometries(seed):
    wl = _random_wide_workload(seed)
    blocks = [b for b in (256, 512, 960, 1024) if _launch_shape_fits(wl, b)]
    block = blocks[seed % len(blocks)]
    _lockstep(wl, block_size=block, prefetch=bool(seed % 2), fuse_store=seed % 4 != 3)


def test_buffer_above_8192_slots():
    # the widest kernel instantiation (16 chunks of 64 slots per wave)
    wl = W.Workload("wide", 1, (0,), R=2, B=9000, K=3000, rb=16, steps=4, topk_kind="uniform",
                    seq_first=("list", 12000, 20000), seed=41)
    _lockstep(wl)


def test_large_buffer_with_the_standard_top_k():
    # a buffer above 8192 slots with top_k 2048: the instantiation with 16
    # buffer chunks and 2 top-k chunks per wave
    wl = W.Workload("wide_k2048", 1, (0,), R=2, B=12288, K=2048, rb=16, steps=4,
                    seq_first=("list", 20000, 30000), seed=46)
    st = _lockstep(wl)
    assert st["misses"] > 0


@pytest.mark.parametrize("prefetch", [True, False], ids=["prefetch", "inline"])
def test_batch_wider_than_the_replay_workgroup(prefetch):
    # 600 batch rows: the replay's prefix of the plan counts runs over several
    # rows per thread (256 threads), and the swap-in grid has 600 workgroups
    wl = W.Workload("wide_batch", 3, (0, 0, 0), R=600, B=64, K=24, rb=16, steps=4, spec=2,
                    seq_first=("uniform", 30, 300), seed=47)
    st = _lockstep(wl, prefetch=prefetch)
    assert st["misses"] > 0


def test_twelve_thousand_requests():
    # a batch so wide that the replay's per-row prefix needs more than 64 KB
    # of LDS (init raises the kernel's dynamic LDS limit for it)
    wl = W.Workload("many_requests", 2, (0, 0), R=12000, B=16, K=8, rb=16, steps=3,
                    seq_first=("uniform", 8, 60), seed=48)
    st = _lockstep(wl)
    assert st["misses"] > 0


def test_million_token_context():
    # production inputs reach 1M tokens (HiCache page): positions past 2^20
    # through the hash, the slot map and the host-pool addressing
    wl = W.Workload("million", 1, (0,), R=2, B=2048, K=512, rb=16, steps=4, topk_kind="uniform",
                    seq_first=("list", 1_000_000, 1_048_600), seed=44)
    st = _lockstep(wl)
    assert st["misses"] > 0


def test_wide_rows():
    # 8 KB per token (512 chunks of 16 bytes per row): the copy's (row, column)
    # walk across many columns, rows much wider than a wave's 1 KB of loads
    wl = W.Workload("wide_rows", 2, (0, 0), R=3, B=300, K=100, rb=8192, steps=5,
                    seq_first=("list", 250, 900, 3000), seed=45)
    _lockstep(wl)


def test_maximum_sizes():
    # the largest buffer and top-k the library accepts: 16384 slots, 4096 top-k entries
    wl = W.Workload("max", 1, (0,), R=2, B=16384, K=4096, rb=16, steps=4,
                    seq_first=("list", 16000, 40000), seed=43)
    _lockstep(wl)


@pytest.mark.parametrize("wl", [W.WORKLOADS["tiny"], RAGGED[0]], ids=["tiny", "ragged_a"])
def test_block_size_960(wl):
    # the serving guide's swap_in_block_size: 15 waves, not a power of two
    _lockstep(wl, block_size=960)
