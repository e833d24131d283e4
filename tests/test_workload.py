"""The seeded input generators (CPU only): shapes, distinctness, the top-k
mixture, padding, and reproducibility."""
import numpy as np
import pytest

from decode_memory_tiering_amd import workload as W


def test_five_workloads_have_the_stated_shapes():
    w = W.WORKLOADS
    assert (w["tiny"].R, w["tiny"].B, w["tiny"].K, w["tiny"].rb, w["tiny"].steps) == (4, 1024, 256, 1152, 16)
    assert (w["fastpath_mix"].R, w["fastpath_mix"].B, w["fastpath_mix"].K) == (64, 6144, 2048)
    d = w["dsv32_decode"]
    assert (d.num_layers, d.R, d.n_resident, d.steps, d.anchors) == (4, 128, 32, 64, (0, 1, 2, 3))
    x = w["indexshare"]
    assert x.anchors == (0,) and x.skip_layers == (1, 2, 3)
    lc = w["long_context"]
    assert (lc.R, lc.B, lc.K, lc.rb, lc.spec, lc.topk_kind) == (32, 4096, 2048, 656, 3, "uniform")
    assert W.first_seq_lens(lc)[0] == 131072 and W.first_seq_lens(d)[0] == 40000


def test_fastpath_mix_lengths_and_share():
    wl = W.WORKLOADS["fastpath_mix"]
    L = W.first_seq_lens(wl)
    assert L.min() >= 512 and L.max() <= 12288
    assert np.array_equal(L, W.first_seq_lens(wl))           # seeded
    share = np.mean(L <= wl.B)
    assert 0.3 < share < 0.7                                   # about half take slot = position


def test_resident_mask_exact_count():
    wl = W.WORKLOADS["dsv32_decode"]
    m = W.resident_mask(wl)
    assert m.sum() == 32 and np.array_equal(m, W.resident_mask(wl))


@pytest.mark.parametrize("L,K", [(40000, 2048), (3000, 2048), (2049, 2048), (131072, 2048), (9, 8)])
def test_topk_rows_distinct_in_range(L, K):
    rng = np.random.default_rng(1)
    prev = None
    for _ in range(4):
        row = W.draw_topk_row(rng, L, K, prev)
        assert row.shape == (K,) and row.min() >= 0 and row.max() < L
        assert np.unique(row).size == K
        prev = row


def test_topk_mixture_proportions():
    rng = np.random.default_rng(2)
    L, K = 40000, 2048
    prev = W.draw_topk_row(rng, L, K, None)
    row = W.draw_topk_row(rng, L, K, prev)
    from_prev = np.isin(row, prev).sum()
    recent = (row >= L - W.RECENT_WINDOW).sum()
    assert from_prev >= K // 2                         # half drawn from the previous selection
    assert recent >= K // 4                            # a quarter from the last 2048 positions
    assert row[: K // 2].max() > 0 and not np.array_equal(np.sort(row), row)   # shuffled order


def test_topk_padding_when_short():
    rng = np.random.default_rng(3)
    row = W.draw_topk_row(rng, 100, 256, None)
    assert sorted(row[:100].tolist()) == list(range(100))
    assert (row[100:] == -1).all()


def test_topk_uniform_kind():
    rng = np.random.default_rng(4)
    row = W.draw_topk_row(rng, 131072, 2048, None, kind="uniform")
    assert np.unique(row).size == 2048 and row.max() < 131072
    assert (row >= 131072 - 2048).sum() < 200          # no recency bias


def test_topk_stream_reproducible():
    wl = W.WORKLOADS["tiny"]
    L = W.seq_lens_at(wl, 0)
    a = W.TopkStream(wl, 0).rows(0, L)
    b = W.TopkStream(wl, 0).rows(0, L)
    c = W.TopkStream(wl, 1).rows(0, L)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_payload_rows_cpu():
    torch = pytest.importorskip("torch")
    wl = W.WORKLOADS["tiny"]
    g = torch.Generator().manual_seed(0)
    rows = W.payload_rows(10, wl, g, "cpu")
    assert rows.shape == (10, 1152) and rows.dtype == torch.uint8
    lc = W.WORKLOADS["long_context"]
    rows = W.payload_rows(3, lc, torch.Generator().manual_seed(0), "cpu")
    assert rows.shape == (3, 656)
    assert torch.equal(rows[:, 512:528].view(torch.float32), torch.ones(3, 4))
    pool = torch.empty(2, 20, 1152, dtype=torch.uint8)
    W.fill_host_pool(pool, wl, 0, [5, 20], "cpu")
    assert (pool[0, 5:] == W.POISON).all() and not (pool[1] == W.POISON).all()
