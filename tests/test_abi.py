"""The C ABI library (CPU only, no compute calls): it loads, exports every
entry point include/hisparse.h declares, and rejects bad configurations on
the host before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisparse.h")


def declared_entry_points():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hisparse_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from decode_memory_tiering_amd.hisparse import load_library
    return load_library()


def test_header_declares_the_boundary():
    names = declared_entry_points()
    for must in ("hisparse_init", "hisparse_swap_in", "hisparse_replay_plan", "hisparse_backup"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    from decode_memory_tiering_amd.hisparse import EXPORTS
    names = declared_entry_points()
    assert sorted(EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_pure_host_calls(lib):
    from decode_memory_tiering_amd import hisparse as H
    assert H.hisparse_version() == 1
    assert H.hisparse_strerror(0) == "ok"
    assert H.hisparse_strerror(-22) == "invalid argument"
    b = H.hisparse_swap_in_lds_bytes(2048, 6144)
    assert 40_000 < b <= 160 * 1024          # fits one gfx950 workgroup
    assert H.hisparse_swap_in_lds_bytes(0, 10) == 0


@pytest.mark.parametrize("bad", [
    dict(top_k=10, device_buffer_size=5),          # K > B
    dict(top_k=0, device_buffer_size=5),
    dict(top_k=8, device_buffer_size=20000),       # B above the supported maximum
    dict(top_k=8, device_buffer_size=16385),       # one slot above it
    dict(top_k=4097, device_buffer_size=8192),     # K above the supported maximum
    dict(row_bytes=24),                            # not a multiple of 16
    dict(num_layers=0),
    dict(block_size=100),
    dict(anchor_of=[1, 0]),                         # anchor of an anchor must be itself
    dict(max_requests=131072, device_buffer_size=16383),   # R * (B + 1) = 2^31: hot rows overflow int32
])
def test_init_rejects_bad_config_on_host(lib, bad):
    from decode_memory_tiering_amd import hisparse as H
    cfg = dict(top_k=8, device_buffer_size=16, num_layers=2, max_requests=2, max_seq_len=64, row_bytes=32,
               host_pool=[0, 0], hot_buffer=[0, 0], anchor_of=[0, 0], block_size=0)
    cfg.update(bad)
    n = cfg["num_layers"]
    cfg["host_pool"] = (cfg["host_pool"] * 2)[:max(n, 1)]
    cfg["hot_buffer"] = (cfg["hot_buffer"] * 2)[:max(n, 1)]
    cfg["anchor_of"] = (list(cfg["anchor_of"]) * 2)[:max(n, 1)]
    with pytest.raises(H.HisparseError) as e:
        H.hisparse_init(**cfg)
    assert e.value.rc == H.HISPARSE_EINVAL


def test_null_context_rejected(lib):
    from decode_memory_tiering_amd import hisparse as H
    assert lib.hisparse_swap_in(None, 0, None, None, None, None, 1, None, H.hisparse_plan(), None) == -22
    assert lib.hisparse_backup(None, 0, None, None, None, 1, None) == -22
    assert lib.hisparse_replay_plan(None, 0, H.hisparse_plan(), None, 1, None) == -22


def test_serving_config_keys():
    from decode_memory_tiering_amd.hisparse import parse_hisparse_config
    kw = parse_hisparse_config('{"top_k": 2048, "device_buffer_size": 6144, "host_to_device_ratio": 10, '
                               '"swap_in_block_size": 960}')
    assert kw == dict(K=2048, B=6144, block_size=960)
    assert parse_hisparse_config({"top_k": 8, "device_buffer_size": 16}) == dict(K=8, B=16)
    for bad in ('{"top_k": 8, "device_buffer_size": 16, "swap_in_block_size": 100}',
                '{"top_k": 32, "device_buffer_size": 16}', '{"top_k": 8}',
                '{"top_k": 8, "device_buffer_size": 16, "page": 4}'):
        with pytest.raises(ValueError):
            parse_hisparse_config(bad)
