"""The C-ABI library: it loads, exports every symbol include/sgt.h declares, and
its host-only queries behave (no GPU call is made here)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgt.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^SGT_API\s+[\w\s\*]+?\b(sgt_\w+)\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from signal_gated_tiled_amd import _sgt
    if not os.path.exists(_sgt.LIB_PATH):
        from signal_gated_tiled_amd import build
        build.build()
    return _sgt.lib()


def test_header_declares_the_api():
    names = _declared()
    for n in ["sgt_ag_gemm", "sgt_gemm_rs", "sgt_moe_ag_gemm", "sgt_ctx_create", "sgt_ctx_destroy", "sgt_sync"]:
        assert n in names
    assert len(names) >= 15


def test_library_exports_every_declared_symbol(L):
    for n in _declared():
        assert hasattr(L, n), n


def test_opts_struct_layout_matches(L):
    from signal_gated_tiled_amd import _sgt
    o = _sgt.Opts()
    L.sgt_opts_init(ctypes.byref(o))
    assert o.in_dtype == _sgt.SGT_BF16 and o.out_dtype == _sgt.SGT_F32 and o.timeout_ms == 2000.0
    assert o.withhold_peer == -1 and o.trace is None and o.tile_rows == 0 and o.k_chunks == 0
    L.sgt_opts_size.restype = ctypes.c_size_t
    assert ctypes.sizeof(_sgt.Opts) == L.sgt_opts_size() == 128
    # every field at the offset the C compiler gave it: the last field is the event pair
    assert _sgt.Opts.consumer_events.offset == 128 - 2 * ctypes.sizeof(ctypes.c_void_p)
    assert o.sdma_peers == 0


def test_version_and_status_strings(L):
    import signal_gated_tiled_amd as sgt
    assert "gfx950" in sgt.version()
    assert L.sgt_status_str(-3) == b"SGT_ETIMEDOUT"


def test_panel_order_matches_pages_fixture():
    """The order the persistent consumer uses (computed by the library) against the hand-derived fixture."""
    import signal_gated_tiled_amd as sgt
    path = os.path.join(ROOT, "tests", "golden", "swizzle_orders.txt")
    n = 0
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, tail = line.split(":")
        order, W, tpp, rank = head.split()
        W, tpp, rank = int(W), int(tpp), int(rank)
        assert sgt.panel_order(W, rank, W * tpp * 16, 16, order) == [int(x) for x in tail.split()]
        n += 1
    assert n >= 8


def test_panel_order_is_a_permutation_for_ragged_panels():
    import signal_gated_tiled_amd as sgt
    for W, R, bm, order in [(4, 200, 256, "mesh"), (3, 300, 256, "shard"), (8, 96, 256, "mesh")]:
        got = sgt.panel_order(W, W - 1, W * R, bm, order)
        assert sorted(got) == list(range(-(-W * R // bm)))
        assert got[0] == ((W - 1) * R) // bm      # starts on the local shard


def test_flag_counts_and_argument_errors():
    import signal_gated_tiled_amd as sgt
    assert sgt.ag_flag_count(8, 16384, 8192) == 16384 // 32           # 512 KiB signal tiles
    assert sgt.ag_flag_count(4, 256, 256, in_dtype=sgt.SGT_F32, flag_rows=16) == 16
    assert sgt.rs_flag_count(8, 8192, 5120) == (64 * 40, 8 * 8 * 40)
    with pytest.raises(sgt.SgtError):
        sgt.ag_flag_count(8, 100, 64)                                   # M % W != 0
    with pytest.raises(sgt.SgtError):
        sgt.ag_flag_count(4, 256, 60)                                   # bf16 needs K % 8 == 0
    with pytest.raises(sgt.SgtError):
        sgt.ag_flag_count(65, 65 * 8, 64)                               # W > 64
    with pytest.raises(sgt.SgtError):
        sgt.rs_flag_count(4, 1024, 256, rs_tile=96)                     # must divide 256
    assert sgt.ag_panel_rows(8, 16384, 8192, 3584) == 256
    assert sgt.ll_buffer_bytes(8, 128, 8192, flag_rows=2) == 2 * 128 * 8192 * 2   # packets: twice the payload
    assert sgt.ll_buffer_bytes(4, 24, 40, in_dtype=sgt.SGT_F32, flag_rows=3) == 2 * 24 * 40 * 4
    with pytest.raises(sgt.SgtError):
        sgt.ll_buffer_bytes(8, 100, 64)                                 # M % W != 0
    assert sgt.ring_flag_count(8, 2048 * 8192) == (4 * 7 * 128, 16384)   # 2M-element chunks, 64 KiB tiles
    assert sgt.ring_flag_count(3, 3 * 16396) == (4 * 2 * 4099, 4)       # 16396 = 4 * 4099: 4-element tiles
    assert sgt.ring_flag_count(1, 16) == (0, 16)
    with pytest.raises(sgt.SgtError):
        sgt.ring_flag_count(4, 4 * 6)                                   # chunk not a multiple of 4


def test_a2a_flag_counts():
    import signal_gated_tiled_amd as sgt
    assert sgt.a2a_flag_count(8, 512, 64) == 64 * 16                     # 32-row chunks by default
    assert sgt.a2a_flag_count(4, 37, 8, flag_rows=5) == 8 * 8             # ragged last chunk
    assert sgt.a2a_flag_count(2, 0, 6) == 0
    for bad in (dict(W=8, T_r=64, E=60), dict(W=8, T_r=64, E=8 * 4097), dict(W=65, T_r=8, E=65)):
        with pytest.raises(sgt.SgtError):
            sgt.a2a_flag_count(bad["W"], bad["T_r"], bad["E"])            # E % W, E too large, W > 64
    with pytest.raises(sgt.SgtError):
        sgt.a2a_flag_count(8, 64, 64, flag_rows=1025)                    # chunk above 1024 rows


def test_rs_trace_words():
    import signal_gated_tiled_amd as sgt
    # Qwen shape: 8 blocks x 4 x 20 GEMM tiles of 256 x 256, 8 x 40 signal tiles of 128 x 128 in 32-row bands
    assert sgt.rs_trace_words(8, 8192, 5120) == 3 * (8 * 4 * 20 + 8 * 40 * 4)
    assert sgt.rs_trace_words(4, 1024, 392, rs_tile=64) == 3 * (4 * 1 * 2 + 4 * 7 * 2)
    assert sgt.rs_trace_words(4, 1024, 392, rs_tile=32) == 3 * (4 * 1 * 2 + 8 * 13)
    with pytest.raises(sgt.SgtError):
        sgt.rs_trace_words(4, 1000, 392)                               # M % W != 0


def test_k_chunk_flag_counts():
    import signal_gated_tiled_amd as sgt
    # one flag per 256-row panel and K chunk
    assert sgt.ag_flag_count(8, 16384, 8192, k_chunks=8) == 64 * 8
    assert sgt.ag_flag_count(8, 8192, 5120, k_chunks=8) == 32 * 8          # Qwen: chunks of 640 columns
    assert sgt.trace_words(8, 16384, 8192, 3584, k_chunks=8) == 64 * 14 * 4 + 64 * 8
    for bad in (dict(W=8, M=16384, K=8192, k_chunks=3),                    # K not a multiple of 128 x 3
                dict(W=8, M=8 * 200, K=1024, k_chunks=8),                  # shards of 200 rows: not whole panels
                dict(W=8, M=16384, K=8192, k_chunks=65)):                  # above 64
        with pytest.raises(sgt.SgtError):
            sgt.ag_flag_count(bad["W"], bad["M"], bad["K"], k_chunks=bad["k_chunks"])
    with pytest.raises(sgt.SgtError):
        sgt.ag_flag_count(4, 256, 256, in_dtype=sgt.SGT_F32, k_chunks=1)    # fp32 inputs
    with pytest.raises(sgt.SgtError):
        sgt.ag_flag_count(8, 16384, 8192, k_chunks=8, flag_rows=128)        # signal tiles are whole panels
    assert sgt.ag_flag_count(8, 16384, 8192, k_chunks=8, flag_rows=256) == 64 * 8
