"""The C-ABI library loads, exports every symbol include/mkv.h declares, and
rejects bad arguments on the host before touching the GPU.  CPU only."""
import ctypes
import os
import re

import pytest

import mixed_format_paged_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mkv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"mkv_append", "mkv_demote_pages", "mkv_decode_attn"} <= set(names)
    L = M.lib()
    for n in names:
        assert hasattr(L, n), n


def test_page_sizes_and_shape_checks():
    assert M.mkv_fp8_page_bytes((24, 4, 256)) == 32768
    assert M.mkv_tq3_page_bytes((24, 4, 256)) == 14336
    assert M.mkv_tq3_page_bytes((24, 4, 128)) == 7168
    assert M.mkv_fp8_page_bytes((64, 4, 256)) == 32768     # 16 query heads per KV head
    for bad in [(24, 4, 64), (24, 5, 256), (68, 4, 256), (17, 1, 128), (24, 4, 256, 32)]:
        assert M.mkv_fp8_page_bytes(bad) == 0


def _call_decode(layout, pool, batch, ws_bytes=1 << 30, q=4096, out=8192, ws=256, sm=0.0625):
    L = M.lib()
    return L.mkv_decode_attn(ctypes.byref(M._layout(layout)), ctypes.byref(pool) if pool else None,
                             ctypes.byref(batch) if batch else None, q, sm, out, None, ws, ws_bytes, None)


def test_host_validation_codes():
    L = M.lib()
    pool = M.PoolDesc(1 << 20, 1 << 21, 1 << 22, 10, 10, 1.0, 1.0)
    batch = M.BatchDesc(1 << 23, 1 << 24, 1 << 25, 2, 100)
    assert _call_decode((24, 4, 100), pool, batch) == -2                      # shape
    assert _call_decode((24, 4, 256), None, batch) == -1                      # null pool
    assert _call_decode((24, 4, 256), pool, batch, q=None) == -1              # null q
    assert _call_decode((24, 4, 256), pool, batch, q=8) == -3                 # misaligned q
    assert _call_decode((24, 4, 256), pool, batch, ws=128) == -3              # ws not 256-aligned
    assert _call_decode((24, 4, 256), pool, batch, ws_bytes=16) == -4         # workspace too small
    assert _call_decode((24, 4, 256), pool, batch, sm=-1.0) == -5             # bad sm_scale
    bad_pool = M.PoolDesc(1 << 20, 1 << 21, 1 << 22, -1, 10, 1.0, 1.0)
    assert _call_decode((24, 4, 256), bad_pool, batch) == -5
    assert "workspace" in M.mkv_status_string(-4)
    lay = ctypes.byref(M._layout((24, 4, 256)))
    assert L.mkv_demote_pages(lay, ctypes.byref(pool), None, None, 3, None) == -1
    assert L.mkv_demote_pages(lay, ctypes.byref(pool), None, None, -3, None) == -5
    assert L.mkv_append(lay, ctypes.byref(pool), 16, 16, 70000, 16, 16, 16, None, 1, None) == -5
    assert L.mkv_append(lay, ctypes.byref(pool), 8, 16, 1, 16, 16, 16, None, 1, None) == -3
    assert L.mkv_debug_gather(lay, ctypes.byref(pool), None, None, 0, 4, None, None) == -1
    assert L.mkv_materialize(lay, ctypes.byref(pool), ctypes.byref(batch), 2, 0, 1, 16, 16, None) == -5  # b >= batch
    assert L.mkv_materialize(lay, ctypes.byref(pool), ctypes.byref(batch), 0, -1, 1, 16, 16, None) == -5
    assert L.mkv_materialize(lay, ctypes.byref(pool), ctypes.byref(batch), 0, 0, 1, 8, 16, None) == -3   # misaligned
    assert L.mkv_materialize(lay, ctypes.byref(pool), None, 0, 0, 1, 16, 16, None) == -1
    assert L.mkv_materialize(lay, ctypes.byref(pool), ctypes.byref(batch), 0, 0, 0, None, None, None) == 0
    # lifecycle: an empty batch is a no-op; a bad window or count is a range error
    pool_t = M.PoolDesc(1 << 20, 1 << 21, 1 << 22, 10, 10, 1.0, 1.0)
    assert L.mkv_lifecycle_step(lay, ctypes.byref(pool_t), 1, None, None, None, 0, 0, 1 << 22, None, None, None, 4,
                                None, 0, None) == 0
    args = (lay, ctypes.byref(pool_t), 1, 1 << 23, 1 << 24, 1 << 25, 2, 100, 1 << 22, 1 << 26, 1 << 27, 1 << 28)
    assert L.mkv_lifecycle_step(*args, 0, 1 << 29, 4096, None) == -5                  # recent_pages < 1
    assert L.mkv_lifecycle_step(*args, 4, 1 << 29, 16, None) == -4                    # workspace too small
    assert L.mkv_lifecycle_step(*args, 4, 1 << 29 | 16, 4096, None) == -3             # misaligned workspace
    assert L.mkv_lifecycle_step(lay, ctypes.byref(pool_t), 1, 1 << 23, 1 << 24, 1 << 25, 2, 100, 1 << 21, 1 << 26,
                                1 << 27, 1 << 28, 4, 1 << 29, 4096, None) == -5       # tier is not the pools' map
    # multi-query decode: n_query outside [1, 16]
    assert L.mkv_decode_attn_multi(lay, ctypes.byref(pool), 1, ctypes.byref(batch), 17, 4096, 0.0625, 8192, None,
                                   256, 1 << 30, None) == -5
    # zero-size work is a successful no-op that launches nothing
    assert L.mkv_demote_pages(lay, ctypes.byref(pool), None, None, 0, None) == 0
    empty = M.BatchDesc(None, None, None, 0, 0)
    assert _call_decode((24, 4, 256), pool, empty) == 0


@pytest.mark.skipif("trace" in os.path.basename(M.LIB_PATH), reason="the item-trace build records a trace")
def test_item_trace_needs_the_trace_build():
    # the product build records no item trace: a range error, before any HIP call
    L = M.lib()
    buf = (ctypes.c_uint64 * 64)()
    assert L.mkv_debug_item_trace(buf, 64) == -5
    assert b"item-trace" in L.mkv_last_error()
    assert L.mkv_debug_item_trace(None, 64) == -1


def test_workspace_is_bounded_not_cache_sized():
    # The workspace holds the plan (8 bytes of page lists per block-table
    # entry) and the split-K partial states, whose count is capped by a
    # constant target (about four work items per CU) or one chunk per 512
    # pages, plus two per request.  It stays a small fraction of the KV bytes
    # it reads, never a dense shadow of the cache: under 1 % at the canary
    # shape, and well under a tenth for a single request split over the whole
    # GPU (chunks of 32 TQ3 pages, 112 KiB each, leave one 6 KiB partial state
    # per KV head).
    lay = (24, 4, 256)
    tq3_page, fp8_page = M.mkv_tq3_page_bytes(lay), M.mkv_fp8_page_bytes(lay)
    canary = M.mkv_decode_workspace_bytes(lay, 2, 7376, 16)
    assert canary < 0.01 * 1_734_344_704
    for batch, cap, layers in [(2, 7376, 16), (2, 73760, 16), (1, 8192, 1), (1, 80 * 8192, 1),
                               (64, 131072, 1), (32, 64730, 1), (8, 8192, 1)]:
        ws = M.mkv_decode_workspace_bytes(lay, batch, cap, layers)
        kv_min = layers * cap * tq3_page          # every page TQ3: the smallest cache of this shape
        assert ws < 0.08 * kv_min, (batch, cap, layers, ws / kv_min)
