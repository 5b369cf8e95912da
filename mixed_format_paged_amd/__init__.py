"""Python binding of libmkv: mixed FP8 / TQ3 paged decode attention on MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of
libmkv.so (include/mkv.h).  Tensors are torch tensors used as device memory;
each function takes the same arguments as its C counterpart, with tensors in
place of pointers, and raises MkvError on a non-zero status.  There is no CPU
fallback: if libmkv.so is missing this module raises on first use.
"""
import ctypes
import os

__all__ = [
    "MkvError", "Layout", "PoolDesc", "BatchDesc", "lib", "make_pool", "make_batch",
    "mkv_fp8_page_bytes", "mkv_tq3_page_bytes", "mkv_append", "mkv_demote_pages",
    "mkv_decode_workspace_bytes", "mkv_decode_attn", "mkv_decode_attn_noalloc", "mkv_decode_attn_layers",
    "mkv_debug_gather", "mkv_stream_read", "mkv_workspace_status", "mkv_demote_pages_layers", "mkv_decode_plan",
    "mkv_attend_fp8", "mkv_attend_tq3", "mkv_attend_partials", "mkv_merge", "mkv_attend", "mkv_append_attend", "mkv_materialize", "mkv_lifecycle_workspace_bytes", "mkv_lifecycle_step",
    "mkv_lifecycle_release", "mkv_decode_workspace_bytes_multi", "mkv_decode_attn_multi", "mkv_status_string",
    "mkv_last_error", "mkv_set_partial_kind", "set_partial_kind", "mkv_debug_item_trace",
    "LIB_PATH", "TIER_RECENT", "TIER_ANCHOR", "TIER_STALE", "TIER_FREE",
    "MKV_DEV_BAD_PAGE_ID", "MKV_DEV_BAD_TIER", "MKV_DEV_BAD_SEQ_LEN", "MKV_DEV_NO_FREE_PAGE", "MKV_DEV_NO_PLAN",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# MKV_LIB_PATH selects another build of the library (e.g. one with host-side
# sanitizers); by default the in-tree libmkv.so
LIB_PATH = os.environ.get("MKV_LIB_PATH") or os.path.join(_HERE, "libmkv.so")

TIER_RECENT, TIER_ANCHOR, TIER_STALE, TIER_FREE = 0, 1, 2, 0xFF
MKV_DEV_BAD_PAGE_ID, MKV_DEV_BAD_TIER, MKV_DEV_BAD_SEQ_LEN, MKV_DEV_NO_FREE_PAGE, MKV_DEV_NO_PLAN = 1, 2, 4, 8, 16

c_i32, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class MkvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"mkv status {status}: {message}")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("num_q_heads", c_i32), ("num_kv_heads", c_i32), ("head_dim", c_i32), ("page_size", c_i32)]


class PoolDesc(ctypes.Structure):
    _fields_ = [("fp8_slab", c_vp), ("tq3_slab", c_vp), ("tier", c_vp), ("n_fp8", c_i32),
                ("n_tq3", c_i32), ("k_scale", c_f32), ("v_scale", c_f32), ("tq3_signs", c_vp)]


class BatchDesc(ctypes.Structure):
    _fields_ = [("bt_offsets", c_vp), ("bt_pages", c_vp), ("seq_lens", c_vp), ("batch", c_i32),
                ("bt_capacity", c_i32)]


_lib = None


def lib():
    """Load libmkv.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MkvError(-100, f"{LIB_PATH} is not built; run `python -m mixed_format_paged_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "mkv_fp8_page_bytes": (c_sz, [P(Layout)]),
        "mkv_tq3_page_bytes": (c_sz, [P(Layout)]),
        "mkv_append": (c_i32, [P(Layout), P(PoolDesc), c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp]),
        "mkv_demote_pages": (c_i32, [P(Layout), P(PoolDesc), c_vp, c_vp, c_i32, c_vp]),
        "mkv_demote_pages_layers": (c_i32, [P(Layout), P(PoolDesc), c_i32, c_vp, c_vp, c_i32, c_vp]),
        "mkv_decode_plan": (c_i32, [P(Layout), P(PoolDesc), P(BatchDesc), c_i32, c_vp, c_sz, c_vp]),
        "mkv_attend_fp8": (c_i32, [P(Layout), P(PoolDesc), c_i32, P(BatchDesc), c_vp, c_f32, c_vp, c_sz, c_vp]),
        "mkv_attend_tq3": (c_i32, [P(Layout), P(PoolDesc), c_i32, P(BatchDesc), c_vp, c_f32, c_vp, c_sz, c_vp]),
        "mkv_attend_partials": (c_i32, [P(Layout), P(PoolDesc), c_i32, P(BatchDesc), c_vp, c_f32, c_vp, c_sz, c_vp]),
        "mkv_merge": (c_i32, [P(Layout), c_i32, P(BatchDesc), c_vp, c_vp, c_vp, c_sz, c_vp]),
        "mkv_attend": (c_i32, [P(Layout), P(PoolDesc), c_i32, P(BatchDesc), c_vp, c_f32, c_vp, c_vp, c_vp, c_sz, c_vp]),
        "mkv_append_attend": (c_i32, [P(Layout), P(PoolDesc), c_i32, P(BatchDesc), c_vp, c_vp, c_vp, c_f32, c_vp, c_vp,
                                      c_vp, c_sz, c_vp]),
        "mkv_decode_workspace_bytes": (c_sz, [P(Layout), c_i32, c_i32, c_i32]),
        "mkv_decode_attn": (c_i32, [P(Layout), P(PoolDesc), P(BatchDesc), c_vp, c_f32, c_vp, c_vp, c_vp, c_sz, c_vp]),
        "mkv_decode_attn_noalloc": (c_i32, [P(Layout), P(PoolDesc), P(BatchDesc), c_vp, c_f32, c_vp, c_vp, c_vp]),
        "mkv_decode_attn_layers": (c_i32, [P(Layout), P(PoolDesc), c_i32, P(BatchDesc), c_vp, c_f32, c_vp, c_vp, c_vp, c_sz, c_vp]),
        "mkv_debug_gather": (c_i32, [P(Layout), P(PoolDesc), c_vp, c_vp, c_i32, c_i32, c_vp, c_vp]),
        "mkv_stream_read": (c_i32, [c_vp, c_sz, c_vp, c_sz, c_vp]),
        "mkv_materialize": (c_i32, [P(Layout), P(PoolDesc), P(BatchDesc), c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
        "mkv_lifecycle_workspace_bytes": (c_sz, [c_i32]),
        "mkv_decode_workspace_bytes_multi": (c_sz, [P(Layout), c_i32, c_i32, c_i32, c_i32]),
        "mkv_decode_attn_multi": (c_i32, [P(Layout), P(PoolDesc), c_i32, P(BatchDesc), c_i32, c_vp, c_f32, c_vp, c_vp,
                                          c_vp, c_sz, c_vp]),
        "mkv_lifecycle_step": (c_i32, [P(Layout), P(PoolDesc), c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp,
                                       c_vp, c_i32, c_vp, c_sz, c_vp]),
        "mkv_lifecycle_release": (c_i32, [P(Layout), P(PoolDesc), c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_i32, c_vp, c_sz, c_vp]),
        "mkv_workspace_status": (c_i32, [c_vp, c_vp]),
        "mkv_status_string": (ctypes.c_char_p, [c_i32]),
        "mkv_last_error": (ctypes.c_char_p, []),
        "mkv_set_partial_kind": (c_i32, [c_i32]),
        "mkv_debug_item_trace": (c_i32, [c_vp, c_sz]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc):
    if rc < 0:
        L = lib()
        raise MkvError(rc, f"{L.mkv_status_string(rc).decode()}: {L.mkv_last_error().decode()}")
    return rc


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise MkvError(-101, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MkvError(-101, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MkvError(-101, f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _layout(layout):
    if isinstance(layout, Layout):
        return layout
    hq, hkv, d = layout[:3]
    return Layout(hq, hkv, d, layout[3] if len(layout) > 3 else 16)


def make_pool(fp8_slab, tq3_slab, tier, n_fp8, n_tq3, k_scale=1.0, v_scale=1.0, tq3_signs=None):
    """PoolDesc over device tensors (uint8 slabs and the uint8 tier map);
    tq3_signs: None, or a device int8 [head_dim] tensor of +-1 (rotated TQ3)."""
    import torch
    signs = None if tq3_signs is None else _ptr(tq3_signs, torch.int8, "tq3_signs")
    p = PoolDesc(_ptr(fp8_slab, torch.uint8, "fp8_slab"), _ptr(tq3_slab, torch.uint8, "tq3_slab"),
                 _ptr(tier, torch.uint8, "tier"), int(n_fp8), int(n_tq3), float(k_scale), float(v_scale), signs)
    p._keep = (fp8_slab, tq3_slab, tier, tq3_signs)
    return p


def make_batch(bt_offsets, bt_pages, seq_lens):
    """BatchDesc over int32 device tensors (CSR block tables and lengths)."""
    import torch
    b = BatchDesc(_ptr(bt_offsets, torch.int32, "bt_offsets"), _ptr(bt_pages, torch.int32, "bt_pages"),
                  _ptr(seq_lens, torch.int32, "seq_lens"), int(seq_lens.numel()), int(bt_pages.numel()))
    b._keep = (bt_offsets, bt_pages, seq_lens)
    return b


def mkv_fp8_page_bytes(layout):
    return int(lib().mkv_fp8_page_bytes(ctypes.byref(_layout(layout))))


def mkv_tq3_page_bytes(layout):
    return int(lib().mkv_tq3_page_bytes(ctypes.byref(_layout(layout))))


def mkv_append(layout, pool, k, v, bt_offsets, bt_pages, pos, counts=None, stream=None):
    import torch
    batch, n_new = (k.shape[0], k.shape[1]) if k.dim() == 4 else (k.shape[0], 1)
    return _check(lib().mkv_append(ctypes.byref(_layout(layout)), ctypes.byref(pool),
                                   _ptr(k, torch.float32, "k"), _ptr(v, torch.float32, "v"), n_new,
                                   _ptr(bt_offsets, torch.int32, "bt_offsets"),
                                   _ptr(bt_pages, torch.int32, "bt_pages"), _ptr(pos, torch.int32, "pos"),
                                   _ptr(counts, torch.int32, "counts"), batch, _stream(stream)))


def mkv_demote_pages(layout, pool, src_fp8, dst_tq3, stream=None):
    import torch
    return _check(lib().mkv_demote_pages(ctypes.byref(_layout(layout)), ctypes.byref(pool),
                                         _ptr(src_fp8, torch.int32, "src_fp8"),
                                         _ptr(dst_tq3, torch.int32, "dst_tq3"), int(src_fp8.numel()),
                                         _stream(stream)))


def mkv_demote_pages_layers(layout, pools, src_fp8, dst_tq3, stream=None):
    import torch
    arr = (PoolDesc * len(pools))(*pools)
    return _check(lib().mkv_demote_pages_layers(ctypes.byref(_layout(layout)), arr, len(pools),
                                                _ptr(src_fp8, torch.int32, "src_fp8"),
                                                _ptr(dst_tq3, torch.int32, "dst_tq3"), int(src_fp8.numel()),
                                                _stream(stream)))


def _ws(ws):
    return _ptr(ws, None, "ws"), int(ws.numel() * ws.element_size())


def mkv_decode_plan(layout, pool, batch, n_layers, ws, stream=None):
    p, n = _ws(ws)
    return _check(lib().mkv_decode_plan(ctypes.byref(_layout(layout)), ctypes.byref(pool), ctypes.byref(batch),
                                        int(n_layers), p, n, _stream(stream)))


def _attend(fn, layout, pools, batch, q, sm_scale, ws, stream):
    import torch
    arr = (PoolDesc * len(pools))(*pools)
    p, n = _ws(ws)
    return _check(fn(ctypes.byref(_layout(layout)), arr, len(pools), ctypes.byref(batch),
                     _ptr(q, torch.float32, "q"), float(sm_scale), p, n, _stream(stream)))


def mkv_attend_fp8(layout, pools, batch, q, sm_scale, ws, stream=None):
    return _attend(lib().mkv_attend_fp8, layout, pools, batch, q, sm_scale, ws, stream)


def mkv_attend_tq3(layout, pools, batch, q, sm_scale, ws, stream=None):
    return _attend(lib().mkv_attend_tq3, layout, pools, batch, q, sm_scale, ws, stream)


def mkv_attend_partials(layout, pools, batch, q, sm_scale, ws, stream=None):
    return _attend(lib().mkv_attend_partials, layout, pools, batch, q, sm_scale, ws, stream)


def mkv_merge(layout, n_layers, batch, out, lse, ws, stream=None):
    import torch
    p, n = _ws(ws)
    return _check(lib().mkv_merge(ctypes.byref(_layout(layout)), int(n_layers), ctypes.byref(batch),
                                  _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), p, n,
                                  _stream(stream)))


def mkv_append_attend(layout, pools, batch, k_new, v_new, q, sm_scale, out, lse, ws, stream=None):
    """mkv_append of each request's newest token + mkv_attend, in the same launches."""
    import torch
    arr = (PoolDesc * len(pools))(*pools)
    p, n = _ws(ws)
    return _check(lib().mkv_append_attend(ctypes.byref(_layout(layout)), arr, len(pools), ctypes.byref(batch),
                                          _ptr(k_new, torch.float32, "k_new"), _ptr(v_new, torch.float32, "v_new"),
                                          _ptr(q, torch.float32, "q"), float(sm_scale), _ptr(out, torch.float32, "out"),
                                          _ptr(lse, torch.float32, "lse"), p, n, _stream(stream)))


def mkv_attend(layout, pools, batch, q, sm_scale, out, lse, ws, stream=None):
    import torch
    arr = (PoolDesc * len(pools))(*pools)
    p, n = _ws(ws)
    return _check(lib().mkv_attend(ctypes.byref(_layout(layout)), arr, len(pools), ctypes.byref(batch),
                                   _ptr(q, torch.float32, "q"), float(sm_scale), _ptr(out, torch.float32, "out"),
                                   _ptr(lse, torch.float32, "lse"), p, n, _stream(stream)))


def mkv_decode_workspace_bytes(layout, batch, bt_capacity, n_layers=1):
    return int(lib().mkv_decode_workspace_bytes(ctypes.byref(_layout(layout)), int(batch),
                                                int(bt_capacity), int(n_layers)))


def mkv_decode_attn(layout, pool, batch, q, sm_scale, out, lse, ws, stream=None):
    import torch
    return _check(lib().mkv_decode_attn(ctypes.byref(_layout(layout)), ctypes.byref(pool), ctypes.byref(batch),
                                        _ptr(q, torch.float32, "q"), float(sm_scale),
                                        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
                                        _ptr(ws, None, "ws"), int(ws.numel() * ws.element_size()),
                                        _stream(stream)))


def mkv_decode_attn_noalloc(layout, pool, batch, q, sm_scale, out, lse, stream=None):
    import torch
    return _check(lib().mkv_decode_attn_noalloc(ctypes.byref(_layout(layout)), ctypes.byref(pool), ctypes.byref(batch),
                                                _ptr(q, torch.float32, "q"), float(sm_scale),
                                                _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
                                                _stream(stream)))


def mkv_decode_attn_layers(layout, pools, batch, q, sm_scale, out, lse, ws, stream=None):
    import torch
    arr = (PoolDesc * len(pools))(*pools)
    return _check(lib().mkv_decode_attn_layers(ctypes.byref(_layout(layout)), arr, len(pools), ctypes.byref(batch),
                                               _ptr(q, torch.float32, "q"), float(sm_scale),
                                               _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
                                               _ptr(ws, None, "ws"), int(ws.numel() * ws.element_size()),
                                               _stream(stream)))


def mkv_debug_gather(layout, pool, bt_offsets, bt_pages, b, n_pages, out, stream=None):
    import torch
    return _check(lib().mkv_debug_gather(ctypes.byref(_layout(layout)), ctypes.byref(pool),
                                         _ptr(bt_offsets, torch.int32, "bt_offsets"),
                                         _ptr(bt_pages, torch.int32, "bt_pages"), int(b), int(n_pages),
                                         _ptr(out, torch.uint8, "out"), _stream(stream)))


def mkv_debug_item_trace(host):
    """Copy the item trace of an MKV_ITEM_TRACE=1 build into host, a
    C-contiguous numpy uint64 array (up to 4096 x 32 words)."""
    import numpy as np
    if not isinstance(host, np.ndarray) or host.dtype != np.uint64 or not host.flags.c_contiguous:
        raise MkvError(-101, "host must be a C-contiguous numpy uint64 array")
    return _check(lib().mkv_debug_item_trace(host.ctypes.data, host.size))


def mkv_stream_read(src, sink, nbytes=None, stream=None):
    """Read the first floor(nbytes / 3584) * 3584 bytes of device tensor src
    (all of it by default) with the page-staging loads; sink: int32 device
    tensor of at least 12 words, per-wave XORs of the units' first words."""
    import torch
    nb = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if nb > src.numel() * src.element_size():
        raise MkvError(-101, "nbytes exceeds src")
    return _check(lib().mkv_stream_read(_ptr(src, name="src"), nb, _ptr(sink, torch.int32, "sink"), sink.numel(),
                                        _stream(stream)))


def mkv_materialize(layout, pool, batch, b, page_lo, n_pages, k_out, v_out, stream=None):
    """Dense bf16 K and V (int16 tensors holding bf16 bits, or torch.bfloat16)
    [n_pages * 16][Hkv][d] of logical pages [page_lo, page_lo + n_pages) of request b."""
    lay = _layout(layout)
    need = int(n_pages) * 16 * lay.num_kv_heads * lay.head_dim
    for t, name in ((k_out, "k_out"), (v_out, "v_out")):
        if t is not None and (t.element_size() != 2 or t.numel() < need):
            raise MkvError(-101, f"{name} must hold {need} 2-byte elements")
    return _check(lib().mkv_materialize(ctypes.byref(_layout(layout)), ctypes.byref(pool), ctypes.byref(batch),
                                        int(b), int(page_lo), int(n_pages), _ptr(k_out, name="k_out"),
                                        _ptr(v_out, name="v_out"), _stream(stream)))


def mkv_decode_workspace_bytes_multi(layout, batch, bt_capacity, n_layers, n_query):
    return lib().mkv_decode_workspace_bytes_multi(ctypes.byref(_layout(layout)), int(batch), int(bt_capacity),
                                                  int(n_layers), int(n_query))


def mkv_decode_attn_multi(layout, pools, batch, q, sm_scale, out, lse, ws, stream=None):
    """Causal multi-query decode: q, out [L][B][T][Hq][d], lse [L][B][T][Hq] (T = q.shape[2])."""
    import torch
    arr = _pool_array(pools)
    p, n = _ws(ws)
    return _check(lib().mkv_decode_attn_multi(ctypes.byref(_layout(layout)), arr, len(arr), ctypes.byref(batch),
                                              int(q.shape[2]), _ptr(q, torch.float32, "q"), float(sm_scale),
                                              _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), p, n,
                                              _stream(stream)))


def mkv_lifecycle_workspace_bytes(batch):
    return lib().mkv_lifecycle_workspace_bytes(int(batch))


def _pool_array(pools):
    pools = list(pools)
    arr = (PoolDesc * len(pools))(*pools)
    arr._keep = pools
    return arr


def mkv_lifecycle_step(layout, pools, bt_offsets, bt_pages, seq_lens, tier, fp8_free, tq3_free, free_tops,
                       recent_pages, ws, stream=None):
    """One decode step's page lifecycle (new FP8 pages, aging into TQ3 in every
    layer, block-table / tier / free-stack updates); int32 / uint8 device tensors."""
    import torch
    arr = _pool_array(pools)
    return _check(lib().mkv_lifecycle_step(
        ctypes.byref(_layout(layout)), arr, len(arr), _ptr(bt_offsets, torch.int32, "bt_offsets"),
        _ptr(bt_pages, torch.int32, "bt_pages"), _ptr(seq_lens, torch.int32, "seq_lens"), int(seq_lens.numel()),
        int(bt_pages.numel()), _ptr(tier, torch.uint8, "tier"), _ptr(fp8_free, torch.int32, "fp8_free"),
        _ptr(tq3_free, torch.int32, "tq3_free"), _ptr(free_tops, torch.int32, "free_tops"), int(recent_pages),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def mkv_lifecycle_release(layout, pool, bt_offsets, bt_pages, seq_lens, tier, fp8_free, tq3_free, free_tops,
                          requests, ws, stream=None):
    """Return every live page of the listed requests to the free stacks."""
    import torch
    return _check(lib().mkv_lifecycle_release(
        ctypes.byref(_layout(layout)), ctypes.byref(pool), _ptr(bt_offsets, torch.int32, "bt_offsets"),
        _ptr(bt_pages, torch.int32, "bt_pages"), _ptr(seq_lens, torch.int32, "seq_lens"), int(seq_lens.numel()),
        int(bt_pages.numel()), _ptr(tier, torch.uint8, "tier"), _ptr(fp8_free, torch.int32, "fp8_free"),
        _ptr(tq3_free, torch.int32, "tq3_free"), _ptr(free_tops, torch.int32, "free_tops"),
        _ptr(requests, torch.int32, "requests"), int(requests.numel()), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))


def mkv_workspace_status(ws, stream=None):
    return _check(lib().mkv_workspace_status(_ptr(ws, None, "ws"), _stream(stream)))


def mkv_status_string(status):
    return lib().mkv_status_string(int(status)).decode()


def mkv_last_error():
    return lib().mkv_last_error().decode()


def mkv_set_partial_kind(kind):
    """Measurement hook: 1 = matrix-core partial kernels, 0 = VALU kernels."""
    return _check(lib().mkv_set_partial_kind(int(kind)))


set_partial_kind = mkv_set_partial_kind
