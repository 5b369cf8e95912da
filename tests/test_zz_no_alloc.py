"""mkv_decode_attn_noalloc (workspace in the library's static device array)
against mkv_decode_attn with a caller workspace: the same kernels, so the
outputs must be bit-identical.  Two calls in a row, the second with a smaller
batch, so the array holds the first call's contents when the second runs."""
import math

import numpy as np
import pytest
import torch

import mixed_format_paged_amd as M
import workloads as W
from workloads.device_cache import DeviceWorkload

pytestmark = pytest.mark.gpu


def _reference(dw):
    """mkv_decode_attn with a caller workspace: outputs and the call's arguments."""
    w = dw.w
    layout = (w.Hq, w.Hkv, w.d)
    B = int(dw.seq_lens.numel())
    ws = torch.empty(M.mkv_decode_workspace_bytes(layout, B, dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
    o = torch.full((B, w.Hq, w.d), float("nan"), device="cuda")
    l = torch.full((B, w.Hq), float("nan"), device="cuda")
    q = dw.q[0].contiguous()
    M.mkv_decode_attn(layout, dw.cache.pools[0], dw.batch(), q, 1 / math.sqrt(w.d), o, l, ws)
    assert M.mkv_workspace_status(ws) == 0
    return o.cpu().numpy(), l.cpu().numpy(), (layout, q)


def test_noalloc_decode_matches_workspace_decode_twice():
    big = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=6, L=1, lengths=("list", (5000, 17, 0, 3000, 1200, 8192)),
                   recent_tokens=64)
    small = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=2, L=1, lengths=("list", (700, 33)), recent_tokens=32,
                     seed=9)
    dws = [DeviceWorkload(w, W.make_structure(w), "cuda") for w in (big, small)]
    refs = [_reference(dw) for dw in dws]
    outs = []
    # two calls in a row: the second (smaller batch) finds the first one's
    # contents in the static array
    for dw, (_, _, (layout, q)) in zip(dws, refs):
        B = int(dw.seq_lens.numel())
        o = torch.full((B, dw.w.Hq, dw.w.d), float("nan"), device="cuda")
        l = torch.full((B, dw.w.Hq), float("nan"), device="cuda")
        M.mkv_decode_attn_noalloc(layout, dw.cache.pools[0], dw.batch(), q, 1 / math.sqrt(dw.w.d), o, l)
        outs.append((o, l))
    torch.cuda.synchronize()
    for (o_ref, l_ref, _), (o, l), w in zip(refs, outs, (big, small)):
        assert np.isfinite(o_ref).all()
        assert np.array_equal(o.cpu().numpy(), o_ref), w.name
        assert np.array_equal(l.cpu().numpy(), l_ref), w.name


def test_noalloc_refuses_a_batch_past_its_array():
    layout = (24, 4, 256)
    pool = M.PoolDesc(1 << 20, 1 << 21, 1 << 22, 10, 10, 1.0, 1.0)
    huge = M.BatchDesc(1 << 23, 1 << 24, 1 << 25, 4096, 1 << 24)
    assert M.mkv_decode_workspace_bytes(layout, 4096, 1 << 24, 1) > 32 << 20
    with pytest.raises(M.MkvError) as e:
        M.mkv_decode_attn_noalloc(layout, pool, huge, torch.zeros(16, device="cuda"), 0.0625,
                                  torch.zeros(16, device="cuda"), None)
    assert e.value.status == -4
