"""Decode under HIP graph capture: mkv_decode_attn_layers, mkv_append_attend
(the step's new token appended inside the attention launch) and
mkv_decode_attn_noalloc are captured once and replayed several times, with
eager work and a synchronisation between replays; every replay's outputs
equal the eager call's bytes and the device status stays 0.  (The library
records no memset into a captured graph: everything it clears, it clears
with its own kernels.)"""
import math

import numpy as np
import pytest
import torch

import mixed_format_paged_amd as M
import workloads as W
from workloads.device_cache import DeviceWorkload

pytestmark = pytest.mark.gpu


def _setup():
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3, L=2, lengths=("list", (1500, 40, 2600)),
                 recent_tokens=64)
    st = W.make_structure(w)
    return w, DeviceWorkload(w, st, "cuda")


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(g, outs, refs, ws=None, reps=4):
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(reps):
        for t in outs:
            t.fill_(float("nan"))
        junk.mul_(1.0001)                          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert np.array_equal(t.cpu().numpy(), r), rep
        if ws is not None:
            assert M.mkv_workspace_status(ws) == 0, rep


def test_decode_layers_and_append_attend_replays_match_eager():
    w, dw = _setup()
    layout, L, sm = (w.Hq, w.Hkv, w.d), 2, 1 / math.sqrt(w.d)
    ws = torch.empty(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), L), dtype=torch.uint8, device="cuda")
    out = torch.empty((L, w.B, w.Hq, w.d), device="cuda")
    lse = torch.empty((L, w.B, w.Hq), device="cuda")

    def decode():
        M.mkv_decode_attn_layers(layout, dw.cache.pools, dw.batch(), dw.q, sm, out, lse, ws)

    decode()
    torch.cuda.synchronize()
    ref = [out.cpu().numpy().copy(), lse.cpu().numpy().copy()]
    _replays_match(_capture(decode), [out, lse], ref, ws)

    # the step's new token appended inside the attention launch, layer by layer
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    k_new = torch.randn((L, w.B, 1, w.Hkv, w.d), generator=gen, device="cuda")
    v_new = torch.randn((L, w.B, 1, w.Hkv, w.d), generator=gen, device="cuda")
    q = [dw.q[l].contiguous() for l in range(L)]
    ws1 = torch.empty(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), 1), dtype=torch.uint8,
                      device="cuda")
    o1 = torch.empty((L, w.B, w.Hq, w.d), device="cuda")
    l1 = torch.empty((L, w.B, w.Hq), device="cuda")

    def append_attend():                           # as a decode step: one plan, then the layers
        M.mkv_decode_plan(layout, dw.cache.pools[0], dw.batch(), 1, ws1)
        for l in range(L):
            M.mkv_append_attend(layout, [dw.cache.pools[l]], dw.batch(), k_new[l], v_new[l], q[l], sm, o1[l], l1[l],
                                ws1)

    append_attend()
    torch.cuda.synchronize()
    ref1 = [o1.cpu().numpy().copy(), l1.cpu().numpy().copy()]
    _replays_match(_capture(append_attend), [o1, l1], ref1, ws1)


def test_noalloc_decode_replays_match_eager():
    w, dw = _setup()
    layout, sm = (w.Hq, w.Hkv, w.d), 1 / math.sqrt(w.d)
    q0 = dw.q[0].contiguous()
    out = torch.empty((w.B, w.Hq, w.d), device="cuda")
    lse = torch.empty((w.B, w.Hq), device="cuda")

    def decode():
        M.mkv_decode_attn_noalloc(layout, dw.cache.pools[0], dw.batch(), q0, sm, out, lse)

    decode()
    torch.cuda.synchronize()
    ref = [out.cpu().numpy().copy(), lse.cpu().numpy().copy()]
    _replays_match(_capture(decode), [out, lse], ref)
