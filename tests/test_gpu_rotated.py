"""Rotated TQ3 pages on the GPU (a sign flip and a Walsh-Hadamard rotation
before the TQ3 rule; oracle/rotation.py).

Bit-exact: the demoted bytes (the rotation's fp32 butterflies run in the
format's stage order on both sides).  Within the attention bar (max-abs 2e-3,
rel-L2 1e-3, lse 1e-3): decode over mixed pools with rotated TQ3 pages,
against the oracle's decode over the same pool definition (dequantise, rotate
back in fp64, dense fp64 attention).  Entry points that do not take rotated
pages refuse them.
"""
import math

import numpy as np
import pytest
import torch

import mixed_format_paged_amd as M
import workloads as W
from workloads.device_cache import DeviceWorkload
from oracle import layout as OL, pool as OP, rotation as OR

from gpu_util import compare, oracle_side

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [128, 256])
def test_demote_rotated_bitexact(d):
    hq, hkv = 24, 4
    rng = np.random.default_rng(40 + d)
    n = 300                                             # more items than one wave of workgroups
    pb = OL.fp8_page_bytes(hkv, d)
    raw = rng.integers(0, 256, (n, pb)).astype(np.uint8)
    raw[(raw & 0x7F) == 0x7F] = 0x7E
    raw[1, :] = 0                                       # all-zero rows
    raw[2, :] &= 0x87                                   # tiny magnitudes
    signs = OR.random_signs(d, d + 1)
    for ks, vs in ((1.0, 1.0), (0.01, 13.0)):
        pool = OP.Pool(hkv, d, n, n, ks, vs, signs=signs)
        pool.fp8[:] = raw
        src = rng.permutation(n)
        dst = n + rng.permutation(n)
        OP.demote(pool, src, dst)
        fp8 = torch.as_tensor(raw, device="cuda")
        tq3 = torch.zeros((n, OL.tq3_page_bytes(hkv, d)), dtype=torch.uint8, device="cuda")
        tier = torch.zeros(2 * n, dtype=torch.uint8, device="cuda")
        sg = torch.as_tensor(signs, device="cuda")
        p = M.make_pool(fp8, tq3, tier, n, n, ks, vs, tq3_signs=sg)
        M.mkv_demote_pages((hq, hkv, d), p, torch.as_tensor(src, dtype=torch.int32, device="cuda"),
                           torch.as_tensor(dst, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        got = tq3.cpu().numpy()
        assert np.array_equal(got, pool.tq3), (ks, vs, np.argwhere(got != pool.tq3)[:5])


ROT = [
    ("tiny-d128", W.WORKLOADS["tiny-1x1024-d128"]),
    ("canary-3L", W.scaled(W.WORKLOADS["canary-2x59008-16L"], L=3, lengths=("fixed", 1500), recent_tokens=256)),
    ("ragged-7", W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=7,
                          lengths=("list", (1, 17, 0, 300, 1031, 2000, 16)), recent_tokens=64)),
    ("demote-4x2048", W.scaled(W.WORKLOADS["demote-64x32768"], B=4, lengths=("fixed", 2048), aging_pages=16)),
    ("heads-32q-4kv", W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3, Hq=32, Hkv=4,
                               lengths=("list", (500, 0, 1025)), recent_tokens=64)),
    ("heads-16q-2kv-d128", W.scaled(W.WORKLOADS["tiny-1x1024-d128"], B=2, Hq=16, Hkv=2,
                                    lengths=("list", (257, 1200)), recent_tokens=32)),
]


@pytest.mark.parametrize("name,w", ROT, ids=[r[0] for r in ROT])
def test_rotated_decode_parity(name, w):
    st = W.make_structure(w)
    # layer 1 (if any) keeps plain TQ3 pages: mixed tables in one launch
    signs = [OR.random_signs(w.d, 100 + li) if li != 1 else None for li in range(w.L)]
    dw = DeviceWorkload(w, st, "cuda", keep_values=True, gen_device="cpu", tq3_signs=signs)
    ref = oracle_side(w, st, dw.values, signs)
    dw.step_demote()
    assert np.array_equal(dw.bt.cpu().numpy(), ref[0][1])
    for li in range(w.L):
        assert np.array_equal(dw.cache.tq3[li].cpu().numpy()[:st.n_tq3], ref[li][0].tq3), f"layer {li} bytes"
    layout = (w.Hq, w.Hkv, w.d)
    L = w.L
    ws = torch.empty(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), L), dtype=torch.uint8, device="cuda")
    out = torch.full((L, w.B, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((L, w.B, w.Hq), float("nan"), device="cuda")
    M.mkv_decode_attn_layers(layout, dw.cache.pools, dw.batch(), dw.q, 1 / math.sqrt(w.d), out, lse, ws)
    torch.cuda.synchronize()
    assert M.mkv_workspace_status(ws) == 0
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for li, (_, _, o_ref, lse_ref) in enumerate(ref):
        compare(o[li], o_ref, l[li], lse_ref, f"{name} layer {li}")
    # the per-layer phase-split path (plan, partials, merge) gives the same bits as the fused call
    for li in range(L):
        ws1 = torch.empty(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
        o1 = torch.empty((w.B, w.Hq, w.d), device="cuda")
        l1 = torch.empty((w.B, w.Hq), device="cuda")
        M.mkv_decode_attn(layout, dw.cache.pools[li], dw.batch(), dw.q[li].contiguous(), 1 / math.sqrt(w.d), o1, l1, ws1)
        o2 = torch.empty_like(o1)
        l2 = torch.empty_like(l1)
        M.mkv_attend(layout, [dw.cache.pools[li]], dw.batch(), dw.q[li].contiguous(), 1 / math.sqrt(w.d), o2, l2, ws1)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        compare(o1.cpu().numpy(), ref[li][2], l1.cpu().numpy(), ref[li][3], f"{name} single layer {li}")


def test_rotated_pools_refused_where_unsupported():
    w = W.scaled(W.WORKLOADS["batch-8x16384"], B=2, lengths=("fixed", 300), recent_tokens=64)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda", tq3_signs=[OR.random_signs(w.d, 1)])
    layout = (w.Hq, w.Hkv, w.d)
    T = 2
    ws = torch.empty(M.mkv_decode_workspace_bytes_multi(layout, w.B, dw.bt.numel(), 1, T), dtype=torch.uint8,
                     device="cuda")
    q = torch.zeros((1, w.B, T, w.Hq, w.d), device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(M.MkvError):
        M.mkv_decode_attn_multi(layout, dw.cache.pools, dw.batch(), q, 0.0625, out, None, ws)
    K = torch.empty((16, w.Hkv, w.d), dtype=torch.int16, device="cuda")
    with pytest.raises(M.MkvError):
        M.mkv_materialize(layout, dw.cache.pools[0], dw.batch(), 0, 0, 1, K, K.clone())
    M.set_partial_kind(0)
    try:
        ws1 = torch.empty(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
        o1 = torch.empty((w.B, w.Hq, w.d), device="cuda")
        with pytest.raises(M.MkvError):
            M.mkv_decode_attn(layout, dw.cache.pools[0], dw.batch(), dw.q[0].contiguous(), 0.0625, o1, None, ws1)
    finally:
        M.set_partial_kind(1)
