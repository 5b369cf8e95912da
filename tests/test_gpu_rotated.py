"""Rotated TQ3 pages on the GPU (a sign flip and a Walsh-Hadamard rotation
before the TQ3 rule; oracle/rotation.py).

Bit-exact: the demoted bytes (the rotation's fp32 butterflies run in the
format's stage order on both sides).  Within the attention bar (max-abs 2e-3,
rel-L2 1e-3, lse 1e-3): decode over mixed pools with rotated TQ3 pages,
single-query (8- and 16-row items) and multi-query, against the oracle's
decode over the same pool definition (dequantise, rotate back in fp64, dense
fp64 attention).  The VALU baseline kernels refuse rotated pools.
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
    # more than 8 query heads per KV head: the 16-row items
    ("heads-40q-4kv", W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=2, L=2, Hq=40, Hkv=4,
                               lengths=("list", (900, 333)), recent_tokens=64)),
    ("heads-32q-2kv-d128", W.scaled(W.WORKLOADS["tiny-1x1024-d128"], B=2, Hq=32, Hkv=2,
                                    lengths=("list", (600, 1100)), recent_tokens=32)),
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


@pytest.mark.parametrize("T,d,hq,hkv", [(2, 256, 24, 4), (5, 128, 16, 2), (3, 256, 8, 8)])
def test_rotated_multi_query_decode_parity(T, d, hq, hkv):
    """mkv_decode_attn_multi over rotated TQ3 pages (layer 0 rotated, layer 1
    plain, one launch): each request's last T tokens as causal queries against
    the oracle's decode over the same pool definition; rows per KV head T G =
    12 (16-row block), 40 (16-row blocks, the last part-filled) and 3 (8-row
    block).  recent = 16 tokens puts logical page n - 2 in TQ3, so the causal
    mask also runs on a rotated page."""
    from oracle import attention as OA
    M.set_partial_kind(1)
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=4, L=2, d=d, Hq=hq, Hkv=hkv,
                 lengths=("list", (1300, 2, 0, 517)), recent_tokens=16)
    st = W.make_structure(w)
    signs = [OR.random_signs(d, 300 + T), None]
    dw = DeviceWorkload(w, st, "cuda", keep_values=True, gen_device="cpu", tq3_signs=signs)
    ref = oracle_side(w, st, dw.values, signs)
    layout = (w.Hq, w.Hkv, w.d)
    L, B = 2, w.B
    g = torch.Generator()
    g.manual_seed(200 + T)
    q = torch.randn((L, B, T, w.Hq, w.d), generator=g)
    ws = torch.empty(M.mkv_decode_workspace_bytes_multi(layout, B, dw.bt.numel(), L, T), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((L, B, T, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((L, B, T, w.Hq), float("nan"), device="cuda")
    M.mkv_decode_attn_multi(layout, dw.cache.pools, dw.batch(), q.to("cuda").contiguous(), 1 / math.sqrt(w.d), out,
                            lse, ws)
    torch.cuda.synchronize()
    assert M.mkv_workspace_status(ws) == 0
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for li, (pool, bt, _, _) in enumerate(ref):
        o_ref, l_ref = OA.decode_batch_multi(pool, q[li].numpy(), st.bt_offsets, bt, st.seq_lens)
        compare(o[li].reshape(-1, w.d), o_ref.reshape(-1, w.d), l[li].reshape(-1), l_ref.reshape(-1),
                f"rotated T={T} d={d} layer {li}")


def test_rotated_pools_refused_by_the_valu_baseline():
    w = W.scaled(W.WORKLOADS["batch-8x16384"], B=2, lengths=("fixed", 300), recent_tokens=64)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda", tq3_signs=[OR.random_signs(w.d, 1)])
    layout = (w.Hq, w.Hkv, w.d)
    M.set_partial_kind(0)
    try:
        ws1 = torch.empty(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
        o1 = torch.empty((w.B, w.Hq, w.d), device="cuda")
        with pytest.raises(M.MkvError):
            M.mkv_decode_attn(layout, dw.cache.pools[0], dw.batch(), dw.q[0].contiguous(), 0.0625, o1, None, ws1)
    finally:
        M.set_partial_kind(1)
