"""Decode parity with per-layer FP8 scales other than 1.

Recent and Anchor pages are FP8 with one k_scale and one v_scale per layer
(arXiv 2608.23834, page 1, Abstract; FP8 values are decode(byte) * scale), and
stale pages are demoted from those FP8 values, so their TQ3 scales carry the
layer's scale too.  The values are drawn in the units of the scales (K times
k_scale, V times v_scale, with a few V entries at +-440 v_scale, near the top
of the FP8 range, and q divided by k_scale), so large v_scale values give
TQ3 V scales up to fp16(448 v_scale / 3): the range where u s no longer fits
fp16.

Bar: attention is linear in V, so out / v_scale is held to the unit-scale bar
(max-abs 2e-3, rel-L2 1e-3) against the oracle's out / v_scale; lse to 1e-3.
Covered: the matrix-core and VALU kernels, single-query decode of several
workloads, the in-launch append, multi-query decode (8- and 16-row blocks),
groups of 9..16 query heads and a rotated layer.
"""
import math

import numpy as np
import pytest
import torch

import mixed_format_paged_amd as M
import workloads as W
from workloads.device_cache import DeviceWorkload
from oracle import attention as OA, pool as OP, rotation as OR

from gpu_util import compare, in_units, oracle_side

pytestmark = pytest.mark.gpu

# (k_scale, v_scale): ordinary, tiny (fp16-subnormal TQ3 scales), large (TQ3
# V products past the fp16 range: a 2^-1 shift), V only very large (2^-3)
SCALES = [(0.37, 2.5), (0.02, 0.05), (100.0, 100.0), (2.0, 300.0)]


@pytest.fixture(params=["mfma", "valu"])
def kind(request):
    M.set_partial_kind(1 if request.param == "mfma" else 0)
    yield request.param
    M.set_partial_kind(1)


def _built(w, ks, vs, signs=None, sat_frac=0.003):
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda", keep_values=True, gen_device="cpu", k_scale=ks, v_scale=vs,
                        value_fn=in_units(ks, vs, seed=7, sat_frac=sat_frac), tq3_signs=signs)
    ref = oracle_side(w, st, dw.values, signs, k_scale=ks, v_scale=vs)
    dw.step_demote()
    assert np.array_equal(dw.bt.cpu().numpy(), ref[0][1])
    for li in range(w.L):
        assert np.array_equal(dw.cache.tq3[li].cpu().numpy()[:st.n_tq3], ref[li][0].tq3), f"layer {li} TQ3 bytes"
    return st, dw, ref


def _decode(dw):
    w = dw.w
    L = len(dw.layers)
    layout = (w.Hq, w.Hkv, w.d)
    ws = torch.empty(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), L), dtype=torch.uint8, device="cuda")
    out = torch.full((L, w.B, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((L, w.B, w.Hq), float("nan"), device="cuda")
    M.mkv_decode_attn_layers(layout, dw.cache.pools, dw.batch(), dw.q, 1 / math.sqrt(w.d), out, lse, ws)
    assert M.mkv_workspace_status(ws) == 0
    return out.cpu().numpy(), lse.cpu().numpy()


# (name, workload, fraction of V entries at +-440 v_scale).  The outlier
# recipe's scores reach tens of nats (lse up to ~60 at d = 128), where the
# fp32 rounding of a score alone (~1e-5) times a V entry of 440 is past the
# bar for any fp32 kernel, so that workload keeps its V values as drawn; the
# log-normal workloads (scores of a few nats) carry the saturated entries.
WL = [
    ("batch-4x1024", W.scaled(W.WORKLOADS["batch-8x16384"], B=4, lengths=("fixed", 1024), recent_tokens=128), 0.003),
    ("ragged-5-d128", W.scaled(W.WORKLOADS["tiny-1x1024-d128"], B=5, L=2,
                               lengths=("list", (1031, 0, 17, 600, 2048)), recent_tokens=64, random_anchor_frac=0.05),
     0.0),
]


@pytest.mark.parametrize("ks,vs", SCALES, ids=[f"k{a}-v{b}" for a, b in SCALES])
@pytest.mark.parametrize("name,w,sat", WL, ids=[x[0] for x in WL])
def test_decode_scales(name, w, sat, ks, vs, kind):
    st, dw, ref = _built(w, ks, vs, sat_frac=sat)
    out, lse = _decode(dw)
    assert np.isfinite(out).all()
    for li, (_, _, o_ref, lse_ref) in enumerate(ref):
        compare(out[li] / vs, o_ref / vs, lse[li], lse_ref, f"{name} k{ks} v{vs} layer {li}")


@pytest.mark.parametrize("ks,vs", SCALES, ids=[f"k{a}-v{b}" for a, b in SCALES])
def test_append_attend_scales(ks, vs):
    """The in-launch append encodes the new token with the layer's scales,
    and decode over it matches the oracle (append, then attention)."""
    M.set_partial_kind(1)
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3, L=2, lengths=("list", (2000, 17, 1025)), recent_tokens=64)
    st, dw, ref = _built(w, ks, vs)
    layout = (w.Hq, w.Hkv, w.d)
    L, B = w.L, w.B
    g = torch.Generator()
    g.manual_seed(5)
    k_new = torch.randn((L, B, w.Hkv, w.d), generator=g) * 2 * ks
    v_new = torch.randn((L, B, w.Hkv, w.d), generator=g) * 2 * vs
    ws = torch.empty(M.mkv_decode_workspace_bytes(layout, B, dw.bt.numel(), L), dtype=torch.uint8, device="cuda")
    out = torch.full((L, B, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((L, B, w.Hq), float("nan"), device="cuda")
    M.mkv_decode_plan(layout, dw.cache.pools[0], dw.batch(), L, ws)
    M.mkv_append_attend(layout, dw.cache.pools, dw.batch(), k_new.cuda().contiguous(), v_new.cuda().contiguous(),
                        dw.q, 1 / math.sqrt(w.d), out, lse, ws)
    assert M.mkv_workspace_status(ws) == 0
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for li, (pool, bt, _, _) in enumerate(ref):
        OP.append(pool, k_new[li].numpy()[:, None], v_new[li].numpy()[:, None], st.bt_offsets, bt, st.seq_lens - 1)
        assert np.array_equal(dw.cache.fp8[li].cpu().numpy(), pool.fp8), f"layer {li} FP8 bytes"
        o_ref, l_ref = OA.decode_batch(pool, dw.values[li]["q"].numpy(), st.bt_offsets, bt, st.seq_lens)
        compare(o[li] / vs, o_ref / vs, l[li], l_ref, f"append k{ks} v{vs} layer {li}")


@pytest.mark.parametrize("ks,vs", SCALES, ids=[f"k{a}-v{b}" for a, b in SCALES])
@pytest.mark.parametrize("T,hq,hkv", [(1, 40, 4), (1, 12, 1), (1, 64, 4), (3, 24, 4), (2, 4, 2)])
def test_multi_query_and_wide_groups_scales(T, hq, hkv, ks, vs):
    """Multi-query decode (rows T G in 8- or 16-row blocks) and single-query
    decode with 9..16 query heads per KV head (16-row blocks), with scales."""
    M.set_partial_kind(1)
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3, L=2, Hq=hq, Hkv=hkv,
                 lengths=("list", (1500, 5, 700)), recent_tokens=16)
    st, dw, ref = _built(w, ks, vs)
    layout = (w.Hq, w.Hkv, w.d)
    L, B = w.L, w.B
    g = torch.Generator()
    g.manual_seed(200 + T)
    q = torch.randn((L, B, T, w.Hq, w.d), generator=g) / ks      # scores of unit size, as in in_units
    ws = torch.empty(M.mkv_decode_workspace_bytes_multi(layout, B, dw.bt.numel(), L, T), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((L, B, T, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((L, B, T, w.Hq), float("nan"), device="cuda")
    M.mkv_decode_attn_multi(layout, dw.cache.pools, dw.batch(), q.cuda().contiguous(), 1 / math.sqrt(w.d), out, lse,
                            ws)
    assert M.mkv_workspace_status(ws) == 0
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for li, (pool, bt, _, _) in enumerate(ref):
        o_ref, l_ref = OA.decode_batch_multi(pool, q[li].numpy(), st.bt_offsets, bt, st.seq_lens)
        compare(o[li].reshape(-1, w.d) / vs, o_ref.reshape(-1, w.d) / vs, l[li].reshape(-1), l_ref.reshape(-1),
                f"T={T} {hq}/{hkv} k{ks} v{vs} layer {li}")


@pytest.mark.parametrize("ks,vs", SCALES, ids=[f"k{a}-v{b}" for a, b in SCALES])
def test_rotated_layer_scales(ks, vs):
    M.set_partial_kind(1)
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3, L=2, lengths=("list", (1200, 40, 2100)), recent_tokens=64)
    signs = [OR.random_signs(w.d, 300), None]
    st, dw, ref = _built(w, ks, vs, signs)
    out, lse = _decode(dw)
    for li, (_, _, o_ref, lse_ref) in enumerate(ref):
        compare(out[li] / vs, o_ref / vs, lse[li], lse_ref, f"rotated k{ks} v{vs} layer {li}")
