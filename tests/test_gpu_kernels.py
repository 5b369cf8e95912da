"""GPU parity: the HIP path (through the C ABI) against the oracle.

Bit-exact: append (FP8 bytes), demote (TQ3 bytes), page-table gather.
Attention: max-abs <= 2e-3 and rel-L2 <= 1e-3 on out, |lse| <= 1e-3, on the
same quantised inputs, for small versions of every workload shape, ragged
and empty requests, tails in either format and a multi-level merge.
"""
import math

import numpy as np
import pytest
import torch

import mixed_format_paged_amd as M
import workloads as W
from workloads.device_cache import DeviceWorkload
from oracle import attention as OA, build as OB, fp8 as OF, layout as OL, pool as OP

from gpu_util import compare, oracle_side

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["mfma", "valu"])
def kind(request):
    """Run a decode test with the matrix-core kernels and with the VALU baseline."""
    M.set_partial_kind(1 if request.param == "mfma" else 0)
    yield request.param
    M.set_partial_kind(1)


def _decode(dw, sm_scale=None):
    w = dw.w
    L = len(dw.layers)
    layout = (w.Hq, w.Hkv, w.d)
    wsb = M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), L)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.full((L, w.B, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((L, w.B, w.Hq), float("nan"), device="cuda")
    M.mkv_decode_attn_layers(layout, dw.cache.pools, dw.batch(), dw.q, sm_scale or 1 / math.sqrt(w.d), out, lse, ws)
    status = M.mkv_workspace_status(ws)
    return out.cpu().numpy(), lse.cpu().numpy(), status


def _both(w, layers=None):
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda", layers=layers, keep_values=True, gen_device="cpu")
    ref = oracle_side(w, st, dw.values)
    return st, dw, ref


def test_append_bitexact_edge_values():
    hq, hkv, d = 8, 2, 128
    rng = np.random.default_rng(0)
    special = np.array([0.0, -0.0, 448.0, -448.0, 449.0, 463.9, 464.0, 1e30, -1e30, 2.0 ** -9, 2.0 ** -10,
                        1.5 * 2.0 ** -9, 2.0 ** -6, 0.9 * 2.0 ** -6, 1.0625, 1.1875, 3e-8], dtype=np.float32)
    n_tok = 40
    k = (rng.standard_normal((1, n_tok, hkv, d)) * np.exp(rng.uniform(-8, 6, (1, n_tok, hkv, 1)))).astype(np.float32)
    v = (rng.standard_normal((1, n_tok, hkv, d)) * 50).astype(np.float32)
    k.reshape(-1)[:len(special)] = special
    v.reshape(-1)[-len(special):] = special
    for ks, vs in ((1.0, 1.0), (0.37, 2.5)):
        pool = OP.Pool(hkv, d, 4, 1, ks, vs)
        pages = np.array([2, 0, 3], dtype=np.int64)
        OP.append(pool, k, v, [0, 3], pages, [5])
        fp8 = torch.zeros((4, OL.fp8_page_bytes(hkv, d)), dtype=torch.uint8, device="cuda")
        tq3 = torch.zeros((1, OL.tq3_page_bytes(hkv, d)), dtype=torch.uint8, device="cuda")
        tier = torch.zeros(5, dtype=torch.uint8, device="cuda")
        p = M.make_pool(fp8, tq3, tier, 4, 1, ks, vs)
        dev = lambda a, dt=torch.int32: torch.as_tensor(np.asarray(a), dtype=dt, device="cuda")
        M.mkv_append((hq, hkv, d), p, dev(k, torch.float32), dev(v, torch.float32), dev([0, 3]), dev(pages), dev([5]))
        torch.cuda.synchronize()
        assert np.array_equal(fp8.cpu().numpy(), pool.fp8), (ks, vs)


@pytest.mark.parametrize("d", [128, 256])
def test_demote_bitexact_random_bytes(d):
    hq, hkv = 24, 4
    rng = np.random.default_rng(d)
    n = 9
    pb = OL.fp8_page_bytes(hkv, d)
    raw = rng.integers(0, 256, (n, pb)).astype(np.uint8)
    raw[(raw & 0x7F) == 0x7F] = 0x7E                    # NaN codes are outside the contract
    raw[1, :] = 0                                       # all-zero groups (s = 0)
    raw[2, :] &= 0x87                                   # tiny magnitudes only (subnormal e4m3, fp16 subnormal scales)
    raw[3, ::7] = 0x7E                                  # saturated maxima
    raw[4, :] &= 0x9F                                   # magnitudes below 0.12: thresholds on both sides of 2^-6
    raw[5, :] &= 0x8F                                   # magnitudes below 0.03
    for ks, vs in ((1.0, 1.0), (0.001, 37.0), (2.0 ** -20, 1500.0)):
        pool = OP.Pool(hkv, d, n, n, ks, vs)
        pool.fp8[:] = raw
        src = np.arange(n)
        dst = n + rng.permutation(n)
        OP.demote(pool, src, dst)
        fp8 = torch.as_tensor(raw, device="cuda")
        tq3 = torch.zeros((n, OL.tq3_page_bytes(hkv, d)), dtype=torch.uint8, device="cuda")
        tier = torch.zeros(2 * n, dtype=torch.uint8, device="cuda")
        p = M.make_pool(fp8, tq3, tier, n, n, ks, vs)
        M.mkv_demote_pages((hq, hkv, d), p, torch.as_tensor(src, dtype=torch.int32, device="cuda"),
                           torch.as_tensor(dst, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        got = tq3.cpu().numpy()
        assert np.array_equal(got, pool.tq3), (ks, vs, np.argwhere(got != pool.tq3)[:5])


@pytest.mark.parametrize("d", [128, 256])
def test_demote_layers_many_items(d):
    # several thousand (layer, page, head) items, more than the workgroups the
    # GPU holds at once, so each workgroup takes several items and prefetches;
    # three layers with their own scales in one launch, ids permuted
    hq, hkv, n, L = 24, 4, 700, 3
    rng = np.random.default_rng(100 + d)
    pb = OL.fp8_page_bytes(hkv, d)
    scales = [(1.0, 1.0), (0.25, 3.0), (7.0, 0.5)]
    raws, pools, ref = [], [], []
    src = rng.permutation(n)[: n - 50]                   # not every FP8 slot, in random order
    dst = n + rng.permutation(n)[: n - 50]
    for l in range(L):
        raw = rng.integers(0, 256, (n, pb)).astype(np.uint8)
        raw[(raw & 0x7F) == 0x7F] = 0x7E
        pool = OP.Pool(hkv, d, n, n, *scales[l])
        pool.fp8[:] = raw
        OP.demote(pool, src, dst)
        ref.append(pool.tq3)
        fp8 = torch.as_tensor(raw, device="cuda")
        tq3 = torch.zeros((n, OL.tq3_page_bytes(hkv, d)), dtype=torch.uint8, device="cuda")
        tier = torch.zeros(2 * n, dtype=torch.uint8, device="cuda")
        raws.append((fp8, tq3, tier))
        pools.append(M.make_pool(fp8, tq3, tier, n, n, *scales[l]))
    M.mkv_demote_pages_layers((hq, hkv, d), pools, torch.as_tensor(src, dtype=torch.int32, device="cuda"),
                              torch.as_tensor(dst, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for l in range(L):
        got = raws[l][1].cpu().numpy()
        assert np.array_equal(got, ref[l]), (l, np.argwhere(got != ref[l])[:5])


def test_build_gather_and_decode_tiny(kind):
    w = W.WORKLOADS["tiny-1x1024-d128"]
    st, dw, ref = _both(w)
    pool, bt, o_ref, lse_ref = ref[0]
    # gather: logical page bytes, bit-exact
    n = int(st.n_pages[0])
    rec = torch.empty((n, OL.fp8_page_bytes(w.Hkv, w.d)), dtype=torch.uint8, device="cuda")
    M.mkv_debug_gather((w.Hq, w.Hkv, w.d), dw.cache.pools[0], dw.bt_offsets, dw.bt, 0, n, rec)
    torch.cuda.synchronize()
    assert np.array_equal(rec.cpu().numpy(), OP.gather_raw(pool, st.bt_offsets, bt, 0, n))
    assert np.array_equal(dw.bt.cpu().numpy(), bt)
    out, lse, status = _decode(dw)
    assert status == 0
    compare(out[0], o_ref, lse[0], lse_ref, "tiny")


SMALL = [
    # (name, workload)
    ("batch-8x1024", W.scaled(W.WORKLOADS["batch-8x16384"], lengths=("fixed", 1024), recent_tokens=128)),
    ("ragged-7", W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=7,
                          lengths=("list", (1, 17, 0, 300, 1031, 2000, 16)), recent_tokens=64)),
    ("no-recent-tq3-tail", W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3,
                                    lengths=("list", (999, 33, 1)), recent_tokens=0, random_anchor_frac=0.1)),
    ("all-fp8", W.scaled(W.WORKLOADS["batch-8x16384"], B=2, lengths=("fixed", 700), recent_tokens=1024)),
    ("long-1x8192", W.scaled(W.WORKLOADS["long-1x131072"], lengths=("fixed", 8192))),
    ("canary-3L", W.scaled(W.WORKLOADS["canary-2x59008-16L"], L=3, lengths=("fixed", 1500), recent_tokens=256)),
    ("demote-4x2048", W.scaled(W.WORKLOADS["demote-64x32768"], B=4, lengths=("fixed", 2048), aging_pages=16)),
    # other head layouts: a full 8-row group (no padding rows), one query head
    # per KV head, a single KV head
    ("heads-32q-4kv", W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3, Hq=32, Hkv=4,
                               lengths=("list", (500, 0, 1025)), recent_tokens=64)),
    ("heads-8q-8kv-d128", W.scaled(W.WORKLOADS["tiny-1x1024-d128"], B=2, Hq=8, Hkv=8,
                                   lengths=("list", (700, 33)), recent_tokens=64)),
    ("heads-16q-2kv-d128", W.scaled(W.WORKLOADS["tiny-1x1024-d128"], B=2, Hq=16, Hkv=2,
                                    lengths=("list", (257, 1200)), recent_tokens=32)),
    ("heads-3q-1kv", W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=2, Hq=3, Hkv=1,
                              lengths=("list", (64, 800)), recent_tokens=32)),
    # more than 1,024 requests, many of them empty or a part of one page: the
    # plan keeps its per-request offsets in global memory (past its LDS rows)
    # and the attention workgroups each take several work items
    ("batch-1100-short", W.scaled(W.WORKLOADS["tiny-1x1024-d128"], B=1100,
                                  lengths=("list", tuple((37 * i) % 120 for i in range(1100))), recent_tokens=32)),
]


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
def test_decode_parity_small(name, w, kind):
    st, dw, ref = _both(w)
    dw.step_demote()
    assert np.array_equal(dw.bt.cpu().numpy(), ref[0][1])
    out, lse, status = _decode(dw)
    assert status == 0
    for li, (_, _, o_ref, lse_ref) in enumerate(ref):
        compare(out[li], o_ref, lse[li], lse_ref, f"{name} layer {li}")


def test_multilayer_equals_per_layer_and_is_deterministic(kind):
    w = W.scaled(W.WORKLOADS["canary-2x59008-16L"], L=3, lengths=("fixed", 900), recent_tokens=128)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda")
    out, lse, _ = _decode(dw)
    for _ in range(5):
        o2, l2, _ = _decode(dw)
        assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    layout = (w.Hq, w.Hkv, w.d)
    for li in range(3):
        wsb = M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), 1)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        o1 = torch.empty((w.B, w.Hq, w.d), device="cuda")
        l1 = torch.empty((w.B, w.Hq), device="cuda")
        M.mkv_decode_attn(layout, dw.cache.pools[li], dw.batch(), dw.q[li].contiguous(), 1 / math.sqrt(w.d), o1, l1, ws)
        torch.cuda.synchronize()
        # chunking differs with the layer count, so agreement is to tolerance
        compare(o1.cpu().numpy(), out[li].astype(np.float64), None, None, f"layer {li}")


def test_device_data_errors_flag_and_nan(kind):
    w = W.scaled(W.WORKLOADS["batch-8x16384"], B=4, lengths=("fixed", 300), recent_tokens=64)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda")
    out0, lse0, status = _decode(dw)
    assert status == 0
    bt_good = dw.bt.clone()
    # request 1: a page id outside the pool
    dw.bt[int(st.bt_offsets[1]) + 3] = st.n_fp8 + st.n_tq3 + 5
    # request 2: an FP8 slot whose tier byte says Stale
    e = int(st.bt_offsets[2]) + int(st.n_pages[2]) - 1
    free_fp8 = int(torch.nonzero(dw.cache.tier[:st.n_fp8] == M.TIER_FREE)[0])
    dw.cache.tier[free_fp8] = M.TIER_STALE
    dw.bt[e] = free_fp8
    # request 3: seq_len longer than its block table
    dw.seq_lens[3] = 300 + 16 * 5
    out, lse, status = _decode(dw)
    assert status == (1 | 2 | 4)
    assert np.all(np.isnan(out[0, 1:4])) and np.all(np.isnan(lse[0, 1:4]))
    assert np.array_equal(out[0, 0], out0[0, 0]) and np.array_equal(lse[0, 0], lse0[0, 0])
    dw.bt.copy_(bt_good)
    dw.seq_lens[3] = 300
    dw.cache.tier[free_fp8] = M.TIER_FREE
    out, lse, status = _decode(dw)
    assert status == 0 and np.array_equal(out, out0)


def test_phase_split_calls_are_bit_identical(kind):
    """plan + attend_fp8 + attend_tq3 + merge, plan + attend_partials + merge,
    plan + attend, and decode_attn_layers give the same bytes, and match the
    oracle."""
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=5, L=2,
                 lengths=("list", (3000, 17, 0, 1200, 4100)), recent_tokens=64)
    st, dw, ref = _both(w)
    layout = (w.Hq, w.Hkv, w.d)
    L = 2
    sm = 1 / math.sqrt(w.d)
    wsb = M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), L)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    bat = dw.batch()
    outs = []
    for variant in ("separate", "partials", "attend"):
        out = torch.full((L, w.B, w.Hq, w.d), float("nan"), device="cuda")
        lse = torch.full((L, w.B, w.Hq), float("nan"), device="cuda")
        M.mkv_decode_plan(layout, dw.cache.pools[0], bat, L, ws)
        if variant == "separate":
            M.mkv_attend_fp8(layout, dw.cache.pools, bat, dw.q, sm, ws)
            M.mkv_attend_tq3(layout, dw.cache.pools, bat, dw.q, sm, ws)
            M.mkv_merge(layout, L, bat, out, lse, ws)
        elif variant == "partials":
            M.mkv_attend_partials(layout, dw.cache.pools, bat, dw.q, sm, ws)
            M.mkv_merge(layout, L, bat, out, lse, ws)
        else:
            M.mkv_attend(layout, dw.cache.pools, bat, dw.q, sm, out, lse, ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    o4, l4, status = _decode(dw)
    assert status == 0
    outs.append((o4, l4))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
    for li, (_, _, o_ref, lse_ref) in enumerate(ref):
        compare(outs[0][0][li], o_ref, outs[0][1][li], lse_ref, f"layer {li}")


def test_append_attend_equals_append_then_attend():
    """mkv_append_attend writes the same cache bytes and gives the same
    outputs, bit for bit, as mkv_append followed by mkv_attend."""
    M.set_partial_kind(1)
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=4, L=2,
                 lengths=("list", (2000, 17, 1025, 3100)), recent_tokens=64)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda")
    layout = (w.Hq, w.Hkv, w.d)
    L, B = 2, w.B
    sm = 1 / math.sqrt(w.d)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    k_new = torch.randn((L, B, w.Hkv, w.d), generator=g, device="cuda") * 3
    v_new = torch.randn((L, B, w.Hkv, w.d), generator=g, device="cuda") * 3
    pos = (dw.seq_lens - 1).to(torch.int32)
    fp8_0 = [p.clone() for p in dw.cache.fp8]
    wsb = M.mkv_decode_workspace_bytes(layout, B, dw.bt.numel(), L)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    bat = dw.batch()
    res = []
    for fused in (False, True):
        for l in range(L):
            dw.cache.fp8[l].copy_(fp8_0[l])
        out = torch.full((L, B, w.Hq, w.d), float("nan"), device="cuda")
        lse = torch.full((L, B, w.Hq), float("nan"), device="cuda")
        M.mkv_decode_plan(layout, dw.cache.pools[0], bat, L, ws)
        if fused:
            M.mkv_append_attend(layout, dw.cache.pools, bat, k_new, v_new, dw.q, sm, out, lse, ws)
        else:
            for l in range(L):
                M.mkv_append(layout, dw.cache.pools[l], k_new[l].unsqueeze(1).contiguous(),
                             v_new[l].unsqueeze(1).contiguous(), dw.bt_offsets, dw.bt, pos)
            M.mkv_attend(layout, dw.cache.pools, bat, dw.q, sm, out, lse, ws)
        torch.cuda.synchronize()
        assert M.mkv_workspace_status(ws) == 0
        res.append(([s.cpu().numpy() for s in dw.cache.fp8], out.cpu().numpy(), lse.cpu().numpy()))
    for l in range(L):
        assert np.array_equal(res[0][0][l], res[1][0][l]), f"layer {l}: cache bytes differ"
        assert not np.array_equal(res[0][0][l], fp8_0[l].cpu().numpy())   # the append did write
    assert np.array_equal(res[0][1], res[1][1]) and np.array_equal(res[0][2], res[1][2])


@pytest.mark.parametrize("d,scales,rotated", [(128, (0.75, 1.25), False), (256, (1.0, 1.0), False),
                                              (128, (0.75, 1.25), True), (256, (1.0, 1.0), True)])
def test_materialize_bitexact(d, scales, rotated):
    """mkv_materialize on the oracle's own pool bytes equals the oracle's dense
    bf16 bits: whole requests, a range starting inside and running past the
    end of a block table (NaN pages), and an id outside the pool.  rotated:
    the layer's TQ3 pages are rotated TQ3 (dense values through the fp32
    inverse transform)."""
    from oracle import dense as OD, rotation as OR
    w = W.scaled(W.WORKLOADS["tiny-1x1024-d128"], d=d, B=3, lengths=("list", (1024, 300, 17)))
    st = W.make_structure(w)
    vals = W.layer_values(w, st, 0)
    signs = OR.random_signs(d, 17) if rotated else None
    pool, bt = OB.build_layer(w, st, [x.numpy() for x in vals["k"]], [x.numpy() for x in vals["v"]], *scales,
                              signs=signs)
    bt = bt.copy()
    bt[int(st.bt_offsets[2])] = pool.n_fp8 + pool.n_tq3 + 3          # request 2, page 0: not in the pool
    dev = "cuda"
    fp8_d = torch.from_numpy(pool.fp8).to(dev)
    tq3_d = torch.from_numpy(pool.tq3).to(dev)
    tier_d = torch.from_numpy(pool.tier).to(dev)
    sg = None if signs is None else torch.as_tensor(signs, device=dev)
    pd = M.make_pool(fp8_d, tq3_d, tier_d, pool.n_fp8, pool.n_tq3, *scales, tq3_signs=sg)
    batch = M.make_batch(torch.as_tensor(st.bt_offsets, dtype=torch.int32, device=dev),
                         torch.as_tensor(bt, dtype=torch.int32, device=dev),
                         torch.as_tensor(st.seq_lens, dtype=torch.int32, device=dev))
    layout = (w.Hq, w.Hkv, w.d)
    n = [int(x) for x in st.n_pages]
    for b, lo, cnt in [(0, 0, n[0]), (1, 5, n[1] - 5 + 3), (2, 0, n[2]), (0, n[0] - 1, 1)]:
        K = torch.full((cnt * 16, w.Hkv, w.d), 0x1234, dtype=torch.int16, device=dev)
        V = torch.full_like(K, 0x1234)
        M.mkv_materialize(layout, pd, batch, b, lo, cnt, K, V)
        torch.cuda.synchronize()
        Kr, Vr = OD.materialize(pool, st.bt_offsets, bt, b, lo, cnt)
        assert np.array_equal(K.cpu().numpy().view(np.uint16), Kr), (b, lo, cnt)
        assert np.array_equal(V.cpu().numpy().view(np.uint16), Vr), (b, lo, cnt)
    assert (Kr[:16] != OD.BF16_NAN).all()
    with pytest.raises(M.MkvError):
        M.mkv_materialize(layout, pd, batch, 3, 0, 1, K, V)                  # b outside the batch


@pytest.mark.parametrize("rotated", [False, True])
def test_lifecycle_steps_match_the_oracle(rotated):
    """mkv_lifecycle_step (+ the step's mkv_append) from the same start state as
    the oracle: block table, seq_lens, tier map, free stacks, tops and every
    slab byte agree bit for bit at every checkpoint; an anchor set by the
    caller stays FP8; a request released mid-way regrows from zero (ragged
    lengths); a step that cannot get free pages changes nothing.  rotated:
    layer 0 demotes to rotated TQ3, layer 1 to plain TQ3, in the same launch."""
    from oracle import lifecycle as LC, rotation as ORot
    hq, hkv, d, R, L, B, cap, n_fp8, n_tq3 = 4, 2, 128, 3, 2, 3, 12, 14, 30
    layout = (hq, hkv, d)
    rng = np.random.default_rng(7)
    tier = np.full(n_fp8 + n_tq3, OP.TIER_FREE, dtype=np.uint8)
    signs = [ORot.random_signs(d, 31) if rotated else None, None]
    pools = [OP.Pool(hkv, d, n_fp8, n_tq3, tier=tier, signs=signs[l]) for l in range(L)]
    t = LC.Tables(np.arange(B + 1) * cap, np.full(B * cap, -1), np.zeros(B, dtype=np.int64), tier,
                  rng.permutation(n_fp8), n_fp8 + rng.permutation(n_tq3), [n_fp8, n_tq3])
    dev = "cuda"
    i32 = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.int32, device=dev).contiguous()
    fp8_d = [torch.from_numpy(p.fp8).to(dev) for p in pools]
    tq3_d = [torch.from_numpy(p.tq3).to(dev) for p in pools]
    tier_d = torch.from_numpy(tier).to(dev)
    signs_d = [None if sg is None else torch.from_numpy(sg).to(dev) for sg in signs]
    pd = [M.make_pool(fp8_d[l], tq3_d[l], tier_d, n_fp8, n_tq3, tq3_signs=signs_d[l]) for l in range(L)]
    offs_d, bt_d, sl_d = i32(t.bt_offsets), i32(t.bt_pages), i32(t.seq_lens)
    ff_d, tf_d, tops_d = i32(t.fp8_free), i32(t.tq3_free), i32(t.tops)
    ws = torch.zeros(M.mkv_lifecycle_workspace_bytes(B), dtype=torch.uint8, device=dev)

    def same(what):
        torch.cuda.synchronize()
        assert np.array_equal(bt_d.cpu().numpy(), t.bt_pages), what
        assert np.array_equal(sl_d.cpu().numpy(), t.seq_lens), what
        assert np.array_equal(tier_d.cpu().numpy(), tier), what
        assert list(tops_d.cpu().numpy()) == list(t.tops), what
        assert np.array_equal(ff_d.cpu().numpy()[:t.tops[0]], t.fp8_free[:t.tops[0]]), what
        assert np.array_equal(tf_d.cpu().numpy()[:t.tops[1]], t.tq3_free[:t.tops[1]]), what
        for l in range(L):
            assert np.array_equal(fp8_d[l].cpu().numpy(), pools[l].fp8), (what, l)
            assert np.array_equal(tq3_d[l].cpu().numpy(), pools[l].tq3), (what, l)

    def step_both(what, append=None):
        assert LC.step(pools, t, R) == 0, what
        M.mkv_lifecycle_step(layout, pd, offs_d, bt_d, sl_d, tier_d, ff_d, tf_d, tops_d, R, ws)
        assert M.mkv_workspace_status(ws) == 0, what
        if append is None:
            return
        kk, vv = append
        for l in range(L):
            OP.append(pools[l], kk[l], vv[l], t.bt_offsets, t.bt_pages, t.seq_lens - 1)
            M.mkv_append(layout, pd[l], torch.from_numpy(kk[l].copy()).to(dev),
                         torch.from_numpy(vv[l].copy()).to(dev), offs_d, bt_d, sl_d - 1)

    T = 150
    k = rng.standard_normal((L, B, T, 1, hkv, d)).astype(np.float32) * 3
    v = rng.standard_normal((L, B, T, 1, hkv, d)).astype(np.float32) * 3
    for step in range(T):
        step_both(f"step {step}", (k[:, :, step], v[:, :, step]))
        if step == 30:                              # the caller protects request 0's page 1
            pid = int(t.bt_pages[t.bt_offsets[0] + 1])
            assert tier[pid] == OP.TIER_R
            tier[pid] = OP.TIER_A
            tier_d[pid] = OP.TIER_A
        if step == 60:                              # request 2 ends; its slot regrows from zero
            assert LC.release(pools[0], t, [2]) == 0
            M.mkv_lifecycle_release(layout, pd[0], offs_d, bt_d, sl_d, tier_d, ff_d, tf_d, tops_d, i32([2]), ws)
            assert M.mkv_workspace_status(ws) == 0
        if step % 16 in (0, 15) or step == 60 or step == T - 1:
            same(f"step {step}")
    assert list(t.seq_lens) == [T, T, T - 61]
    # up to a page boundary of requests 0 and 1, then a step with one free FP8 id
    for i in range((16 - T % 16) % 16):
        step_both(f"advance {i}")
    t.tops[0] = 1
    tops_d[0] = 1
    same("before the failing step")
    assert LC.step(pools, t, R) == LC.NO_FREE_PAGE
    M.mkv_lifecycle_step(layout, pd, offs_d, bt_d, sl_d, tier_d, ff_d, tf_d, tops_d, R, ws)
    assert M.mkv_workspace_status(ws) == LC.NO_FREE_PAGE
    same("after the failing step")


def test_attend_on_a_workspace_without_a_plan_is_refused(kind):
    """The phase calls need a plan from mkv_decode_plan in their workspace.  On
    a zeroed workspace (no plan stamp) the partial kernels read nothing, the
    merge writes NaN and the status gets MKV_DEV_NO_PLAN; after a plan the
    same call decodes normally."""
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=3, L=1, lengths=("list", (900, 40, 1600)),
                 recent_tokens=64)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda")
    layout, sm = (w.Hq, w.Hkv, w.d), 1 / math.sqrt(w.d)
    ws = torch.zeros(M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
    out = torch.zeros((1, w.B, w.Hq, w.d), device="cuda")
    lse = torch.zeros((1, w.B, w.Hq), device="cuda")
    q = dw.q[:1].contiguous()
    M.mkv_attend(layout, dw.cache.pools[:1], dw.batch(), q, sm, out, lse, ws)
    status = M.mkv_workspace_status(ws)
    assert status & M.MKV_DEV_NO_PLAN
    assert np.all(np.isnan(out.cpu().numpy())) and np.all(np.isnan(lse.cpu().numpy()))
    M.mkv_decode_plan(layout, dw.cache.pools[0], dw.batch(), 1, ws)
    M.mkv_attend(layout, dw.cache.pools[:1], dw.batch(), q, sm, out, lse, ws)
    assert M.mkv_workspace_status(ws) == 0
    o_ref = torch.empty_like(out[0])
    l_ref = torch.empty_like(lse[0])
    ws2 = torch.empty_like(ws)
    M.mkv_decode_attn(layout, dw.cache.pools[0], dw.batch(), q[0], sm, o_ref, l_ref, ws2)
    torch.cuda.synchronize()
    assert np.array_equal(out[0].cpu().numpy(), o_ref.cpu().numpy())


def test_decode_on_two_streams_with_their_own_workspaces(kind):
    """Decode calls with disjoint workspaces and outputs, enqueued on two
    streams and interleaved, give the same bytes as the same calls run one
    after the other: the library keeps no device state of its own that such
    calls could share."""
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=4, L=2, lengths=("list", (3000, 17, 1500, 2200)),
                 recent_tokens=64)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda")
    layout = (w.Hq, w.Hkv, w.d)
    wsb = M.mkv_decode_workspace_bytes(layout, w.B, dw.bt.numel(), 1)
    ws = [torch.empty(wsb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    out = [torch.full((w.B, w.Hq, w.d), float("nan"), device="cuda") for _ in range(2)]
    lse = [torch.full((w.B, w.Hq), float("nan"), device="cuda") for _ in range(2)]
    q = [dw.q[l].contiguous() for l in range(2)]
    sm = 1 / math.sqrt(w.d)

    def decode(l):
        M.mkv_decode_attn(layout, dw.cache.pools[l], dw.batch(), q[l], sm, out[l], lse[l], ws[l])

    decode(0)
    decode(1)
    torch.cuda.synchronize()
    ref = [(out[l].cpu().numpy().copy(), lse[l].cpu().numpy().copy()) for l in range(2)]
    assert M.mkv_workspace_status(ws[0]) == 0 and M.mkv_workspace_status(ws[1]) == 0
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for l in range(2):
        streams[l].wait_stream(torch.cuda.current_stream())
        out[l].fill_(float("nan"))
        lse[l].fill_(float("nan"))
    for _ in range(5):
        for l in range(2):
            with torch.cuda.stream(streams[l]):
                decode(l)
    torch.cuda.synchronize()
    for l in range(2):
        assert np.array_equal(out[l].cpu().numpy(), ref[l][0]), l
        assert np.array_equal(lse[l].cpu().numpy(), ref[l][1]), l
        assert M.mkv_workspace_status(ws[l]) == 0


def test_multi_query_decode_parity_past_the_plan_lds_rows():
    """Multi-query decode with 1,100 requests of 0 to 119 tokens (several
    shorter than T): the causal-mask rows the items read from the plan
    (previous page's format and index, last page's tokens) come from its
    per-request rows in global memory."""
    M.set_partial_kind(1)
    T = 3
    w = W.scaled(W.WORKLOADS["tiny-1x1024-d128"], B=1100, L=1,
                 lengths=("list", tuple((37 * i) % 120 for i in range(1100))), recent_tokens=16)
    st, dw, ref = _both(w)
    layout = (w.Hq, w.Hkv, w.d)
    B = w.B
    g = torch.Generator()
    g.manual_seed(7)
    q = torch.randn((1, B, T, w.Hq, w.d), generator=g)
    wsb = M.mkv_decode_workspace_bytes_multi(layout, B, dw.bt.numel(), 1, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.full((1, B, T, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((1, B, T, w.Hq), float("nan"), device="cuda")
    M.mkv_decode_attn_multi(layout, dw.cache.pools, dw.batch(), q.to("cuda").contiguous(), 1 / math.sqrt(w.d), out, lse,
                            ws)
    assert M.mkv_workspace_status(ws) == 0
    pool, bt, _, _ = ref[0]
    o_ref, l_ref = OA.decode_batch_multi(pool, q[0].numpy(), st.bt_offsets, bt, st.seq_lens)
    compare(out.cpu().numpy()[0].reshape(-1, w.d), o_ref.reshape(-1, w.d), lse.cpu().numpy()[0].reshape(-1),
            l_ref.reshape(-1), "T=3, 1,100 requests")


def test_lifecycle_past_one_planning_block():
    """mkv_lifecycle_step with 1,100 requests (more than the 1,024 threads of
    its planning workgroup, so every pass runs over two blocks of requests):
    40 steps with appends, a recent window of one page, so that 2,200 pages
    age into TQ3; tables, free stacks and every slab byte agree with the
    oracle bit for bit."""
    from oracle import lifecycle as LC
    hq, hkv, d, R, B, cap = 2, 1, 128, 1, 1100, 4
    n_fp8, n_tq3 = 3 * B, 3 * B
    layout = (hq, hkv, d)
    rng = np.random.default_rng(11)
    tier = np.full(n_fp8 + n_tq3, OP.TIER_FREE, dtype=np.uint8)
    pool = OP.Pool(hkv, d, n_fp8, n_tq3, tier=tier)
    t = LC.Tables(np.arange(B + 1) * cap, np.full(B * cap, -1), np.zeros(B, dtype=np.int64), tier,
                  rng.permutation(n_fp8), n_fp8 + rng.permutation(n_tq3), [n_fp8, n_tq3])
    i32 = lambda x: torch.as_tensor(np.asarray(x), dtype=torch.int32, device="cuda").contiguous()
    fp8_d, tq3_d = torch.from_numpy(pool.fp8).to("cuda"), torch.from_numpy(pool.tq3).to("cuda")
    tier_d = torch.from_numpy(tier).to("cuda")
    pd = M.make_pool(fp8_d, tq3_d, tier_d, n_fp8, n_tq3)
    offs_d, bt_d, sl_d = i32(t.bt_offsets), i32(t.bt_pages), i32(t.seq_lens)
    ff_d, tf_d, tops_d = i32(t.fp8_free), i32(t.tq3_free), i32(t.tops)
    ws = torch.zeros(M.mkv_lifecycle_workspace_bytes(B), dtype=torch.uint8, device="cuda")
    T = 40
    k = rng.standard_normal((B, T, 1, hkv, d)).astype(np.float32) * 3
    v = rng.standard_normal((B, T, 1, hkv, d)).astype(np.float32) * 3
    for step in range(T):
        assert LC.step([pool], t, R) == 0
        M.mkv_lifecycle_step(layout, [pd], offs_d, bt_d, sl_d, tier_d, ff_d, tf_d, tops_d, R, ws)
        assert M.mkv_workspace_status(ws) == 0, step
        kk, vv = k[:, step], v[:, step]
        OP.append(pool, kk, vv, t.bt_offsets, t.bt_pages, t.seq_lens - 1)
        M.mkv_append(layout, pd, torch.from_numpy(kk.copy()).to("cuda"), torch.from_numpy(vv.copy()).to("cuda"),
                     offs_d, bt_d, sl_d - 1)
        if step in (20, T - 1):
            torch.cuda.synchronize()
            assert np.array_equal(bt_d.cpu().numpy(), t.bt_pages), step
            assert np.array_equal(sl_d.cpu().numpy(), t.seq_lens), step
            assert np.array_equal(tier_d.cpu().numpy(), tier), step
            assert list(tops_d.cpu().numpy()) == list(t.tops), step
            assert np.array_equal(ff_d.cpu().numpy()[:t.tops[0]], t.fp8_free[:t.tops[0]]), step
            assert np.array_equal(tf_d.cpu().numpy()[:t.tops[1]], t.tq3_free[:t.tops[1]]), step
            assert np.array_equal(fp8_d.cpu().numpy(), pool.fp8), step
            assert np.array_equal(tq3_d.cpu().numpy(), pool.tq3), step
    assert int((tier == OP.TIER_S).sum()) == 2 * B


@pytest.mark.parametrize("T,d,recent,hq,hkv", [(2, 256, 64, 24, 4), (5, 256, 16, 24, 4), (16, 128, 16, 24, 4),
                                               (3, 128, 64, 24, 4), (4, 256, 16, 4, 2), (2, 128, 16, 16, 2),
                                               (3, 256, 64, 8, 8)])
def test_multi_query_decode_parity(T, d, recent, hq, hkv):
    """mkv_decode_attn_multi: each request's last T tokens as causal queries,
    against the oracle; ragged lengths including a request shorter than T and
    an empty one; recent = 16 tokens puts logical page n - 2 in TQ3, so the
    causal mask runs on a TQ3 page too.  Rows per KV head T G: 12, 30, 96
    and 18 (16-row blocks, the last one part-filled), 8 (one 8-row block,
    full), 16 (one 16-row block, full) and 3."""
    M.set_partial_kind(1)
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=5, L=2, d=d, Hq=hq, Hkv=hkv,
                 lengths=("list", (1500, 3, 0, 700, 33)), recent_tokens=recent)
    st, dw, ref = _both(w)
    layout = (w.Hq, w.Hkv, w.d)
    L, B = 2, w.B
    g = torch.Generator()
    g.manual_seed(100 + T)
    q = torch.randn((L, B, T, w.Hq, w.d), generator=g)
    qd = q.to("cuda").contiguous()
    wsb = M.mkv_decode_workspace_bytes_multi(layout, B, dw.bt.numel(), L, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.full((L, B, T, w.Hq, w.d), float("nan"), device="cuda")
    lse = torch.full((L, B, T, w.Hq), float("nan"), device="cuda")
    M.mkv_decode_attn_multi(layout, dw.cache.pools, dw.batch(), qd, 1 / math.sqrt(w.d), out, lse, ws)
    assert M.mkv_workspace_status(ws) == 0
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for li, (pool, bt, _, _) in enumerate(ref):
        o_ref, l_ref = OA.decode_batch_multi(pool, q[li].numpy(), st.bt_offsets, bt, st.seq_lens)
        compare(o[li].reshape(-1, w.d), o_ref.reshape(-1, w.d), l[li].reshape(-1), l_ref.reshape(-1),
                f"T={T} d={d} layer {li}")
    # a single query token through the same call is the single-query decode, bit for bit
    if T == 2:
        out1 = torch.full((L, B, 1, w.Hq, w.d), float("nan"), device="cuda")
        lse1 = torch.full((L, B, 1, w.Hq), float("nan"), device="cuda")
        M.mkv_decode_attn_multi(layout, dw.cache.pools, dw.batch(), qd[:, :, -1:].contiguous(), 1 / math.sqrt(w.d),
                                out1, lse1, ws)
        wsb1 = M.mkv_decode_workspace_bytes(layout, B, dw.bt.numel(), L)
        ws1 = torch.empty(wsb1, dtype=torch.uint8, device="cuda")
        out2 = torch.full((L, B, w.Hq, w.d), float("nan"), device="cuda")
        lse2 = torch.full((L, B, w.Hq), float("nan"), device="cuda")
        M.mkv_decode_attn_layers(layout, dw.cache.pools, dw.batch(), qd[:, :, -1].contiguous(), 1 / math.sqrt(w.d),
                                 out2, lse2, ws1)
        torch.cuda.synchronize()
        assert np.array_equal(out1[:, :, 0].cpu().numpy(), out2.cpu().numpy())
        assert np.array_equal(lse1[:, :, 0].cpu().numpy(), lse2.cpu().numpy())


def test_append_attend_refuses_a_tq3_last_page():
    """mkv_append_attend needs each request's last logical page to be FP8
    (Recent).  With no recent window the last pages are TQ3 (unless drawn as
    anchors): those requests get NaN outputs and MKV_DEV_BAD_TIER, the others
    decode normally, and a plain decode of the same plan is unaffected."""
    M.set_partial_kind(1)
    w = W.scaled(W.WORKLOADS["ragged-32x4096-65536"], B=4, L=1, lengths=("list", (900, 33, 1, 500)),
                 recent_tokens=0, random_anchor_frac=0.0, fixed_anchor_pages=2)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda")
    layout = (w.Hq, w.Hkv, w.d)
    B = w.B
    last_is_tq3 = np.array([st.tiers[st.bt_offsets[b + 1] - 1] == W.TIER_S for b in range(B)])
    assert last_is_tq3.any() and not last_is_tq3.all()
    ws = torch.empty(M.mkv_decode_workspace_bytes(layout, B, dw.bt.numel(), 1), dtype=torch.uint8, device="cuda")
    out = torch.full((1, B, w.Hq, w.d), 0.0, device="cuda")
    lse = torch.full((1, B, w.Hq), 0.0, device="cuda")
    k_new = torch.zeros((1, B, w.Hkv, w.d), device="cuda")
    M.mkv_decode_plan(layout, dw.cache.pools[0], dw.batch(), 1, ws)
    M.mkv_append_attend(layout, dw.cache.pools[:1], dw.batch(), k_new, k_new, dw.q, 1 / math.sqrt(w.d), out, lse, ws)
    assert M.mkv_workspace_status(ws) == M.MKV_DEV_BAD_TIER
    o = out.cpu().numpy()[0]
    for b in range(B):
        assert np.isnan(o[b]).all() == last_is_tq3[b], b
        assert np.isfinite(o[b]).all() != last_is_tq3[b], b


def test_stream_read_probe_reads_every_unit():
    # the streaming-read probe reads each 3584-byte unit once: the XOR of its
    # per-wave words is the XOR of every unit's first word (a partial unit at
    # the end is not read)
    g = torch.Generator()
    g.manual_seed(11)
    n_units = 20000
    words = torch.randint(-2**31, 2**31 - 1, (n_units * 896 + 200,), dtype=torch.int32, generator=g)
    src = words.cuda()
    sink = torch.zeros(12 * 300, dtype=torch.int32, device="cuda")
    M.mkv_stream_read(src, sink)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(words[0:n_units * 896:896].numpy())
    assert np.bitwise_xor.reduce(sink.cpu().numpy()) == expect
    # a small sink (12 words: one workgroup) covers every unit too
    sink1 = torch.zeros(12, dtype=torch.int32, device="cuda")
    M.mkv_stream_read(src, sink1, nbytes=1000 * 3584 + 17)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink1.cpu().numpy()) == np.bitwise_xor.reduce(words[0:1000 * 896:896].numpy())


def test_debug_sync_reports_device_status(capfd, monkeypatch):
    """MKV_DEBUG_SYNC=1: each call synchronises its stream before returning
    and prints the device status bits its workspace holds; the call itself
    still returns MKV_OK and the outputs are the same as without the flag."""
    M.set_partial_kind(1)
    w = W.scaled(W.WORKLOADS["batch-8x16384"], B=2, lengths=("fixed", 300), recent_tokens=64)
    st = W.make_structure(w)
    dw = DeviceWorkload(w, st, "cuda")
    out0, lse0, status = _decode(dw)
    assert status == 0
    dw.bt[int(st.bt_offsets[1]) + 3] = st.n_fp8 + st.n_tq3 + 5        # request 1: an id outside the pool
    monkeypatch.setenv("MKV_DEBUG_SYNC", "1")
    capfd.readouterr()
    out, lse, status = _decode(dw)
    err = capfd.readouterr().err
    assert status == M.MKV_DEV_BAD_PAGE_ID
    assert "[mkv] mkv_decode_attn_layers: device status bits 0x1" in err, err
    assert np.all(np.isnan(out[0, 1])) and np.array_equal(out[0, 0], out0[0, 0])
    monkeypatch.delenv("MKV_DEBUG_SYNC")
    capfd.readouterr()
    _decode(dw)
    assert "[mkv]" not in capfd.readouterr().err
