"""Pins for the oracle's page pool, gather, demotion and byte accounting."""
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention, build, fp8, layout, pool as P, tq3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accounting.txt")


def _tiny(seed_shift=0, **kw):
    w = W.WORKLOADS["tiny-1x1024-d128"]
    if kw or seed_shift:
        w = W.scaled(w, seed=w.seed + seed_shift, **kw)
    st = W.make_structure(w)
    vals = W.layer_values(w, st, 0)
    k = [x.numpy() for x in vals["k"]]
    v = [x.numpy() for x in vals["v"]]
    return w, st, k, v, vals["q"].numpy()


def test_append_places_tokens_and_gather_decodes_them():
    w, st, k, v, q = _tiny()
    pool, bt = build.build_layer(w, st, k, v)
    K, V = P.gather_kv(pool, st.bt_offsets, bt, 0, int(st.seq_lens[0]))
    tiers = st.tiers[st.bt_offsets[0]:st.bt_offsets[1]]
    for lp in range(st.n_pages[0]):
        sl = slice(lp * 16, lp * 16 + 16)
        fp = fp8.e4m3_decode(fp8.e4m3_quantize(k[0][sl]))
        if tiers[lp] != P.TIER_S:
            assert np.array_equal(K[sl], fp)            # FP8 page: exactly the E4M3 values
        else:                                           # TQ3 page: TQ3 of the FP8 values
            u, s = tq3.quantize_groups(fp.astype(np.float32).reshape(16, w.Hkv, -1, 32))
            assert np.array_equal(K[sl], tq3.dequantize_groups(u, s).reshape(16, w.Hkv, w.d))


def test_value_path_equals_byte_path():
    w, st, k, v, q = _tiny()
    pool, bt = build.build_layer(w, st, k, v)
    K, V = P.gather_kv(pool, st.bt_offsets, bt, 0, int(st.seq_lens[0]))
    is_tq3 = st.tiers[:st.n_pages[0]] == P.TIER_S
    for h in range(w.Hkv):
        assert np.array_equal(P.quantized_values(k[0][:, h], is_tq3, 1.0), K[:, h])
        assert np.array_equal(P.quantized_values(v[0][:, h], is_tq3, 1.0), V[:, h])


def test_physical_placement_does_not_change_output():
    w, st, k, v, q = _tiny()
    pool, bt = build.build_layer(w, st, k, v)
    o1, l1 = attention.decode_batch(pool, q, st.bt_offsets, bt, st.seq_lens)
    # same values, a different random placement of the pages in both slabs
    rng = np.random.default_rng(99)
    st2 = W.make_structure(w)
    st2.staging_ids = rng.permutation(st2.n_fp8).astype(np.int32)
    tq = st2.tiers == P.TIER_S
    st2.final_ids = np.where(tq, st2.n_fp8 + rng.permutation(st2.n_tq3)[np.cumsum(tq) - 1], st2.staging_ids).astype(np.int32)
    pool2, bt2 = build.build_layer(w, st2, k, v)
    assert not np.array_equal(bt, bt2)
    o2, l2 = attention.decode_batch(pool2, q, st2.bt_offsets, bt2, st2.seq_lens)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # and the logical page bytes are the same
    r1 = P.gather_raw(pool, st.bt_offsets, bt, 0, int(st.n_pages[0]))
    r2 = P.gather_raw(pool2, st2.bt_offsets, bt2, 0, int(st2.n_pages[0]))
    assert np.array_equal(r1, r2)


def test_needle_in_every_tier_and_position():
    # "every live-request page remains addressable": a dominant key planted at
    # any token of any page, in any tier, takes the whole softmax.
    w, st, k, v, q = _tiny()
    tiers = st.tiers[:st.n_pages[0]]
    probe = []
    for tier in (P.TIER_R, P.TIER_A, P.TIER_S):
        pages = np.nonzero(tiers == tier)[0]
        for lp in (pages[0], pages[-1]):
            for slot in (0, 7, 15):
                probe.append(lp * 16 + slot)
    h = 1
    qi = np.zeros((w.Hq, w.d), dtype=np.float32)
    qi[h * 6:(h + 1) * 6, 5] = 1.0
    for t in probe:
        kk = [k[0].copy()]
        vv = [v[0].copy()]
        kk[0][:, :, 5] = 0.0
        kk[0][t, h, :] = 0.0
        kk[0][t, h, 5] = 400.0              # huge score after quantisation in either format
        vv[0][t, h, :] = 3.0
        pool, bt = build.build_layer(w, st, kk, vv)
        o, _ = attention.decode_batch(pool, qi[None], st.bt_offsets, bt, st.seq_lens)
        for i in range(h * 6, (h + 1) * 6):
            assert np.allclose(o[0, i], 3.0, atol=1e-6), (t, tiers[t // 16])


def test_demoted_bytes_roundtrip_codes():
    w, st, k, v, q = _tiny()
    pool, bt = build.build_layer(w, st, k, v)
    pid = int(bt[np.nonzero(st.tiers == P.TIER_S)[0][0]])
    blk = pool.tq3[pid - pool.n_fp8]
    hb = layout.tq3_head_bytes(w.d)
    uK, sK, uV, sV = layout.decode_tq3_head(blk[:hb], w.d)
    assert uK.min() >= 1 and uV.min() >= 1            # u = 0 is never produced
    assert blk.shape[0] == w.Hkv * hb


def test_accounting_formula():
    vals = dict(l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#"))
    kib, r_bf16, r_fp8 = float(vals["kib_per_token"]), float(vals["ratio_vs_bf16"]), float(vals["ratio_vs_fp8"])
    # the pages' form: BF16 bytes / ratio; 16 layers x 4 KV heads x 256 x 2 (K,V) x 2 B = 64 KiB
    bf16_kib = 16 * 4 * 256 * 2 * 2 / 1024
    assert abs(bf16_kib / r_bf16 - kib) < 0.05
    assert abs((bf16_kib / 2) / r_fp8 - kib) < 0.05
    # our layout: exact bytes per token per layer
    for d in (128, 256):
        Hkv = 4
        assert layout.fp8_page_bytes(Hkv, d) == 16 * 2 * Hkv * d
        assert layout.tq3_page_bytes(Hkv, d) == 16 * 2 * Hkv * (3 * d // 8 + d // 16)
    # canary shape (2 x 59,008 tokens, 16 layers): 72 FP8 and 3,616 TQ3 pages per request
    mixed = 16 * 2 * (72 * layout.fp8_page_bytes(4, 256) + 3616 * layout.tq3_page_bytes(4, 256))
    assert mixed == 1_734_344_704
    assert 16 * 2 * 3688 * layout.fp8_page_bytes(4, 256) == 3_867_148_288


@pytest.mark.parametrize("name", ["batch-8x16384", "ragged-32x4096-65536", "demote-64x32768", "long-1x131072", "canary-2x59008-16L"])
def test_workload_structure(name):
    w = W.WORKLOADS[name]
    st = W.make_structure(w)
    assert st.total_pages == int(np.sum(-(-st.seq_lens.astype(np.int64) // 16)))
    # tier invariant: tier in {R, A} <=> FP8 id; S <=> TQ3 id
    fp = st.tiers != P.TIER_S
    assert np.all(st.final_ids[fp] < st.n_fp8) and np.all(st.final_ids[~fp] >= st.n_fp8)
    assert len(np.unique(st.final_ids)) == st.total_pages
    rec = w.recent_tokens // 16
    for b in range(min(w.B, 4)):
        t = st.tiers[st.bt_offsets[b]:st.bt_offsets[b + 1]]
        assert np.all(t[-rec:] == P.TIER_R)
        assert np.all(t[:w.fixed_anchor_pages] == P.TIER_A)
