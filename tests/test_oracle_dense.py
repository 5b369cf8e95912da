"""Pins for the oracle's bf16 rounding and dense materialisation of pages."""
import numpy as np
import torch

import workloads as W
from oracle import build, dense, fp8, layout, pool as P, tq3


def _torch_bf16_bits(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_library_conversion():
    rng = np.random.default_rng(0)
    # wide exponent range, both signs, subnormals included
    x = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-140, 120, 200_000))).astype(np.float32)
    assert np.array_equal(dense.bf16_rne_bits(x), _torch_bf16_bits(x))
    # every kind of rounding decision: bf16 values, exact midpoints (ties), and
    # one fp32 ulp either side of them
    base = rng.integers(0, 0x7F7F, 50_000, dtype=np.uint32) << np.uint32(16)
    base |= rng.integers(0, 2, base.size, dtype=np.uint32) << np.uint32(31)
    cand = [base, base | 0x8000, (base | 0x8000) + 1, (base | 0x8000) - 1, base | 0x0001, base | 0xFFFF]
    y = np.concatenate(cand).view(np.float32)
    y = y[np.isfinite(y) & np.isfinite(y.astype(np.float64) * 1.01)]
    assert np.array_equal(dense.bf16_rne_bits(y), _torch_bf16_bits(y))


def test_bf16_ties_go_to_even_and_exact_values_stay():
    one_ulp = 2.0 ** -7                           # bf16 spacing in [1, 2)
    assert dense.bf16_rne_bits(np.float32(1.0 + one_ulp / 2)) == 0x3F80      # tie, even below
    assert dense.bf16_rne_bits(np.float32(1.0 + 3 * one_ulp / 2)) == 0x3F82  # tie, even above
    assert dense.bf16_rne_bits(np.float32(-(1.0 + one_ulp / 2))) == 0xBF80
    # every finite E4M3 value has 4 significant bits, so it is exact in bf16
    codes = np.array([c for c in range(256) if c not in fp8.NAN_CODES], dtype=np.uint8)
    vals = fp8.e4m3_decode(codes)
    assert np.array_equal(dense.bf16_to_float(dense.bf16_rne_bits(vals.astype(np.float32))), vals)


def _pool_and_table(d=128, k_scale=1.0, v_scale=1.0):
    w = W.scaled(W.WORKLOADS["tiny-1x1024-d128"], d=d) if d != 128 else W.WORKLOADS["tiny-1x1024-d128"]
    st = W.make_structure(w)
    vals = W.layer_values(w, st, 0)
    k = [x.numpy() for x in vals["k"]]
    v = [x.numpy() for x in vals["v"]]
    pool, bt = build.build_layer(w, st, k, v, k_scale, v_scale)
    return w, st, pool, bt


def test_materialize_values_follow_the_page_formats():
    w, st, pool, bt = _pool_and_table(k_scale=0.75, v_scale=1.25)
    n = int(st.n_pages[0])
    K, V = dense.materialize(pool, st.bt_offsets, bt, 0, 0, n)
    Kx, Vx = P.gather_kv(pool, st.bt_offsets, bt, 0, n * 16)          # float64 values of the pages
    tiers = st.tiers[st.bt_offsets[0]:st.bt_offsets[1]]
    for lp in range(n):
        sl = slice(16 * lp, 16 * lp + 16)
        pid = int(bt[st.bt_offsets[0] + lp])
        if tiers[lp] == P.TIER_S:
            # TQ3: (u - 4) s rounded once to bf16 (8 significant bits): within half an ulp
            for got, ref in ((K[sl], Kx[sl]), (V[sl], Vx[sl])):
                g = dense.bf16_to_float(got)
                assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-300)
        else:
            # FP8: bf16 of fl32(decode * scale); decode itself is exact in bf16
            e = pool.fp8[pid].reshape(w.Hkv, 2, 16, w.d)
            for kv, got, sc in ((0, K[sl], 0.75), (1, V[sl], 1.25)):
                f32 = (fp8.e4m3_decode(e[:, kv]).astype(np.float32) * np.float32(sc)).astype(np.float32)
                assert np.array_equal(got, dense.bf16_rne_bits(f32).transpose(1, 0, 2))


def test_materialize_scale_one_is_exact_and_range_edges_are_nan():
    w, st, pool, bt = _pool_and_table()
    n = int(st.n_pages[0])
    K, V = dense.materialize(pool, st.bt_offsets, bt, 0, n - 3, 5)   # 3 pages in the table, 2 past its end
    Kx, Vx = P.gather_kv(pool, st.bt_offsets, bt, 0, n * 16)
    tail = slice(16 * (n - 3), 16 * n)
    fp8_pages = st.tiers[st.bt_offsets[0] + n - 3:st.bt_offsets[0] + n] != P.TIER_S
    for i in range(3):
        if fp8_pages[i]:                        # scale 1: FP8 values exactly
            sl = slice(16 * i, 16 * i + 16)
            assert np.array_equal(dense.bf16_to_float(K[sl]), Kx[tail][sl])
            assert np.array_equal(dense.bf16_to_float(V[sl]), Vx[tail][sl])
    assert (K[48:] == dense.BF16_NAN).all() and (V[48:] == dense.BF16_NAN).all()
    # an id outside the pool
    bt2 = bt.copy()
    bt2[st.bt_offsets[0] + 1] = pool.n_fp8 + pool.n_tq3 + 7
    K2, _ = dense.materialize(pool, st.bt_offsets, bt2, 0, 0, 3)
    assert (K2[16:32] == dense.BF16_NAN).all() and not (K2[:16] == dense.BF16_NAN).any()


def test_materialize_token_order_by_hand():
    """One TQ3 page written by hand: every (t, c) lands at row t, channel c."""
    d, hkv = 128, 1
    G = d // 32
    rng = np.random.default_rng(5)
    uK = rng.integers(1, 8, (16, d))
    uV = rng.integers(1, 8, (16, d))
    sK = rng.uniform(0.5, 2, (16, G)).astype(np.float16)
    sV = rng.uniform(0.5, 2, (16, G)).astype(np.float16)
    pool = P.Pool(hkv, d, 1, 1)
    pool.tq3[0] = layout.encode_tq3_head(uK, sK, uV, sV)
    K, V = dense.materialize(pool, np.array([0, 1]), np.array([1]), 0, 0, 1)
    for t in range(16):
        for c in range(d):
            for got, u, s in ((K, uK, sK), (V, uV, sV)):
                ref = np.float32((int(u[t, c]) - 4) * float(s[t, c // 32]))
                assert got[t, 0, c] == dense.bf16_rne_bits(ref)
