"""Pins for the oracle's page lifecycle (allocation, aging, free stacks, release)."""
import copy

import numpy as np

from oracle import lifecycle as LC, pool as P

HKV, D, R = 2, 128, 3


def _state(n_layers=2, B=2, cap=12, n_fp8=10, n_tq3=20, seed=0):
    rng = np.random.default_rng(seed)
    tier = np.full(n_fp8 + n_tq3, P.TIER_FREE, dtype=np.uint8)
    pools = [P.Pool(HKV, D, n_fp8, n_tq3, tier=tier) for _ in range(n_layers)]
    t = LC.Tables(np.arange(B + 1) * cap, np.full(B * cap, -1), np.zeros(B, dtype=np.int64), tier,
                  rng.permutation(n_fp8), n_fp8 + rng.permutation(n_tq3), [n_fp8, n_tq3])
    return pools, t


def _live(t, b):
    lo = int(t.bt_offsets[b])
    return [int(x) for x in t.bt_pages[lo:lo + -(-int(t.seq_lens[b]) // 16)]]


def _check_invariants(pools, t, anchors):
    n_fp8, n_tq3 = pools[0].n_fp8, pools[0].n_tq3
    live = [pid for b in range(len(t.seq_lens)) for pid in _live(t, b)]
    free_f = [int(x) for x in t.fp8_free[:t.tops[0]]]
    free_t = [int(x) for x in t.tq3_free[:t.tops[1]]]
    # every id is either live (exactly once) or free (exactly once)
    assert sorted([p for p in live if p < n_fp8] + free_f) == list(range(n_fp8))
    assert sorted([p for p in live if p >= n_fp8] + free_t) == list(range(n_fp8, n_fp8 + n_tq3))
    assert all(t.tier[p] == P.TIER_FREE for p in free_f + free_t)
    for b in range(len(t.seq_lens)):
        pages = _live(t, b)
        n = len(pages)
        for lp, pid in enumerate(pages):
            if (b, lp) in anchors:
                assert pid < n_fp8 and t.tier[pid] == P.TIER_A
            elif lp >= n - R:
                assert pid < n_fp8 and t.tier[pid] == P.TIER_R
            else:
                assert pid >= n_fp8 and t.tier[pid] == P.TIER_S


def test_growth_keeps_window_anchors_and_values():
    """Tokens appended one step at a time: after every step the last R pages
    are Recent FP8, the anchor stays FP8, older pages are TQ3, no id is lost
    or duplicated; at the end the cache holds exactly the value path's values
    for that tier pattern (FP8 of the token, TQ3 of that FP8 value)."""
    pools, t = _state()
    B, T = 2, 150
    rng = np.random.default_rng(1)
    k = rng.standard_normal((len(pools), B, T, HKV, D)).astype(np.float32) * 3
    v = rng.standard_normal((len(pools), B, T, HKV, D)).astype(np.float32) * 3
    anchors = set()
    for step in range(T):
        assert LC.step(pools, t, R) == 0
        for li, pool in enumerate(pools):
            P.append(pool, k[li, :, step:step + 1], v[li, :, step:step + 1], t.bt_offsets, t.bt_pages,
                     t.seq_lens - 1)
        if step == 20:                                  # the caller protects request 0's page 1
            pid = int(t.bt_pages[t.bt_offsets[0] + 1])
            assert t.tier[pid] == P.TIER_R
            t.tier[pid] = P.TIER_A
            anchors.add((0, 1))
        _check_invariants(pools, t, anchors)
    assert list(t.seq_lens) == [T, T]
    n = -(-T // 16)
    for b in range(B):
        is_tq3 = np.array([(b, lp) not in anchors and lp < n - R for lp in range(n)])
        for li, pool in enumerate(pools):
            K, V = P.gather_kv(pool, t.bt_offsets, t.bt_pages, b, T)
            for h in range(HKV):
                assert np.array_equal(K[:, h], P.quantized_values(k[li, b, :, h], is_tq3, 1.0))
                assert np.array_equal(V[:, h], P.quantized_values(v[li, b, :, h], is_tq3, 1.0))


def test_pops_follow_request_order():
    pools, t = _state(B=3, n_fp8=6, n_tq3=4)
    t.fp8_free[:4] = [5, 1, 2, 4]
    t.tops = [4, 4]
    t.seq_lens[:] = [0, 5, 16]                   # request 1 fits its page; 0 and 2 start pages
    t.bt_pages[t.bt_offsets[1]] = 0
    t.bt_pages[t.bt_offsets[2]] = 3
    t.tier[[0, 3]] = P.TIER_R
    assert LC.step(pools, t, R) == 0
    assert t.bt_pages[t.bt_offsets[0]] == 4 and t.bt_pages[t.bt_offsets[2] + 1] == 2
    assert t.tops == [2, 4] and list(t.seq_lens) == [1, 6, 17]


def test_failure_changes_nothing():
    pools, t = _state(B=2, n_fp8=3, n_tq3=4)
    t.tops = [1, 4]                                # one free FP8 id, two requests need one
    before = copy.deepcopy((t.bt_pages, t.seq_lens, t.tier.copy(), t.fp8_free, t.tq3_free, list(t.tops)))
    assert LC.step(pools, t, R) == LC.NO_FREE_PAGE
    after = (t.bt_pages, t.seq_lens, t.tier, t.fp8_free, t.tq3_free, t.tops)
    for x, y in zip(before, after):
        assert np.array_equal(np.asarray(x), np.asarray(y))
    # a full block-table row
    pools, t = _state(B=1, cap=2)
    t.seq_lens[:] = [32]
    t.bt_pages[:2] = [0, 1]
    t.tier[[0, 1]] = P.TIER_R
    assert LC.step(pools, t, R) == LC.BAD_SEQ_LEN and t.seq_lens[0] == 32


def test_release_returns_every_page():
    pools, t = _state()
    for _ in range(100):
        assert LC.step(pools, t, R) == 0
    ids0 = _live(t, 0)
    assert LC.release(pools[0], t, [0]) == 0
    assert t.seq_lens[0] == 0 and all(t.tier[p] == P.TIER_FREE for p in ids0)
    _check_invariants(pools, t, set())
    assert LC.release(pools[0], t, [0]) == 0        # nothing live left: a no-op
    assert LC.release(pools[0], t, [5]) == LC.BAD_SEQ_LEN
