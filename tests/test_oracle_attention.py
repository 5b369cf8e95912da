"""Pins for the oracle's fp64 decode attention and LSE merge (oracle/attention.py).

Pinned against closed forms, brute-force Python loops, the library routine
torch.nn.functional.scaled_dot_product_attention in fp64, and the invariance
that any split of tokens into parts, merged in any order, equals one softmax.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import workloads as W
from oracle import attention as A


def _rand(T, Hq=6, Hkv=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, d)).astype(np.float32)
    K = rng.standard_normal((T, Hkv, d))
    V = rng.standard_normal((T, Hkv, d))
    return q, K, V


def test_one_token_gives_v():
    q, K, V = _rand(1)
    o, lse = A.decode_attention(q, K, V)
    G = 3
    for i in range(6):
        assert np.array_equal(o[i], V[0, i // G])
        s = float(np.dot(K[0, i // G], q[i].astype(np.float64))) / math.sqrt(8)
        assert abs(lse[i] - s) < 1e-12


def test_identical_keys_and_zero_query_give_mean():
    q, K, V = _rand(37)
    K[:] = K[0]
    o, lse = A.decode_attention(q, K, V)
    for i in range(6):
        assert np.allclose(o[i], V[:, i // 3].mean(axis=0), atol=1e-13)
    q0 = np.zeros_like(q)
    _, K2, _ = _rand(37, seed=1)
    o, lse = A.decode_attention(q0, K2, V)
    for i in range(6):
        assert np.allclose(o[i], V[:, i // 3].mean(axis=0), atol=1e-13)
        assert abs(lse[i] - math.log(37)) < 1e-12


def test_two_tokens_sigmoid():
    q, K, V = _rand(2, seed=2)
    o, _ = A.decode_attention(q, K, V, sm_scale=0.3)
    for i in range(6):
        h = i // 3
        s1 = 0.3 * float(K[0, h] @ q[i].astype(np.float64))
        s2 = 0.3 * float(K[1, h] @ q[i].astype(np.float64))
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        assert np.allclose(o[i], w1 * V[0, h] + (1 - w1) * V[1, h], atol=1e-13)


def test_empty_sequence():
    q, K, V = _rand(0)
    o, lse = A.decode_attention(q, K, V)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    m, l, acc = A.partial_state(q, K, V)
    assert np.all(np.isneginf(m)) and np.all(l == 0) and np.all(acc == 0)


def test_bruteforce_loops_tiny():
    # 3 pages of 16 tokens, d = 8, 2 KV heads, GQA 3, written as plain Python loops
    q, K, V = _rand(48, seed=3)
    o, lse = A.decode_attention(q, K, V)
    for i in range(6):
        h = i // 3
        s = []
        for t in range(48):
            acc = 0.0
            for c in range(8):
                acc += float(q[i, c]) * K[t, h, c]
            s.append(acc / math.sqrt(8))
        m = max(s)
        e = [math.exp(x - m) for x in s]
        L = sum(e)
        for c in range(8):
            oc = sum(e[t] * V[t, h, c] for t in range(48)) / L
            assert abs(oc - o[i, c]) < 1e-12
        assert abs(lse[i] - (m + math.log(L))) < 1e-12


def test_matches_library_sdpa_fp64():
    rng = np.random.default_rng(4)
    T, Hq, Hkv, d = 300, 24, 4, 128
    q = (rng.standard_normal((Hq, d)) * 2).astype(np.float32)
    K = rng.standard_normal((T, Hkv, d)) * 1.5
    V = rng.standard_normal((T, Hkv, d))
    o, _ = A.decode_attention(q, K, V)
    G = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64))[:, None, :]                    # [Hq, 1, d]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)          # [Hq, T, d]
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous())[:, 0, :].numpy()
    assert np.max(np.abs(ref - o)) < 1e-12


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 80), st.lists(st.integers(0, 79), max_size=6), st.integers(0, 10 ** 6), st.booleans())
def test_merge_invariance(T, cuts, seed, reverse):
    q, K, V = _rand(T, seed=seed)
    q = q * 3
    o, lse = A.decode_attention(q, K, V)
    bounds = sorted(set([0, T] + [c % (T + 1) for c in cuts]))
    rng = np.random.default_rng(seed)
    perm = rng.permutation(T)                       # parts need not be contiguous (mixed formats)
    parts = [perm[a:b] for a, b in zip(bounds[:-1], bounds[1:])]
    parts.append(np.array([], dtype=np.int64))     # an empty partial is allowed
    states = [A.partial_state(q, K[p], V[p]) for p in parts]
    if reverse:
        states = states[::-1]
    o2, lse2 = A.merge_states(states)
    assert np.max(np.abs(o2 - o)) < 1e-12
    assert np.max(np.abs(lse2 - lse)) < 1e-12


def test_merge_two_part_closed_form():
    q, K, V = _rand(10, seed=7)
    s1 = A.partial_state(q, K[:4], V[:4])
    s2 = A.partial_state(q, K[4:], V[4:])
    o, lse = A.merge_states([s1, s2])
    for i in range(6):
        a = s1[1][i] * math.exp(s1[0][i] - lse[i])
        b = s2[1][i] * math.exp(s2[0][i] - lse[i])
        assert abs(a + b - 1.0) < 1e-12
        assert np.allclose(o[i], (s1[2][i] / s1[1][i]) * a + (s2[2][i] / s2[1][i]) * b, atol=1e-12)
    o_e, lse_e = A.merge_states([A.partial_state(q, K[:0], V[:0])])
    assert np.all(o_e == 0) and np.all(np.isneginf(lse_e))


def test_multi_query_is_causal_and_matches_a_masked_library_softmax():
    """decode_batch_multi against torch's SDPA in fp64 with an explicit causal
    mask over the last T positions; T = 1 equals decode_batch; queries whose
    visible prefix is empty give 0 / -inf."""
    import torch
    from oracle import build, pool as P
    w = W.scaled(W.WORKLOADS["tiny-1x1024-d128"], B=2, lengths=("list", (300, 2)))
    st = W.make_structure(w)
    vals = W.layer_values(w, st, 0)
    pool, bt = build.build_layer(w, st, [x.numpy() for x in vals["k"]], [x.numpy() for x in vals["v"]])
    T = 4
    rng = np.random.default_rng(3)
    q = rng.standard_normal((w.B, T, w.Hq, w.d)).astype(np.float32)
    out, lse = A.decode_batch_multi(pool, q, st.bt_offsets, bt, st.seq_lens)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        sl = int(st.seq_lens[b])
        K, V = P.gather_kv(pool, st.bt_offsets, bt, b, sl)
        for t in range(T):
            vis = sl - T + t + 1
            if vis <= 0:
                assert np.all(out[b, t] == 0) and np.all(np.isneginf(lse[b, t]))
                continue
            for i in range(w.Hq):
                h = i // G
                mask = torch.zeros(1, sl, dtype=torch.float64)
                mask[0, vis:] = -float("inf")
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q[b, t, i].astype(np.float64))[None, None],
                    torch.from_numpy(K[:, h])[None], torch.from_numpy(V[:, h])[None], attn_mask=mask[None])
                assert np.allclose(out[b, t, i], ref[0, 0].numpy(), rtol=0, atol=1e-12)
    o1, l1 = A.decode_batch(pool, q[:, -1], st.bt_offsets, bt, st.seq_lens)
    assert np.array_equal(o1, out[:, -1]) and np.array_equal(l1, lse[:, -1])
