"""Dense fp64 decode attention and the log-sum-exp merge -- oracle side.

Test infrastructure only.

The pages' method computes partial attention states per page format and
combines them with a globally normalised online-softmax merge, which is
mathematically the same as one softmax over all tokens (arXiv 2608.23834,
page 1, Abstract; page 2, "Enhanced Key Takeaways", third bullet, and
"Technical Deep Dive", second bullet).  So the oracle computes the plain
definition: dense softmax attention in fp64 over the dequantised cache.

Readings: one query token per request (decode_batch) or the request's last
T tokens as queries (decode_batch_multi: query token t of T attends to the
tokens at positions [0, seq_len - T + t], causal); query head i reads KV head
i // (Hq / Hkv); softmax scale 1 / sqrt(d) unless given; tokens at or beyond
seq_len are absent; seq_len = 0 gives o = 0 and lse = -inf; lse is the
natural log of the softmax denominator including the running max.
"""
import numpy as np


def decode_attention(q, K, V, sm_scale=None):
    """q [Hq][d] (fp32 widened), K, V [T][Hkv][d] float64 -> (o [Hq][d], lse [Hq])."""
    q = np.asarray(q, dtype=np.float32).astype(np.float64)
    Hq, d = q.shape
    T, Hkv = K.shape[0], K.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    o = np.zeros((Hq, d))
    lse = np.full(Hq, -np.inf)
    if T == 0:
        return o, lse
    for i in range(Hq):
        h = i // G
        s = (K[:, h, :] @ q[i]) * sm_scale
        m = s.max()
        p = np.exp(s - m)
        l = p.sum()
        o[i] = (p @ V[:, h, :]) / l
        lse[i] = m + np.log(l)
    return o, lse


def partial_state(q, K, V, sm_scale=None):
    """Unnormalised partial state over a token subset: (m [Hq], l [Hq], acc [Hq][d]).

    An empty subset gives (-inf, 0, 0).
    """
    q = np.asarray(q, dtype=np.float32).astype(np.float64)
    Hq, d = q.shape
    T, Hkv = K.shape[0], K.shape[1]
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    m = np.full(Hq, -np.inf)
    l = np.zeros(Hq)
    acc = np.zeros((Hq, d))
    if T == 0:
        return m, l, acc
    for i in range(Hq):
        h = i // G
        s = (K[:, h, :] @ q[i]) * sm_scale
        m[i] = s.max()
        p = np.exp(s - m[i])
        l[i] = p.sum()
        acc[i] = p @ V[:, h, :]
    return m, l, acc


def merge_states(states):
    """Log-sum-exp merge of partial states [(m, l, acc), ...] -> (o, lse).

    M = max m_p; L = sum l_p e^(m_p - M); o = sum acc_p e^(m_p - M) / L;
    lse = M + ln L.  Empty partials (m = -inf) contribute nothing; if all are
    empty, o = 0 and lse = -inf.
    """
    ms = np.stack([s[0] for s in states])            # [P][Hq]
    M = ms.max(axis=0)
    Hq, d = states[0][2].shape
    o = np.zeros((Hq, d))
    lse = np.full(Hq, -np.inf)
    for i in range(Hq):
        if not np.isfinite(M[i]):
            continue
        L = 0.0
        acc = np.zeros(d)
        for (m, l, a) in states:
            if not np.isfinite(m[i]):
                continue
            w = np.exp(m[i] - M[i])
            L += l[i] * w
            acc += a[i] * w
        o[i] = acc / L
        lse[i] = M[i] + np.log(L)
    return o, lse


def decode_batch(pool, q, bt_offsets, bt_pages, seq_lens, sm_scale=None):
    """Oracle decode over a byte pool: q [B][Hq][d] -> (out [B][Hq][d], lse [B][Hq])."""
    from .pool import gather_kv
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        K, V = gather_kv(pool, bt_offsets, bt_pages, b, int(seq_lens[b]))
        out[b], lse[b] = decode_attention(q[b], K, V, sm_scale)
    return out, lse


def decode_batch_multi(pool, q, bt_offsets, bt_pages, seq_lens, sm_scale=None):
    """Multi-query decode: q [B][T][Hq][d] holds the queries of each request's
    last T tokens (positions seq_len - T .. seq_len - 1); query token t attends
    to the tokens at positions [0, seq_len - T + t] (none if that is empty).
    Returns (out [B][T][Hq][d], lse [B][T][Hq])."""
    from .pool import gather_kv
    B, T, Hq, d = q.shape
    out = np.zeros((B, T, Hq, d))
    lse = np.zeros((B, T, Hq))
    for b in range(B):
        sl = int(seq_lens[b])
        K, V = gather_kv(pool, bt_offsets, bt_pages, b, sl)
        for t in range(T):
            n = max(0, sl - T + t + 1)
            out[b, t], lse[b, t] = decode_attention(q[b, t], K[:n], V[:n], sm_scale)
    return out, lse
