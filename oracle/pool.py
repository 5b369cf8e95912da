"""Byte-level page pool: append, FP8 -> TQ3 demotion, page-table gather.

Oracle side, test infrastructure only.

Pages (arXiv 2608.23834): every live-request page stays addressable through
the page table and pages of both formats live in one PagedAttention block
structure (page 1, Abstract; page 2, "Technical Deep Dive", fourth bullet);
Recent and protected Anchor pages are FP8 and older non-anchor pages move to
packed TQ3 (page 1, Abstract).

Readings: the tier map is one byte per physical page (R = 0, A = 1, S = 2,
free = 0xFF); physical ids [0, n_fp8) are FP8 slots and [n_fp8, n_fp8 + n_tq3)
TQ3 slots; block tables are CSR (bt_offsets[B + 1], bt_pages[]); a token at
position p of a request lives in logical page p // 16, slot p % 16.  One
fp32 k_scale and one v_scale per layer.
"""
import numpy as np

from . import fp8, rotation, tq3
from .layout import (PAGE, fp8_page_bytes, tq3_page_bytes, tq3_head_bytes, fp8_offset,
                     encode_tq3_head, decode_tq3_head)

TIER_R, TIER_A, TIER_S, TIER_FREE = 0, 1, 2, 0xFF


class Pool:
    """One layer's pool: an FP8 slab, a TQ3 slab, and (shared) tier map."""

    def __init__(self, num_kv_heads, d, n_fp8, n_tq3, k_scale=1.0, v_scale=1.0, tier=None, signs=None):
        """signs: None, or the layer's +-1 vector [d]: its TQ3 pages are rotated
        (oracle/rotation.py)."""
        self.Hkv, self.d = num_kv_heads, d
        self.signs = None if signs is None else np.asarray(signs, dtype=np.int8)
        self.n_fp8, self.n_tq3 = n_fp8, n_tq3
        self.fp8 = np.zeros((n_fp8, fp8_page_bytes(num_kv_heads, d)), dtype=np.uint8)
        self.tq3 = np.zeros((n_tq3, tq3_page_bytes(num_kv_heads, d)), dtype=np.uint8)
        self.tier = tier if tier is not None else np.full(n_fp8 + n_tq3, TIER_FREE, dtype=np.uint8)
        self.k_scale, self.v_scale = np.float32(k_scale), np.float32(v_scale)


def append(pool, k, v, bt_offsets, bt_pages, pos, counts=None):
    """Quantise k, v [B][n_new][Hkv][d] (fp32) to E4M3 and store token pos[b] + i.

    The token's logical page must already map to an FP8 page.  counts[b]
    (optional) limits how many of the n_new tokens of request b are written.
    """
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    B, n_new = k.shape[0], k.shape[1]
    d = pool.d
    for b in range(B):
        n = n_new if counts is None else int(counts[b])
        ek = fp8.e4m3_quantize(k[b, :n], pool.k_scale)          # [n][Hkv][d]
        ev = fp8.e4m3_quantize(v[b, :n], pool.v_scale)
        for i in range(n):
            p = int(pos[b]) + i
            lp, slot = divmod(p, PAGE)
            pid = int(bt_pages[int(bt_offsets[b]) + lp])
            assert 0 <= pid < pool.n_fp8, "append target must be an FP8 page"
            for h in range(pool.Hkv):
                o = fp8_offset(d, h, 0, slot, 0)
                pool.fp8[pid, o:o + d] = ek[i, h]
                o = fp8_offset(d, h, 1, slot, 0)
                pool.fp8[pid, o:o + d] = ev[i, h]


def fp8_page_values(pool, pid):
    """FP8 page -> fl32(decode(e) * scale) as float32 array [Hkv][2][16][d]."""
    e = pool.fp8[pid].reshape(pool.Hkv, 2, PAGE, pool.d)
    x = fp8.e4m3_decode(e).astype(np.float32)
    sc = np.array([pool.k_scale, pool.v_scale], dtype=np.float32)[None, :, None, None]
    return (x * sc).astype(np.float32)


def demote(pool, src_fp8, dst_tq3):
    """Demote FP8 pages src[i] into TQ3 slots dst[i] (physical ids >= n_fp8).

    For every head, K and V, token and 32-channel group: quantise the FP8
    page's dequantised values with the TQ3 rule and write the head blocks.
    With pool.signs set, each (head, K/V, token) row of d values is rotated
    first (rotation.rotate_f32).  The caller updates the block table and the
    tier map afterwards.
    """
    d = pool.d
    G = d // tq3.GROUP
    for s, t in zip(src_fp8, dst_tq3):
        s, t = int(s), int(t)
        assert 0 <= s < pool.n_fp8 and pool.n_fp8 <= t < pool.n_fp8 + pool.n_tq3
        x = fp8_page_values(pool, s)                                # [Hkv][2][16][d]
        if pool.signs is not None:
            x = rotation.rotate_f32(x, pool.signs)
        u, sc = tq3.quantize_groups(x.reshape(pool.Hkv, 2, PAGE, G, tq3.GROUP))
        u = u.reshape(pool.Hkv, 2, PAGE, d)
        hb = tq3_head_bytes(d)
        for h in range(pool.Hkv):
            blk = encode_tq3_head(u[h, 0], sc[h, 0], u[h, 1], sc[h, 1])
            pool.tq3[t - pool.n_fp8, h * hb:(h + 1) * hb] = blk


def page_values(pool, pid):
    """Dequantised values of physical page pid as float64 [Hkv][2][16][d]."""
    pid = int(pid)
    if pid < pool.n_fp8:
        e = pool.fp8[pid].reshape(pool.Hkv, 2, PAGE, pool.d)
        x = fp8.e4m3_decode(e)
        return x * np.array([float(pool.k_scale), float(pool.v_scale)])[None, :, None, None]
    out = tq3_page_codes_values(pool, pid)
    if pool.signs is not None:
        out = rotation.unrotate_f64(out, pool.signs)             # back to the channels of the cache
    return out


def tq3_page_codes_values(pool, pid):
    """(u - 4) s of every code of TQ3 page pid, float64 [Hkv][2][16][d] (exact):
    for a rotated pool these are the rotated values y, before unrotation."""
    pid = int(pid)
    assert pool.n_fp8 <= pid < pool.n_fp8 + pool.n_tq3
    hb = tq3_head_bytes(pool.d)
    out = np.zeros((pool.Hkv, 2, PAGE, pool.d))
    blk_all = pool.tq3[pid - pool.n_fp8]
    for h in range(pool.Hkv):
        uK, sK, uV, sV = decode_tq3_head(blk_all[h * hb:(h + 1) * hb], pool.d)
        G = pool.d // tq3.GROUP
        out[h, 0] = tq3.dequantize_groups(uK.reshape(PAGE, G, tq3.GROUP), sK).reshape(PAGE, pool.d)
        out[h, 1] = tq3.dequantize_groups(uV.reshape(PAGE, G, tq3.GROUP), sV).reshape(PAGE, pool.d)
    return out


def gather_kv(pool, bt_offsets, bt_pages, b, seq_len):
    """Walk request b's logical pages and return K, V float64 [seq_len][Hkv][d]."""
    n = -(-int(seq_len) // PAGE)
    K = np.zeros((n * PAGE, pool.Hkv, pool.d))
    V = np.zeros((n * PAGE, pool.Hkv, pool.d))
    for lp in range(n):
        pid = int(bt_pages[int(bt_offsets[b]) + lp])
        vals = page_values(pool, pid)
        K[lp * PAGE:(lp + 1) * PAGE] = vals[:, 0].transpose(1, 0, 2)
        V[lp * PAGE:(lp + 1) * PAGE] = vals[:, 1].transpose(1, 0, 2)
    return K[:seq_len], V[:seq_len]


def gather_raw(pool, bt_offsets, bt_pages, b, n_pages):
    """Raw bytes of request b's first n_pages logical pages, one record each.

    Record size is the FP8 page size; a TQ3 page fills the first
    tq3_page_bytes bytes of its record and the rest is zero.
    """
    rec = fp8_page_bytes(pool.Hkv, pool.d)
    out = np.zeros((n_pages, rec), dtype=np.uint8)
    for lp in range(n_pages):
        pid = int(bt_pages[int(bt_offsets[b]) + lp])
        if pid < pool.n_fp8:
            out[lp] = pool.fp8[pid]
        else:
            tb = tq3_page_bytes(pool.Hkv, pool.d)
            out[lp, :tb] = pool.tq3[pid - pool.n_fp8]
    return out


def quantized_values(x, page_is_tq3, scale, signs=None):
    """Value path without bytes: what one head's tokens dequantise to.

    x: fp32 [T][d] source values of one KV head (K or V) of one request;
    page_is_tq3[lp]: whether logical page lp is stored as TQ3.  FP8 tokens give
    decode(encode(x / scale)) * scale; TQ3 tokens quantise fl32(that FP8 value)
    with the TQ3 rule and give (u - 4) * s.  Float64 [T][d].  Used for samples
    of workloads too large to build as byte pools on the CPU; tests show it
    equals the byte path.  signs: rotated TQ3 (rotate, quantise, dequantise,
    rotate back in fp64).
    """
    x = np.asarray(x, dtype=np.float32)
    T, d = x.shape
    e = fp8.e4m3_quantize(x, scale)
    f32 = (fp8.e4m3_decode(e).astype(np.float32) * np.float32(scale)).astype(np.float32)
    out = fp8.e4m3_decode(e) * float(scale)
    tq = np.repeat(np.asarray(page_is_tq3, dtype=bool), PAGE)[:T]
    if tq.any():
        G = d // tq3.GROUP
        y = f32[tq] if signs is None else rotation.rotate_f32(f32[tq], signs)
        u, s = tq3.quantize_groups(y.reshape(-1, G, tq3.GROUP))
        deq = tq3.dequantize_groups(u, s).reshape(-1, d)
        out[tq] = deq if signs is None else rotation.unrotate_f64(deq, signs)
    return out
