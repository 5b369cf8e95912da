"""Byte layout of FP8 and TQ3 pages -- oracle side (test infrastructure only).

The pages fix only that pages are PagedAttention-style blocks holding either
FP8 or "packed TQ3" data within one block structure (arXiv 2608.23834, page 1,
Abstract; page 2, "Technical Deep Dive", fourth bullet).  Everything below is
this implementation's documented reading; the oracle writes it out with plain
index loops so that a reader can check each position by eye.

Page size is 16 tokens.  d = head_dim (128 or 256), G = d / 32 scale groups
per token (a multiple of 4), Hkv KV heads.

FP8 page (physical id < n_fp8), Hkv * 2 * 16 * d bytes:
    byte ((h * 2 + kv) * 16 + t) * d + c  holds the E4M3 code of
    head h, kv (0 = K, 1 = V), token t, channel c.

TQ3 page, Hkv head blocks of 14 * d bytes each, block h at h * 14 * d:
    [0,    6d)  K codes      16 token rows of 3d/8 bytes
    [6d,  12d)  V codes      4 token quarters x 16 channel slices x G triples
    [12d, 13d)  K scales     fp16, little endian
    [13d, 14d)  V scales     fp16, little endian

A triple is 3 bytes = 8 codes: code slot k sits at bits [3k, 3k + 3) of the
little-endian 24-bit word b0 | b1 << 8 | b2 << 16 ("8 codes per 3 bytes").

K codes: token row t starts at t * 3d/8; in it, channel quarter j (channels
8 j .. 8 j + 7 of every group, j = 0..3) takes the G triples from byte 3 j G,
in blocks of 4 triples, block b for groups 4 b .. 4 b + 3.  Channel
c = 32 g + 8 j + e (e = 0..7), with gg = g % 4, sits in triple
4 (g // 4) + 2 (gg % 2) + e // 4 of its quarter, slot 2 (e % 4) + gg // 2.
(Read as 16 six-bit fields, field f of a block holds channel 8 j + f % 8 of
group 4 b + f // 8 in its low three bits and of group 4 b + 2 + f // 8 in its
high three bits.)

V codes: the triple at byte 3 * ((j * 16 + n) * G + p) (token quarter j = 0..3,
channel slice n = 0..15, p = 0..G-1) holds tokens 4 j .. 4 j + 3 of the two
channels a = n * d/16 + 2 p and b = a + 1: slot 2 r holds (a, 4 j + r) and
slot 2 r + 1 holds (b, 4 j + r), r = 0..3.

Scales (K and V alike): the scale of token t = 4 j + r, group g is the fp16 at
element (j * G + g) * 4 + r of the scale block.

Why this arrangement: each GPU lane's triples sit next to each other, so they
arrive in one aligned vector load, and a block of 4 triples read as six-bit
fields decodes with two FP6 conversions (low codes, then high codes) straight
into matrix-core operands.  The oracle does not depend on why; it only
follows the map.
"""
import functools
import numpy as np

PAGE = 16


def fp8_page_bytes(num_kv_heads, d):
    return num_kv_heads * 2 * PAGE * d


def tq3_head_bytes(d):
    return 14 * d


def tq3_page_bytes(num_kv_heads, d):
    return num_kv_heads * tq3_head_bytes(d)


def fp8_offset(d, h, kv, t, c):
    return ((h * 2 + kv) * PAGE + t) * d + c


# V-triple slot -> (channel offset within the pair, token offset within the quarter)
V_SLOT = {0: (0, 0), 1: (1, 0), 2: (0, 1), 3: (1, 1), 4: (0, 2), 5: (1, 2), 6: (0, 3), 7: (1, 3)}


@functools.lru_cache(maxsize=None)
def k_code_map(d):
    """(byte offset of the triple inside the head block, slot) for every (t, c) of K."""
    G = d // 32
    row = 3 * d // 8
    tri = np.zeros((PAGE, d), dtype=np.int64)
    slot = np.zeros((PAGE, d), dtype=np.int64)
    assert G % 4 == 0
    for t in range(PAGE):
        for g in range(G):
            gg = g % 4
            for j in range(4):
                for e in range(8):
                    c = 32 * g + 8 * j + e
                    triple = 4 * (g // 4) + 2 * (gg % 2) + e // 4
                    tri[t, c] = t * row + 3 * (j * G + triple)
                    slot[t, c] = 2 * (e % 4) + gg // 2
    return tri, slot


@functools.lru_cache(maxsize=None)
def v_code_map(d):
    """(byte offset of the triple inside the head block, slot) for every (t, c) of V."""
    G = d // 32
    per_slice = d // 16
    tri = np.full((PAGE, d), -1, dtype=np.int64)
    slot = np.full((PAGE, d), -1, dtype=np.int64)
    for j in range(4):
        for n in range(16):
            for p in range(G):
                a = n * per_slice + 2 * p
                for k, (ci, r) in V_SLOT.items():
                    t = 4 * j + r
                    c = a + ci
                    tri[t, c] = 6 * d + 3 * ((j * 16 + n) * G + p)
                    slot[t, c] = k
    assert (tri >= 0).all()
    return tri, slot


@functools.lru_cache(maxsize=None)
def scale_map(d):
    """Byte offset (inside the head block) of the K scale of (t, g); V adds d."""
    G = d // 32
    off = np.zeros((PAGE, G), dtype=np.int64)
    for t in range(PAGE):
        j, r = divmod(t, 4)
        for g in range(G):
            off[t, g] = 12 * d + 2 * ((j * G + g) * 4 + r)
    return off


def pack_triple(codes):
    """Scalar: 8 codes (each 0..7) -> 3 bytes."""
    w = 0
    for k, u in enumerate(codes):
        assert 0 <= u < 8
        w |= int(u) << (3 * k)
    return bytes([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF])


def unpack_triple(b3):
    """Scalar: 3 bytes -> 8 codes."""
    w = b3[0] | (b3[1] << 8) | (b3[2] << 16)
    return [(w >> (3 * k)) & 7 for k in range(8)]


def pack_triples(codes):
    """Vectorised pack: codes[..., 8] (0..7) -> uint8[..., 3]."""
    c = np.asarray(codes, dtype=np.uint32)
    w = np.zeros(c.shape[:-1], dtype=np.uint32)
    for k in range(8):
        w |= c[..., k] << np.uint32(3 * k)
    return np.stack([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], axis=-1).astype(np.uint8)


def unpack_triples(b):
    """Vectorised unpack: uint8[..., 3] -> codes uint8[..., 8]."""
    b = np.asarray(b, dtype=np.uint32)
    w = b[..., 0] | (b[..., 1] << np.uint32(8)) | (b[..., 2] << np.uint32(16))
    return np.stack([(w >> np.uint32(3 * k)) & 7 for k in range(8)], axis=-1).astype(np.uint8)


def encode_tq3_head(uK, sK, uV, sV):
    """Assemble one TQ3 head block from codes u[16, d] and fp16 scales s[16, G]."""
    d = uK.shape[1]
    block = np.zeros(tq3_head_bytes(d), dtype=np.uint8)
    triples = np.zeros((4 * d, 8), dtype=np.uint8)        # the 12d code bytes as 4d triples
    for u, (tri, slot) in ((uK, k_code_map(d)), (uV, v_code_map(d))):
        triples[tri // 3, slot] = u
    block[:12 * d] = pack_triples(triples).reshape(-1)
    off = scale_map(d)
    for s, extra in ((sK, 0), (sV, d)):
        raw = np.asarray(s, dtype=np.float16).view(np.uint16).astype(np.int64)
        block[off + extra] = (raw & 0xFF).astype(np.uint8)
        block[off + extra + 1] = (raw >> 8).astype(np.uint8)
    return block


def decode_tq3_head(block, d):
    """Inverse of encode_tq3_head: returns (uK, sK, uV, sV)."""
    block = np.asarray(block, dtype=np.uint8)
    triples = unpack_triples(block[:12 * d].reshape(-1, 3))
    ktri, kslot = k_code_map(d)
    vtri, vslot = v_code_map(d)
    uK = triples[ktri // 3, kslot]
    uV = triples[vtri // 3, vslot]
    off = scale_map(d)
    scales = []
    for extra in (0, d):
        raw = block[off + extra].astype(np.uint16) | (block[off + extra + 1].astype(np.uint16) << np.uint16(8))
        scales.append(raw.view(np.float16))
    return uK, scales[0], uV, scales[1]
