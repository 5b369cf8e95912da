"""Pins for the oracle's page byte layout (oracle/layout.py)."""
import os

import numpy as np

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tq3_layout_d128.txt")


def test_golden_positions_d128():
    ktri, kslot = layout.k_code_map(128)
    vtri, vslot = layout.v_code_map(128)
    sm = layout.scale_map(128)
    n = 0
    for line in open(GOLDEN):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        n += 1
        if f[0] in ("K", "V"):
            t, c, byte, slot = map(int, f[1:])
            tri, sl = (ktri, kslot) if f[0] == "K" else (vtri, vslot)
            assert (tri[t, c], sl[t, c]) == (byte, slot), line
        else:
            t, g, byte = map(int, f[1:])
            assert sm[t, g] + (128 if f[0] == "SV" else 0) == byte, line
    assert n == 18


def _check_bijection(d):
    for tri, slot, lo, hi in ((*layout.k_code_map(d), 0, 6 * d), (*layout.v_code_map(d), 6 * d, 12 * d)):
        assert tri.min() >= lo and tri.max() + 3 <= hi
        assert np.all((tri - lo) % 3 == 0)
        keys = tri * 8 + slot
        assert len(np.unique(keys)) == 16 * d            # every (triple, slot) used exactly once
        assert len(np.unique(tri)) * 3 == 6 * d          # and every code byte belongs to a triple
    sm = layout.scale_map(d)
    assert sm.min() == 12 * d and sm.max() + 2 == 13 * d and len(np.unique(sm)) == 16 * (d // 32)


def test_maps_are_bijections():
    for d in (128, 256):
        _check_bijection(d)
    assert layout.tq3_head_bytes(256) == 3584 and layout.tq3_page_bytes(4, 256) == 14336
    assert layout.fp8_page_bytes(4, 256) == 32768


def test_v_triple_holds_two_channels_four_tokens():
    d = 256
    tri, slot = layout.v_code_map(d)
    for start in np.unique(tri)[:64]:
        t, c = np.nonzero(tri == start)
        assert len(t) == 8
        assert len(set(c)) == 2 and max(c) - min(c) == 1 and min(c) % 2 == 0
        assert len(set(t)) == 4 and min(t) % 4 == 0 and max(t) - min(t) == 3


def test_head_block_roundtrip():
    rng = np.random.default_rng(0)
    for d in (128, 256):
        G = d // 32
        uK = rng.integers(0, 8, (16, d)).astype(np.uint8)
        uV = rng.integers(0, 8, (16, d)).astype(np.uint8)
        sK = rng.standard_normal((16, G)).astype(np.float16)
        sV = rng.standard_normal((16, G)).astype(np.float16)
        blk = layout.encode_tq3_head(uK, sK, uV, sV)
        a, b, c, e = layout.decode_tq3_head(blk, d)
        assert np.array_equal(a, uK) and np.array_equal(c, uV)
        assert np.array_equal(b.view(np.uint16), sK.view(np.uint16))
        assert np.array_equal(e.view(np.uint16), sV.view(np.uint16))


def test_k_block_read_as_six_bit_fields():
    # The map's second description: a block of 4 K triples, read as a 96-bit
    # little-endian stream of 16 six-bit fields, holds in field f channel
    # 8 j + f % 8 of group 4 b + f // 8 (low three bits) and of group
    # 4 b + 2 + f // 8 (high three bits).  Slot k of a triple is bits [3k, 3k+3).
    for d in (128, 256):
        G = d // 32
        tri, slot = layout.k_code_map(d)
        for t in (0, 7, 15):
            for j in range(4):
                for b in range(G // 4):
                    base = t * 3 * d // 8 + 3 * (j * G + 4 * b)
                    for f in range(16):
                        for part, g in ((0, 4 * b + f // 8), (1, 4 * b + 2 + f // 8)):
                            c = 32 * g + 8 * j + f % 8
                            bit = 6 * f + 3 * part
                            assert tri[t, c] == base + 3 * (bit // 24), (d, t, c)
                            assert slot[t, c] == (bit % 24) // 3, (d, t, c)


def test_v_slots_alternate_channels_token_major():
    # slot 2 r: channel a (even) of token 4 j + r; slot 2 r + 1: channel b = a + 1
    d = 256
    tri, slot = layout.v_code_map(d)
    for start in np.unique(tri)[:64]:
        t, c = np.nonzero(tri == start)
        by_slot = {int(slot[ti, ci]): (int(ti), int(ci)) for ti, ci in zip(t, c)}
        a, t0 = by_slot[0][1], by_slot[0][0]
        for k in range(8):
            assert by_slot[k] == (t0 + k // 2, a + k % 2)
