"""Pins for the oracle's TQ3 quantiser and triple packing (oracle/tq3.py, oracle/layout.py).

Pinned against: an exhaustive round trip over all 2^24 triples, a brute-force
nearest-level search (argmin with ties to even) over every finite positive
fp16 scale, the complete demotion domain at scale 1, and an exact rational
computation of the scale rule.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8, layout, tq3


def test_triple_roundtrip_exhaustive():
    step = 1 << 20
    for lo in range(0, 1 << 24, step):
        w = np.arange(lo, lo + step, dtype=np.uint32)
        b = np.stack([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], axis=-1).astype(np.uint8)
        codes = layout.unpack_triples(b)
        assert codes.max() <= 7
        assert np.array_equal(layout.pack_triples(codes), b)
        # code octets -> bytes -> code octets is the identity as well
        assert np.array_equal(layout.unpack_triples(layout.pack_triples(codes)), codes)


def test_triple_scalar_matches_vector():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 8, size=(500, 8))
    vec = layout.pack_triples(codes)
    for c, v in zip(codes, vec):
        assert layout.pack_triple(list(c)) == bytes(v)
        assert layout.unpack_triple(bytes(v)) == list(c)
    # code k occupies bits [3k, 3k+3) of the little-endian 24-bit word
    assert layout.pack_triple([7, 0, 0, 0, 0, 0, 0, 0]) == bytes([0x07, 0, 0])
    assert layout.pack_triple([0, 0, 1, 0, 0, 0, 0, 0]) == bytes([0x40, 0, 0])
    assert layout.pack_triple([0, 0, 2, 0, 0, 0, 0, 0]) == bytes([0x80, 0, 0])
    assert layout.pack_triple([0, 0, 4, 0, 0, 0, 0, 0]) == bytes([0x00, 0x01, 0])
    assert layout.pack_triple([0, 0, 0, 0, 0, 0, 0, 7]) == bytes([0, 0, 0xE0])


def _brute_code(x, s):
    """argmin_q |x - q s| over q in -3..3 with ties to the even q (exact in fp64)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    s = np.asarray(s, dtype=np.float16).astype(np.float64)
    qs = np.arange(-3, 4)
    err = np.abs(x[..., None] - qs * s[..., None])
    best = err.min(axis=-1, keepdims=True)
    tie = err == best
    # among tied candidates prefer the even q
    pref = np.where(tie & (qs % 2 == 0), 0, np.where(tie, 1, 2))
    q = qs[np.argmin(pref, axis=-1)]
    return np.where(s == 0, 0, q)


def test_code_bruteforce_all_fp16_scales():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)          # every finite positive fp16
    s = bits.view(np.float16)
    s32 = s.astype(np.float32)
    xs = []
    for k in (0.5, 1.5, 2.5, 3.5, 1.0, 2.0, 3.0, 0.25, 3.2):
        t = (np.float32(k) * s32).astype(np.float32)
        xs += [t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(0))]
    X = np.stack(xs, axis=-1)
    S = np.broadcast_to(s[:, None], X.shape)
    for sign in (1, -1):
        got = tq3.tq3_code(sign * X, S)
        want = _brute_code(sign * X, S)
        bad = np.nonzero(got != want)
        assert got.shape == want.shape and len(bad[0]) == 0, (X[bad][:5], S[bad][:5], got[bad][:5], want[bad][:5])


def test_code_exhaustive_demote_domain_scale1():
    vals = fp8.e4m3_decode(np.arange(256))
    fin = vals[~np.isnan(vals)].astype(np.float32)
    mags = np.unique(np.abs(fin))
    assert len(mags) == 127
    X, A = np.meshgrid(fin, mags, indexing="ij")
    ok = np.abs(X) <= A                                     # x must lie in a group whose absmax is a
    s = tq3.tq3_scale(A)
    got = tq3.tq3_code(X, s)
    want = _brute_code(X, s)
    assert np.array_equal(got[ok], want[ok])


def _round_rational(r, p, emin, emax_val):
    """Round a non-negative Fraction to a binary float with p significant bits,
    minimum exponent emin (subnormal spacing 2^(emin-p+1)), ties to even;
    values above emax_val return None (overflow)."""
    if r == 0:
        return Fraction(0)
    e = r.numerator.bit_length() - r.denominator.bit_length()
    while Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = r / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    out = fl * ulp
    return None if out > emax_val else out


def test_scale_rule_exact_rational():
    vals = fp8.e4m3_decode(np.arange(256))
    mags = np.unique(np.abs(vals[~np.isnan(vals)]))
    rng = np.random.default_rng(3)
    extra = np.exp(rng.uniform(-80, 80, 300)).astype(np.float32)
    a_all = np.concatenate([mags.astype(np.float32), extra, np.float32([1e-30, 65504 * 3, 2e5, 3.4e38])])
    got = tq3.tq3_scale(a_all)
    for a, g in zip(a_all, got):
        r32 = _round_rational(Fraction(float(a)) / 3, 24, -126, Fraction(2) ** 128)
        r16 = _round_rational(r32, 11, -14, Fraction(65504))
        want = 65504.0 if r16 is None else float(r16)
        assert float(g) == want, (a, float(g), want)


def test_quantize_scalar_matches_vector():
    rng = np.random.default_rng(4)
    for _ in range(200):
        x = (rng.standard_normal(32) * np.exp(rng.uniform(-6, 6))).astype(np.float32)
        if rng.random() < 0.1:
            x[rng.integers(32)] *= 40
        u, s = tq3.quantize_groups(x)
        us, ss = tq3.quantize_scalar(x)
        assert list(u) == us and float(s) == ss


def test_zero_group_and_code_range():
    u, s = tq3.quantize_groups(np.zeros(32, dtype=np.float32))
    assert float(s) == 0.0 and np.all(u == 4)
    x = np.random.default_rng(5).standard_normal((1000, 32)).astype(np.float32)
    u, s = tq3.quantize_groups(x)
    assert u.min() >= 1 and u.max() <= 7
    v = tq3.dequantize_groups(u, s)
    # every element within half a step (plus the fp16 rounding slack of s at the clamp)
    err = np.abs(v - x.astype(np.float64))
    s64 = s.astype(np.float64)[:, None]
    a = np.abs(x).max(axis=1, keepdims=True).astype(np.float64)
    assert np.all(err <= np.maximum(0.5 * s64, a - 3 * s64) + 1e-12)
    # the group's absmax element is represented by +-3 (or +-2 if ties force it) codes
    assert np.all(np.abs(u.astype(int) - 4).max(axis=1) == 3)
