"""Pins for the oracle's E4M3FN codec (oracle/fp8.py).

Pinned against: published OCP points (tests/golden/e4m3_points.txt), torch's
float8_e4m3fn (a library codec) on all 256 codes and on in-range values,
and a brute-force nearest-value search with ties to the even code.
"""
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_points.txt")


def _finite_table():
    codes = np.arange(256)
    vals = fp8.e4m3_decode(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]


def test_golden_points():
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        got = fp8.e4m3_decode(np.array([int(c, 16)]))[0]
        if v == "nan":
            assert np.isnan(got)
        else:
            assert got == float(v) and np.signbit(got) == v.startswith("-")
            if not np.isnan(float(v)):
                assert int(fp8.e4m3_encode(np.float32(float(v)))) == int(c, 16)


def test_decode_matches_library_all_codes():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    ours = fp8.e4m3_decode(np.arange(256))
    both_nan = np.isnan(lib) & np.isnan(ours)
    assert np.all(both_nan | (lib == ours))


def test_roundtrip_every_finite_code():
    codes, vals = _finite_table()
    back = fp8.e4m3_encode(vals.astype(np.float32))
    # -0.0 (0x80) keeps its sign bit
    assert np.array_equal(back, codes.astype(np.uint8))


def _brute_encode(y):
    codes, vals = _finite_table()
    out = []
    for v in np.asarray(y, dtype=np.float32).astype(np.float64):
        a = abs(v)
        if a > 448.0:
            a = 448.0
        pos = [(c, x) for c, x in zip(codes, vals) if x >= 0 and c < 0x80]
        best = min(abs(x - a) for _, x in pos)
        cands = [c for c, x in pos if abs(x - a) == best]
        c = [c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]
        if np.signbit(v):
            c |= 0x80
        out.append(c)
    return np.array(out, dtype=np.uint8)


def test_midpoints_round_to_even():
    codes, vals = _finite_table()
    pos = np.sort(np.unique(np.abs(vals)))
    mids = (pos[:-1] + pos[1:]) / 2.0              # exact in fp32 (<= 5 significant bits)
    assert len(mids) == 126
    for sign in (1.0, -1.0):
        y = (sign * mids).astype(np.float32)
        assert np.array_equal(fp8.e4m3_encode(y), _brute_encode(y))


def test_random_values_vs_bruteforce_and_library():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.standard_normal(3000) * 30,
                        rng.standard_normal(1000) * 0.01,
                        np.exp(rng.uniform(-12, 6.2, 1000)) * rng.choice([-1, 1], 1000)]).astype(np.float32)
    ours = fp8.e4m3_encode(y)
    assert np.array_equal(ours, _brute_encode(y))
    inrange = np.abs(y) <= 448.0
    lib = torch.from_numpy(y[inrange]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours[inrange], lib)


def test_saturation():
    y = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e4, 3.0e38, -500.0, -1e30], dtype=np.float32)
    got = fp8.e4m3_encode(y)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_scale_divides_first():
    x = np.array([3.0, -7.5, 100.0], dtype=np.float32)
    assert np.array_equal(fp8.e4m3_quantize(x, 2.0), fp8.e4m3_encode(x / np.float32(2.0)))


def test_encode_is_monotone():
    y = np.sort(np.random.default_rng(1).uniform(-500, 500, 20000)).astype(np.float32)
    v = fp8.e4m3_decode(fp8.e4m3_encode(y))
    assert np.all(np.diff(v) >= 0)
