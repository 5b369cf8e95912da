"""Dense BF16 materialisation of pages -- oracle side (test infrastructure only).

Minima-KV's quality profile runs on materialised pages, while its decode
path attends the mixed pages in place without building a dense dequantised
buffer (arXiv 2608.23834, page 1, Abstract; page 2, "Technical Deep Dive").
The pages give no format for the dense values; the reading taken here is
bfloat16 (the pages measure their compression against a BF16 cache, page 1,
Abstract), rounded to nearest with ties to even from the fp32 value the
cache holds:

* FP8 page: x = fl32(decode(e) * scale) (the same fp32 product the TQ3 demote
  starts from), then bf16.
* TQ3 page: x = (u - 4) * s, exact in fp32, then bf16.
* Rotated TQ3 page (the pool has a sign vector): y = (u - 4) * s is the
  rotated value; x = signs . (H y) / (c d) with H applied by the format's
  fast transform in fp32 (oracle.rotation.unrotate_f32: the butterflies are
  the only rounding), then bf16.  The pages fix no dense form of rotated
  pages; this one spends no precision beyond fp32 and inverts the demote
  side's transform stage by stage.

Every function is pinned by tests/test_oracle_dense.py.
"""
import numpy as np

from . import pool as opool
from . import rotation
from .layout import PAGE

BF16_NAN = 0x7FC0


def bf16_rne_bits(x):
    """uint16 bf16 bits of finite fp32 values x, round to nearest, ties to even.

    Written from the definition: the two bf16 neighbours of x are x with its
    low 16 fraction bits cleared (toward zero) and the next bf16 value away
    from zero; the nearer one is taken (distances compared exactly in fp64),
    and on a tie the one whose last kept bit is 0.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.int64)
    toward = bits & ~0xFFFF                                   # |toward| <= |x|
    away = toward + 0x10000                                   # next magnitude up (same sign)
    xv = x.astype(np.float64)
    lo = (toward.astype(np.uint32)).view(np.float32).astype(np.float64)
    hi = (away.astype(np.uint32)).view(np.float32).astype(np.float64)
    d_lo = np.abs(xv - lo)
    d_hi = np.abs(hi - xv)
    even_lo = ((toward >> 16) & 1) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~even_lo & (d_lo > 0))
    out = np.where(pick_hi, away, toward) >> 16
    return out.astype(np.uint16)


def bf16_to_float(bits):
    """bf16 bits -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def page_fp32(pool, pid):
    """The fp32 values a page holds, [Hkv][2][16][d]: fl32(decode(e) * scale) for
    an FP8 page, (u - 4) * s for a TQ3 page (exact in fp32), and for a rotated
    TQ3 page those values taken back through unrotate_f32."""
    pid = int(pid)
    if pid < pool.n_fp8:
        return opool.fp8_page_values(pool, pid)
    vals = opool.tq3_page_codes_values(pool, pid)              # float64, exact
    f32 = vals.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), vals), "TQ3 values are exact in fp32"
    if pool.signs is not None:
        return rotation.unrotate_f32(f32, pool.signs)
    return f32


def materialize(pool, bt_offsets, bt_pages, b, page_lo, n_pages):
    """Dense bf16 bits (K, V), each uint16 [n_pages * 16][Hkv][d], of logical
    pages [page_lo, page_lo + n_pages) of request b.  A logical page outside the
    request's block table, or an id outside the pool, is all bf16 NaN."""
    Hkv, d = pool.Hkv, pool.d
    K = np.full((n_pages * PAGE, Hkv, d), BF16_NAN, dtype=np.uint16)
    V = np.full((n_pages * PAGE, Hkv, d), BF16_NAN, dtype=np.uint16)
    lo, hi = int(bt_offsets[b]), int(bt_offsets[b + 1])
    for i in range(n_pages):
        entry = lo + page_lo + i
        if entry >= hi or entry >= len(bt_pages):
            continue
        pid = int(bt_pages[entry])
        if not 0 <= pid < pool.n_fp8 + pool.n_tq3:
            continue
        x = page_fp32(pool, pid)                               # [Hkv][2][16][d]
        K[i * PAGE:(i + 1) * PAGE] = bf16_rne_bits(x[:, 0]).transpose(1, 0, 2)
        V[i * PAGE:(i + 1) * PAGE] = bf16_rne_bits(x[:, 1]).transpose(1, 0, 2)
    return K, V
