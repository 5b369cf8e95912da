"""Rotated TQ3: a sign flip and a Walsh-Hadamard rotation before quantising.

Oracle side, test infrastructure only.

The pages name the stale-page format "TQ3" and cite TurboQuant among the
related work (page 1: the abstract and its references); TurboQuant rotates
vectors before scalar quantisation, and the pages do not say whether TQ3 does.
The rotated variant reads it that way, with the plainest fast orthogonal
rotation:

  y = c * H (sigma . x)

per (token, KV head, K or V) row of d channels, where sigma in {-1, +1}^d is a
sign vector the caller gives per layer, H is the d x d Sylvester-Hadamard
matrix (H[i][j] = (-1)^popcount(i & j), H H = d I) and c = 2^-floor(log2(d)/2)
(1/16 at d = 256, 1/8 at d = 128), so c is a power of two and every step but
the butterflies is exact.  The TQ3 rule then quantises y.  Since H^T = H,
x = sigma . (H y) / (c d).  Queries meet rotated keys as q' = H (sigma . q) /
(c d): q' . y = q . x.

H is applied by the fast transform in a fixed order, in fp32: stage s = 0, 1,
..., log2(d) - 1 pairs channels i and i + 2^s (bit s of i clear) and replaces
(a, b) by (a + b, a - b), each rounded to fp32.  That order is part of the
format (the demoted bytes depend on it).
"""
import numpy as np


def sylvester(d):
    """The d x d Sylvester-Hadamard matrix, int64 (pins only)."""
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def rot_scale(d):
    """c = 2^-floor(log2(d) / 2)."""
    lg = int(d).bit_length() - 1
    assert 1 << lg == d, "d must be a power of two"
    return 2.0 ** -(lg // 2)


def fwht_f32(x):
    """H x along the last axis in fp32, stage by stage in the order above."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b          # float32 + float32 -> float32, rounded to nearest even
        v[..., 1, :] = a - b
        h *= 2
    return y


def rotate_f32(x, signs):
    """y = c * H (signs . x), fp32 (signs +-1 and c a power of two: exact)."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(signs).astype(np.float32)
    return (fwht_f32(x * s) * np.float32(rot_scale(x.shape[-1]))).astype(np.float32)


def unrotate_f64(y, signs):
    """x = signs . (H y) / (c d) in fp64 (the exact inverse of the rotation)."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    H = sylvester(d).astype(np.float64)
    return (y @ H) * np.asarray(signs, dtype=np.float64) / (rot_scale(d) * d)


def unrotate_f32(y, signs):
    """x = signs . (H y) / (c d) in fp32, H by the fast transform in the
    format's stage order (fwht_f32); signs and 1 / (c d) (a power of two) are
    exact.  This is the value a dense (materialised) copy of a rotated TQ3
    page holds: y = (u - 4) s is exact in fp32, so only the butterflies round."""
    y = np.asarray(y, dtype=np.float32)
    d = y.shape[-1]
    s = np.asarray(signs).astype(np.float32)
    return (fwht_f32(y) * s * np.float32(1.0 / (rot_scale(d) * d))).astype(np.float32)


def rotate_query_f64(q, signs):
    """q' = H (signs . q) / (c d) in fp64, so that q' . rotate(k) = q . k."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    H = sylvester(d).astype(np.float64)
    return ((q * np.asarray(signs, dtype=np.float64)) @ H) / (rot_scale(d) * d)


def random_signs(d, seed):
    """A seeded sign vector (int8 +-1)."""
    return np.where(np.random.default_rng(seed).integers(0, 2, d) == 0, 1, -1).astype(np.int8)
