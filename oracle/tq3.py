"""TQ3: 3-bit symmetric group quantiser -- oracle side (test infrastructure only).

The pages say only that older non-anchor pages "move to packed TQ3" and call
TQ3 a 3-bit format (arXiv 2608.23834, page 1, Abstract; page 2, "Technical
Deep Dive", first bullet).  The readings taken here:

* groups of 32 consecutive channels of one token of one KV head, K and V
  separately, with one fp16 scale per group;
* symmetric codes q in {-3..3} (seven of the eight 3-bit levels), stored as
  u = q + 4 in [1, 7]; u = 0 is never produced and decodes as -4;
* scale s = fp16_RNE(fl32(a / 3)) with a = max |x_i| over the group (an IEEE
  fp32 divide, then round-to-nearest-even to fp16, saturating at 65504);
* q_i = the exact nearest integer to x_i / s, ties to even, clamped to +-3,
  and q_i = 0 when s = 0.  Because s has at most 11 significant bits the
  half-integer thresholds 0.5 s, 1.5 s and 2.5 s are exact in fp32, so the
  rule is evaluated as exact comparisons, never as rint(x / s) in fp32;
* the source values are the FP8-dequantised page values x_i =
  fl32(decode_e4m3(e_i) * k_or_v_scale) -- demotion sees the FP8 page.

Dequantisation: v = (u - 4) * s, exact in fp32 and fp64.
"""
import numpy as np

GROUP = 32
FP16_MAX = 65504.0


def tq3_scale(absmax):
    """s = fp16_RNE(fl32(a / 3.0f)), saturating to 65504.  Returns float16."""
    a = np.asarray(absmax, dtype=np.float32)
    r = (a / np.float32(3.0)).astype(np.float32)        # IEEE fp32 divide (correctly rounded)
    with np.errstate(over="ignore"):
        s = r.astype(np.float16)                         # numpy float32->float16 is RNE
    s = np.where(np.isinf(s), np.float16(FP16_MAX), s)
    return s.astype(np.float16)


def tq3_code(x, s):
    """Signed code q in {-3..3}: nearest integer to x/s, ties to even, clamped.

    x: fp32 values; s: fp16 scale broadcastable to x.  Evaluated with exact
    fp32 thresholds: |q| = [|x| > s/2] + [|x| >= 3s/2] + [|x| > 5s/2].
    """
    x = np.asarray(x, dtype=np.float32)
    s32 = np.asarray(s, dtype=np.float16).astype(np.float32)
    ax = np.abs(x)
    half = np.float32(0.5) * s32          # exact (power-of-two scaling of an fp16 value)
    three_half = np.float32(1.5) * s32    # exact: <= 13 significant bits
    five_half = np.float32(2.5) * s32     # exact: <= 14 significant bits
    mag = (ax > half).astype(np.int64) + (ax >= three_half).astype(np.int64) + (ax > five_half).astype(np.int64)
    mag = np.where(s32 == 0, 0, mag)
    return np.where(np.signbit(x), -mag, mag).astype(np.int64)


def quantize_groups(x):
    """Quantise x[..., 32] (fp32) per group.  Returns (u uint8[..., 32], s float16[...])."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == GROUP
    a = np.max(np.abs(x), axis=-1)
    s = tq3_scale(a)
    q = tq3_code(x, s[..., None])
    u = (q + 4).astype(np.uint8)
    return u, s


def dequantize_groups(u, s):
    """v = (u - 4) * s in float64 (exact)."""
    return (np.asarray(u, dtype=np.int64) - 4).astype(np.float64) * np.asarray(s, dtype=np.float16).astype(np.float64)[..., None]


def quantize_scalar(xs):
    """Scalar (pure Python) version of one group, for tiny cross-checks.

    Returns (list of u, fp16 scale as float).  Implements the same rule one
    element at a time: absmax, fp32 divide, fp16 rounding, threshold codes.
    """
    xs = [float(np.float32(v)) for v in xs]
    a = max(abs(v) for v in xs)
    s = float(tq3_scale(np.float32(a)))
    us = []
    for v in xs:
        av = abs(v)
        if s == 0.0:
            m = 0
        else:
            m = int(av > 0.5 * s) + int(av >= 1.5 * s) + int(av > 2.5 * s)
        neg = np.signbit(np.float32(v))
        us.append((-m if neg else m) + 4)
    return us, s
