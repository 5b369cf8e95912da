"""OCP E4M3FN ("FP8 e4m3") codec -- oracle side (test infrastructure only).

Minima-KV keeps Recent and protected Anchor pages in FP8 (arXiv 2608.23834,
page 1, Abstract; page 2, "Technical Deep Dive", first bullet).  The pages do
not name the FP8 variant; the reading taken is OCP E4M3FN: 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111,
largest finite 448, smallest normal 2^-6, subnormals m * 2^-9 (m = 1..7).

Encoding is round-to-nearest-even on the exact fp32 value with saturation of
finite overflow to +-448; -0.0 encodes as 0x80.  NaN inputs are outside the
contract (they map to 0x7F / 0xFF).
"""
import numpy as np

E4M3_MAX = 448.0
NAN_CODES = (0x7F, 0xFF)


def e4m3_decode(codes):
    """Decode uint8 E4M3FN codes to float64 (exact).  NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    out = np.where((c & 0x7F) == 0x7F, np.nan, out)
    return out


def e4m3_encode(y):
    """Encode fp32 values (already divided by the layer scale) to E4M3FN codes.

    Round to nearest, ties to even, on the exact fp32 value; |y| > 448
    saturates to the largest finite code 0x7E (with the sign kept).
    """
    y = np.asarray(y, dtype=np.float32)
    yd = y.astype(np.float64)                      # exact widening
    neg = np.signbit(y)
    a_in = np.abs(yd)
    a = np.where(np.isfinite(a_in), a_in, 0.0)             # non-finite inputs handled at the end
    code = np.zeros(a.shape, dtype=np.int64)

    sub = a < 2.0 ** -6
    # subnormal range: value = m * 2^-9; q = 8 rolls over into the smallest normal
    q_sub = np.rint(np.minimum(a, 1.0) * 2.0 ** 9).astype(np.int64)   # np.rint is ties-to-even
    code = np.where(sub, q_sub, code)

    norm = ~sub
    mant, ex = np.frexp(np.where(norm, a, 1.0))              # a = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1                                           # a = (2*mant) * 2^e, 2*mant in [1, 2)
    frac = (2.0 * mant - 1.0) * 8.0                           # exact: a has 24 significant bits
    q = np.rint(frac).astype(np.int64)
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    code_norm = ((e + 7) << 3) | q
    code = np.where(norm, code_norm, code)

    code = np.where(a_in > E4M3_MAX, 0x7E, code)             # saturate (also 448 < a < 464, and inf)
    code = np.where(np.isnan(yd), 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def e4m3_quantize(x, scale=1.0):
    """y = fl32(x / scale) then E4M3FN encode (the append rule)."""
    y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return e4m3_encode(y.astype(np.float32))
