"""bfloat16 codec for the oracle, written from the number format's definition.

bf16 is the upper 16 bits of an IEEE-754 binary32: 1 sign bit, 8 exponent
bits, 7 stored significand bits. Decoding is exact. Encoding rounds a real
value to the nearest bf16 value, ties to the value whose last significand bit
is 0, which is IEEE round-to-nearest-even at 8 significant bits with binary32's
exponent range (subnormals included).
"""

import numpy as np

_BF16_MAX = float(np.float32(2.0 ** 127 * (2.0 - 2.0 ** -7)))


def bf16_to_f64(u) -> np.ndarray:
    """uint16 bit patterns -> float64 values (exact)."""
    u = np.asarray(u, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # signalling NaN patterns stay NaN
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Real values (float64 array) -> nearest bf16 bit patterns, ties to even.

    For finite x with |x| in [2**e, 2**(e+1)) the bf16 spacing is
    2**(max(e, -126) - 7); x is divided by that power of two (exact), rounded
    to an integer with ties to even (numpy.rint), and scaled back (exact).
    Values whose rounded magnitude exceeds the largest finite bf16 become
    infinities; NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    xf = x[finite]
    _, ex = np.frexp(xf)               # xf = m * 2**ex, 0.5 <= |m| < 1
    e = np.maximum(ex.astype(np.int64) - 1, -126)
    spacing = np.ldexp(1.0, (e - 7).astype(np.int32))
    y = np.rint(xf / spacing) * spacing
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, y), y)
    # y is exactly representable in bf16, hence in binary32
    out[finite] = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nonfinite = ~finite
    xn = x[nonfinite]
    bits = np.where(np.isnan(xn), 0x7FC0, np.where(xn > 0, 0x7F80, 0xFF80))
    out[nonfinite] = bits.astype(np.uint16)
    return out


def f32_to_bf16(x) -> np.ndarray:
    """float32 array -> bf16 bit patterns (round to nearest even)."""
    return round_bf16(np.asarray(x, dtype=np.float32).astype(np.float64))
