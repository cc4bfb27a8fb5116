"""bfloat16 decode/encode for the oracle (test infrastructure only).

bfloat16 is the upper 16 bits of an IEEE-754 binary32 pattern: 1 sign bit,
8 exponent bits, 7 stored significand bits. Decoding is therefore exact.

Encoding rounds a float64 value ONCE to the nearest bfloat16, ties to even.
It never passes through float32 first: rounding to float32 and then to
bfloat16 can land on the wrong side of a bf16 midpoint (double rounding).

The method is the textbook one: find the spacing ``q`` of bf16 numbers at the
value's magnitude (8 significant bits for normal numbers, a fixed 2**-133 for
subnormals), scale by ``1/q`` (exact, a power of two), round to an integer
with ties-to-even (``numpy.rint``), scale back (exact). The rounded magnitude
is then a bf16 number, so its float32 pattern has 16 zero low bits.
"""

import numpy as np

BF16_MIN_NORMAL_EXP = -126   # smallest normal binary exponent
BF16_SIG_BITS = 8            # significant bits of a normal bf16 (1 implicit + 7)
BF16_OVERFLOW = 2.0 ** 128   # first magnitude past the largest finite bf16 binade


def bf16_bits_to_f64(bits):
    """Exact value of bf16 bit patterns (uint16 array) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(values):
    """Round float64 values once to bf16 (nearest, ties to even) -> uint16.

    NaN maps to the quiet NaN 0x7FC0 (sign kept); magnitudes that round to
    2**128 or beyond map to infinity, as IEEE round-to-nearest requires.
    """
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a)
    safe = np.where(finite, a, 0.0)

    # a = m * 2**k with m in [0.5, 1): the leading bit is 2**(k-1).
    _, k = np.frexp(safe)
    lead_exp = k.astype(np.int64) - 1
    # bf16 spacing at this magnitude: 8 significant bits for normals, fixed
    # below the normal range (subnormals share the spacing of the smallest
    # normal binade).
    q_exp = np.maximum(lead_exp, BF16_MIN_NORMAL_EXP) - (BF16_SIG_BITS - 1)
    scaled = np.ldexp(safe, -q_exp)       # exact: power-of-two scaling
    rounded = np.rint(scaled)             # round half to even
    mag = np.ldexp(rounded, q_exp)        # exact

    overflow = mag >= BF16_OVERFLOW
    mag = np.where(overflow, 0.0, mag)
    hi = (mag.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    hi = np.where(overflow | np.isinf(a), np.uint16(0x7F80), hi)
    hi = np.where(np.isnan(v), np.uint16(0x7FC0), hi)
    sign = np.where(np.signbit(v), np.uint16(0x8000), np.uint16(0))
    return (hi | sign).astype(np.uint16)
