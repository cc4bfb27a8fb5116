"""FP8 E4M3 (OCP "E4M3FN") decode/encode for the oracle (test infrastructure only).

Format: 1 sign bit, 4 exponent bits (bias 7), 3 stored significand bits.
Exponent field 0 holds subnormals m/8 * 2^-6; fields 1..15 hold normals
(1 + m/8) * 2^(e-7). The two patterns with all exponent and significand bits
set (0x7F, 0xFF) are NaN; there is no infinity, and the largest finite value
is 1.75 * 2^8 = 448.

Encoding rounds a float64 value ONCE to the nearest E4M3 value (ties to even),
as for bf16, and saturates: results beyond +-448 become +-448 (the
"saturate to finite" convention for activations). NaN stays NaN.
"""

import numpy as np

E4M3_MIN_NORMAL_EXP = -6
E4M3_SIG_BITS = 4              # 1 implicit + 3 stored
E4M3_MAX = 448.0


def _table():
    v = np.empty(256, dtype=np.float64)
    for b in range(256):
        s = -1.0 if b & 0x80 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            v[b] = np.nan
        elif e == 0:
            v[b] = s * (m / 8.0) * 2.0 ** -6
        else:
            v[b] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


E4M3_VALUES = _table()


def fp8_bits_to_f64(bits):
    """Exact value of E4M3 bit patterns (uint8 array) as float64."""
    return E4M3_VALUES[np.asarray(bits, dtype=np.uint8).astype(np.intp)]


def f64_to_fp8_bits(values):
    """Round float64 values once to E4M3 (nearest, ties to even, saturating) -> uint8."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    nan = np.isnan(v)
    safe = np.where(np.isfinite(a), a, E4M3_MAX)
    _, k = np.frexp(safe)
    lead_exp = k.astype(np.int64) - 1
    q_exp = np.maximum(lead_exp, E4M3_MIN_NORMAL_EXP) - (E4M3_SIG_BITS - 1)
    mag = np.ldexp(np.rint(np.ldexp(safe, -q_exp)), q_exp)   # exact scalings around one rint
    mag = np.minimum(mag, E4M3_MAX)
    # the rounded magnitude is an E4M3 value: look its pattern up
    pos = E4M3_VALUES[:0x7F]                                  # 0x00 .. 0x7E, increasing
    idx = np.searchsorted(pos, mag)
    bits = idx.astype(np.uint8)
    bits = np.where(np.signbit(v), bits | np.uint8(0x80), bits)
    return np.where(nan, np.uint8(0x7F), bits).astype(np.uint8)
