"""Pins for the oracle's bf16 decode/encode (CPU only).

The oracle rounds its float64 results once to bf16. These tests tie that
rounding to things outside the oracle: the IEEE definition checked with exact
rational arithmetic, every bf16 pattern, every midpoint between neighbours,
and torch's float32 -> bfloat16 cast (a single correct rounding) on float32
inputs.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
EXP = (ALL.astype(np.uint32) >> 7) & 0xFF
FINITE = ALL[EXP != 0xFF]
POS_FINITE = FINITE[(FINITE & 0x8000) == 0]          # 0x0000 .. 0x7F7F, increasing values


def test_decode_matches_float32_upper_half():
    # bf16 is the top half of a binary32 pattern; torch agrees on every pattern.
    got = bf16_bits_to_f64(ALL)
    ref = torch.from_numpy(ALL.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_roundtrip_every_finite_pattern():
    assert np.array_equal(f64_to_bf16_bits(bf16_bits_to_f64(FINITE)), FINITE)


def test_specials():
    v = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0])
    b = f64_to_bf16_bits(v)
    assert list(b[:2]) == [0x7F80, 0xFF80]
    assert (b[2] & 0x7FFF) > 0x7F80          # a NaN
    assert list(b[3:]) == [0x0000, 0x8000]


def test_midpoints_go_to_even_and_nearby_values_to_nearest():
    lo = POS_FINITE[:-1]
    hi = POS_FINITE[1:]
    a = bf16_bits_to_f64(lo)
    b = bf16_bits_to_f64(hi)
    mid = (a + b) / 2                      # exact: both have <= 8 significant bits
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(f64_to_bf16_bits(mid), even)
    assert np.array_equal(f64_to_bf16_bits(-mid), even | 0x8000)
    # just below / above the midpoint: nearest neighbour, whatever the parity
    gap = b - a
    assert np.array_equal(f64_to_bf16_bits(mid - gap * 2.0 ** -30), lo)
    assert np.array_equal(f64_to_bf16_bits(mid + gap * 2.0 ** -30), hi)


def test_overflow_threshold():
    max_finite = bf16_bits_to_f64(np.array([0x7F7F], np.uint16))[0]
    half_ulp = 2.0 ** (127 - 8)
    assert f64_to_bf16_bits(np.array([max_finite + half_ulp * 0.999]))[0] == 0x7F7F
    assert f64_to_bf16_bits(np.array([max_finite + half_ulp]))[0] == 0x7F80   # tie -> even = inf
    assert f64_to_bf16_bits(np.array([1e300]))[0] == 0x7F80


def test_single_rounding_not_double():
    # 1 + 2^-8 + 2^-40: through float32 it becomes 1 + 2^-8 (a bf16 tie) and then 1.0;
    # rounded once it is just above the tie and goes up to 1 + 2^-7.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(v) == np.float32(1.0 + 2.0 ** -8)
    assert f64_to_bf16_bits(np.array([v]))[0] == 0x3F81
    assert f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def test_float32_inputs_match_torch_cast():
    # For float32-representable inputs one rounding is one rounding: torch's
    # float32 -> bfloat16 cast rounds to nearest even.
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    edges = []
    for e in range(1, 255):
        for m in (0, 1, 0x7FFF, 0x8000, 0x8001, 0x17FFF, 0x18000, 0x7FFFFF):
            edges.append((e << 23) | m)
    edges += list(range(0, 70000, 7))      # subnormals
    f = np.concatenate([f, np.array(edges, np.uint32).view(np.float32)])
    f = np.concatenate([f, -f])
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, ref)


def _nearest_bf16_exact(v):
    """Brute force with exact rationals: the finite bf16 nearest to v, ties to even."""
    fv = Fraction(v)
    vals = bf16_bits_to_f64(POS_FINITE)
    idx = int(np.searchsorted(vals, abs(v)))
    best = None
    for j in (idx - 1, idx, idx + 1):
        if 0 <= j < len(POS_FINITE):
            d = abs(Fraction(float(vals[j])) - abs(fv))
            key = (d, int(POS_FINITE[j]) & 1)
            if best is None or key < best[0]:
                best = (key, int(POS_FINITE[j]))
    bits = best[1]
    return bits | (0x8000 if v < 0 else 0)


def test_random_float64_against_exact_rational_brute_force():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000)),
        rng.standard_normal(1000),
    ])
    got = f64_to_bf16_bits(vals)
    for v, g in zip(vals, got):
        assert int(g) == _nearest_bf16_exact(float(v)), v


@pytest.mark.parametrize("v,bits", [(0.4, 0x3ECD), (0.8, 0x3F4D), (1.6, 0x3FCD), (-0.6, 0xBF1A)])
def test_hand_rounded_values(v, bits):
    # Worked by hand. 0.4 = 1.1001100|1100..._2 x 2^-2: the bits after the 7 kept
    # ones start 11..., above half, so 1.1001101_2 x 2^-2 = 0x3ECD. 0.8 and 1.6
    # have the same significand one and two binades up. 0.6 = 1.0011001|1001..._2
    # x 2^-1: above half again, 1.0011010_2 x 2^-1 = 0x3F1A, with the sign 0xBF1A.
    assert f64_to_bf16_bits(np.array([v]))[0] == bits
