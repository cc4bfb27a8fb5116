"""Pins for the oracle's FP8 E4M3 (OCP E4M3FN) decode/encode (CPU only):
hand-derived values, every pattern against torch's float8_e4m3fn, every
midpoint between neighbours, saturation, exact rational brute force, and
torch's float32 -> float8_e4m3fn cast (a single rounding) inside the range
where torch does not turn overflow into NaN."""

from fractions import Fraction

import numpy as np
import torch

from oracle.fp8 import E4M3_VALUES, f64_to_fp8_bits, fp8_bits_to_f64

ALL = np.arange(256, dtype=np.uint8)
FINITE = ALL[~np.isnan(E4M3_VALUES)]
POS = np.arange(0x7F, dtype=np.uint8)                      # 0x00 .. 0x7E, increasing


def test_hand_derived_values():
    # 0x38: exponent 7 (bias 7), significand 1.000 -> 1.0; 0x7E: 1.110b x 2^8 = 448;
    # 0x08: smallest normal 2^-6; 0x01: smallest subnormal 1/8 x 2^-6 = 2^-9.
    v = fp8_bits_to_f64(np.array([0x38, 0x7E, 0x08, 0x01, 0x07, 0xB8, 0x00, 0x80], np.uint8))
    assert list(v) == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, -1.0, 0.0, 0.0]
    assert np.isnan(fp8_bits_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_decode_matches_torch_every_pattern():
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8_bits_to_f64(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_roundtrip_and_specials():
    assert np.array_equal(f64_to_fp8_bits(fp8_bits_to_f64(FINITE)), FINITE)
    b = f64_to_fp8_bits(np.array([np.nan, np.inf, -np.inf, 1e9, -500.0, 449.0, -0.0]))
    assert (b[0] & 0x7F) == 0x7F
    assert list(b[1:]) == [0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0x80]


def test_midpoints_to_even():
    lo, hi = POS[:-1], POS[1:]
    a, b = fp8_bits_to_f64(lo), fp8_bits_to_f64(hi)
    mid = (a + b) / 2
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(f64_to_fp8_bits(mid), even)
    assert np.array_equal(f64_to_fp8_bits(-mid), even | 0x80)
    gap = b - a
    assert np.array_equal(f64_to_fp8_bits(mid - gap * 2.0 ** -20), lo)
    assert np.array_equal(f64_to_fp8_bits(mid + gap * 2.0 ** -20), hi)


def test_matches_torch_cast_in_range():
    rng = np.random.default_rng(3)
    f = np.concatenate([rng.standard_normal(200000) * np.exp2(rng.integers(-12, 9, 200000)),
                        rng.uniform(-464, 464, 100000)]).astype(np.float32)
    f = f[np.abs(f) <= 464]
    ref = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f64_to_fp8_bits(f.astype(np.float64)), ref)


def test_random_values_against_exact_rationals():
    rng = np.random.default_rng(5)
    vals = rng.standard_normal(3000) * np.exp2(rng.integers(-11, 9, 3000))
    got = f64_to_fp8_bits(vals)
    table = [Fraction(float(x)) for x in fp8_bits_to_f64(POS)]
    for v, g in zip(vals, got):
        fv = abs(Fraction(float(v)))
        best = min(range(len(table)), key=lambda i: (abs(table[i] - fv), i & 1))
        want = best | (0x80 if v < 0 else 0)
        assert int(g) == want, (v, hex(int(g)), hex(want))
