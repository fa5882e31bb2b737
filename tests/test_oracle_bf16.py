"""Pins for the oracle's bf16 conversions (widening and the single rounding)."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import bf16_fields_value, round_exact_to_bf16
from oracle import bf16_bits_to_f64, f64_to_bf16_bits


KNOWN = {
    0x3F80: 1.0,
    0xBF80: -1.0,
    0x4000: 2.0,
    0x4049: 3.140625,
    0x3E80: 0.25,
    0x7F7F: (2 - 2**-7) * 2.0**127,
    0x0080: 2.0**-126,
    0x0001: 2.0**-133,
    0x007F: 127 * 2.0**-133,
    0x0000: 0.0,
    0x7F80: math.inf,
    0xFF80: -math.inf,
}


def test_widen_known_patterns():
    for bits, val in KNOWN.items():
        got = bf16_bits_to_f64(np.array([bits], dtype=np.uint16))[0]
        assert got == val, (hex(bits), got, val)
    neg_zero = bf16_bits_to_f64(np.array([0x8000], dtype=np.uint16))[0]
    assert neg_zero == 0.0 and math.copysign(1.0, neg_zero) < 0
    assert math.isnan(bf16_bits_to_f64(np.array([0x7FC0], dtype=np.uint16))[0])


def test_widen_all_patterns_match_field_decoding():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = bf16_bits_to_f64(bits)
    for b in range(0, 1 << 16, 7):  # every 7th pattern: 9363 exact comparisons
        ref = bf16_fields_value(b)
        g = got[b]
        if isinstance(ref, float) and math.isnan(ref):
            assert math.isnan(g)
        elif isinstance(ref, float):
            assert g == ref
        else:
            assert Fraction(g) == ref, hex(b)


def test_round_trip_all_finite_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    back = f64_to_bf16_bits(vals[finite])
    assert np.array_equal(back, bits[finite])


def test_round_matches_torch_on_float32_values():
    # float32 values round identically whether seen as float32 or float64, so
    # torch's float32 -> bfloat16 conversion (round to nearest even) is an
    # independent reference on these.
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    # force exact ties: low 16 bits == 0x8000
    u[:100_000] = (u[:100_000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(f.astype(np.float64))
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])


def test_round_is_single_rounding():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint between 1 and 1 + 2^-7.
    # Rounding to float32 first would land exactly on the midpoint and then
    # round to even (1.0); a single rounding gives 1 + 2^-7.
    y = 1.0 + 2.0**-8 + 2.0**-30
    assert f64_to_bf16_bits(np.array([y]))[0] == 0x3F81
    assert f64_to_bf16_bits(np.array([1.0 + 2.0**-8]))[0] == 0x3F80  # tie -> even
    assert f64_to_bf16_bits(np.array([1.0 + 3 * 2.0**-8]))[0] == 0x3F82  # tie -> even (up)


def test_round_matches_exact_rational_rounding():
    rng = np.random.default_rng(2)
    mant = rng.random(3000) + 0.5
    expo = rng.integers(-140, 130, size=3000)
    sign = np.where(rng.random(3000) < 0.5, -1.0, 1.0)
    y = sign * np.ldexp(mant, expo)
    got = f64_to_bf16_bits(y)
    for yi, gi in zip(y, got):
        assert int(gi) == round_exact_to_bf16(Fraction(float(yi))), (yi, hex(int(gi)))


def test_round_special_values():
    y = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, -3.4e38, 1e39, 2.0**-134, -(2.0**-134), 2.0**-133 * 1.5])
    got = f64_to_bf16_bits(y)
    assert got[0] == 0x0000 and got[1] == 0x8000
    assert got[2] == 0x7F80 and got[3] == 0xFF80
    assert got[4] == 0x7FC0
    assert got[5] == 0x7F80  # 3.4e38 is above the bf16 overflow threshold
    assert got[6] == 0xFF80
    assert got[7] == 0x7F80
    assert got[8] == 0x0000  # 2^-134 is a tie between 0 and 2^-133 -> even (0)
    assert got[9] == 0x8000
    assert got[10] == 0x0002  # 1.5 * 2^-133 is a tie -> even significand 2


@pytest.mark.parametrize("k", [-20, -3, 0, 5, 40])
def test_round_commutes_with_power_of_two_scaling(k):
    rng = np.random.default_rng(3)
    y = rng.standard_normal(10_000)
    a = f64_to_bf16_bits(y * 2.0**k).astype(np.uint32)
    b = f64_to_bf16_bits(y).astype(np.uint32)
    # scaling by 2^k adds k to the exponent field (no overflow/underflow here)
    nz = (b & 0x7FFF) != 0
    assert np.array_equal(((a >> 7) & 0xFF)[nz].astype(np.int64), ((b >> 7) & 0xFF)[nz].astype(np.int64) + k)
    assert np.array_equal(a & 0x807F, b & 0x807F)
