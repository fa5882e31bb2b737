"""Pins for the fp16 storage variant of the oracle: the binary16 conversions
and the operators evaluated with dtype="f16"."""

import math
from fractions import Fraction

import numpy as np

from exact import exact_rmsnorm_row, exact_layernorm_row, f16_fields_value, midpoint_distance, round_exact_to_f16
from oracle import f16_bits_to_f64, f64_to_f16_bits, layernorm_fwd, qk_norm_rope_fwd, rmsnorm_fwd


def _f16_bits(rng, shape, scale=1.0, lo=None, hi=None):
    if lo is not None:
        v = lo + (hi - lo) * rng.random(shape)
    else:
        v = rng.standard_normal(shape) * scale
    return v.astype(np.float16).view(np.uint16)


def test_widen_every_pattern_matches_fields():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = f16_bits_to_f64(bits)
    for b in range(0, 1 << 16, 5):
        ref = f16_fields_value(b)
        if isinstance(ref, float):
            assert (math.isnan(ref) and math.isnan(got[b])) or ref == got[b]
        else:
            assert Fraction(got[b]) == ref, hex(b)


def test_round_matches_numpy_float16_conversion():
    # numpy's float64 -> float16 conversion rounds to nearest even: a library
    # routine independent of the oracle's frexp/rint implementation
    rng = np.random.default_rng(80)
    y = np.ldexp(rng.random(300_000) + 0.5, rng.integers(-30, 18, 300_000))
    y *= np.where(rng.random(300_000) < 0.5, -1.0, 1.0)
    ties = np.ldexp((np.arange(2048, 4096) * 2 + 1).astype(np.float64), -12)  # exact midpoints in [1, 2)
    y = np.concatenate([y, ties, -ties])
    with np.errstate(over="ignore"):
        ref = y.astype(np.float16).view(np.uint16)
    assert np.array_equal(f64_to_f16_bits(y), ref)


def test_round_matches_exact_rationals_and_is_single_rounding():
    rng = np.random.default_rng(81)
    y = np.ldexp(rng.random(3000) + 0.5, rng.integers(-28, 17, 3000))
    for v in y:
        assert int(f64_to_f16_bits(np.array([v]))[0]) == round_exact_to_f16(Fraction(float(v)))
    # just above the midpoint between 1 and 1 + 2^-10: one rounding goes up
    assert f64_to_f16_bits(np.array([1.0 + 2.0**-11 + 2.0**-40]))[0] == 0x3C01
    assert f64_to_f16_bits(np.array([1.0 + 2.0**-11]))[0] == 0x3C00
    assert f64_to_f16_bits(np.array([65504.0, 65519.9, 65520.0, 1e6]))[0:4].tolist() == [0x7BFF, 0x7BFF, 0x7C00, 0x7C00]
    sub = f64_to_f16_bits(np.array([2.0**-25, 2.0**-25 * 3, np.nan, -np.inf]))
    assert sub[0:2].tolist() == [0x0000, 0x0002]
    assert (sub[2] & 0x7C00) == 0x7C00 and (sub[2] & 0x03FF) != 0  # NaN stays NaN
    assert sub[3] == 0xFC00


def test_rmsnorm_f16_brute_force():
    rng = np.random.default_rng(82)
    for _ in range(20):
        x = _f16_bits(rng, (4, 8), scale=float(rng.choice([0.01, 1.0, 300.0])))
        w = _f16_bits(rng, (8,), lo=0.5, hi=1.5)
        y = rmsnorm_fwd(x, w, 1e-6, dtype="f16")
        for i in range(4):
            xs = [f16_fields_value(int(b)) for b in x[i]]
            ws = [f16_fields_value(int(b)) for b in w]
            ex = exact_rmsnorm_row(xs, ws, Fraction(float(np.float32(1e-6))))
            for j in range(8):
                if int(y[i, j]) != round_exact_to_f16(ex[j]):
                    assert midpoint_distance(ex[j]) < Fraction(1, 10**12)


def test_layernorm_f16_brute_force():
    rng = np.random.default_rng(83)
    for _ in range(10):
        x = _f16_bits(rng, (4, 8), scale=3.0)
        w = _f16_bits(rng, (8,), lo=0.5, hi=1.5)
        b = _f16_bits(rng, (8,), lo=-0.5, hi=0.5)
        y = layernorm_fwd(x, w, b, 1e-5, dtype="f16")
        for i in range(4):
            ex = exact_layernorm_row([f16_fields_value(int(v)) for v in x[i]], [f16_fields_value(int(v)) for v in w],
                                     [f16_fields_value(int(v)) for v in b], Fraction(float(np.float32(1e-5))))
            for j in range(8):
                assert int(y[i, j]) == round_exact_to_f16(ex[j])


def test_qk_f16_position_zero_is_per_head_rmsnorm():
    rng = np.random.default_rng(84)
    t, hq, hk, d = 4, 2, 1, 128
    qkv = _f16_bits(rng, (t, (hq + 2 * hk) * d))
    q_w = _f16_bits(rng, (d,), lo=0.5, hi=1.5)
    k_w = _f16_bits(rng, (d,), lo=0.5, hi=1.5)
    out = qk_norm_rope_fwd(qkv, q_w, k_w, np.zeros(t, np.int64), hq, hk, d, 1e-6, 1e6, dtype="f16")
    heads = qkv[:, : (hq + hk) * d].reshape(t, hq + hk, d)
    assert np.array_equal(out[:, : hq * d], rmsnorm_fwd(heads[:, :hq].reshape(-1, d), q_w, 1e-6, dtype="f16").reshape(t, -1))
    assert np.array_equal(out[:, hq * d : (hq + hk) * d],
                          rmsnorm_fwd(heads[:, hq:].reshape(-1, d), k_w, 1e-6, dtype="f16").reshape(t, -1))
    assert np.array_equal(out[:, (hq + hk) * d :], qkv[:, (hq + hk) * d :])
