"""Pins for the RMSNorm oracle: brute force, closed forms and invariants.

The pages print no worked numeric example, so the oracle is pinned by what the
mathematics fixes ("[Inductor] Codegen Gluon", section 3.1, defines the
computation: the sum of squares of x, then x scaled by rstd and the weight).
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from exact import (
    bf16_fields_value,
    exact_rmsnorm_row,
    midpoint_distance,
    round_exact_to_bf16,
)
from oracle import bf16_bits_to_f64, rmsnorm_fwd, rmsnorm_fwd_f64
from workloads import f32_to_bf16_bits, random_bf16_bits


def _eps32(eps):
    return float(np.float32(eps))


@pytest.mark.parametrize("eps", [1e-6, 1e-5, 0.25])
def test_brute_force_4x8_against_exact_arithmetic(eps):
    """P1: 100 random 4x8 problems, exact rationals + 70-digit sqrt, then RNE."""
    rng = np.random.default_rng(10)
    near_mid = 0
    for trial in range(25):
        x = random_bf16_bits(rng, (4, 8), scale=float(rng.choice([0.01, 1.0, 30.0])))
        w = random_bf16_bits(rng, (8,), lo=0.5, hi=1.5)
        got = rmsnorm_fwd(x, w, eps)
        for i in range(4):
            xs = [bf16_fields_value(int(b)) for b in x[i]]
            ws = [bf16_fields_value(int(b)) for b in w]
            ys = exact_rmsnorm_row(xs, ws, Fraction(_eps32(eps)))
            for j in range(8):
                ref = round_exact_to_bf16(ys[j])
                if int(got[i, j]) != ref:
                    # allowed only when the exact value sits on a rounding
                    # midpoint to within float64 accuracy
                    assert midpoint_distance(ys[j]) < Fraction(1, 10**14), (trial, i, j)
                    near_mid += 1
    assert near_mid <= 2


def test_constant_row_closed_form():
    """P2: a row of constant c gives y_j = w_j * c / sqrt(c^2 + eps)."""
    rng = np.random.default_rng(11)
    w = random_bf16_bits(rng, (64,), lo=0.5, hi=1.5)
    wv = [bf16_fields_value(int(b)) for b in w]
    for c in [1.0, -3.0, 0.0078125, 100.0, 0.3]:
        cb = f32_to_bf16_bits(np.float32([c]))[0]
        cv = bf16_fields_value(int(cb))
        x = np.full((3, 64), cb, dtype=np.uint16)
        for eps in [1e-6, 1e-5, 0.5]:
            got = rmsnorm_fwd(x, w, eps)
            from exact import dec_sqrt

            root = dec_sqrt(cv * cv + Fraction(_eps32(eps)))
            for j in range(64):
                ref = round_exact_to_bf16(Fraction(cv * wv[j]) / Fraction(root))
                assert all(int(got[r, j]) == ref for r in range(3)), (c, eps, j)
        # eps = 0: y_j = sign(c) * w_j exactly
        if c != 0.0:
            got0 = rmsnorm_fwd(x, w, 0.0)
            ref0 = w if c > 0 else (w ^ np.uint16(0x8000))
            assert np.array_equal(got0[0], ref0)


def test_mean_over_n_and_eps_inside_sqrt():
    """A row with one nonzero a among N gives y = w * a / sqrt(a^2/N + eps)."""
    n = 16
    a = 2.0
    x = np.zeros((1, n), dtype=np.uint16)
    x[0, 3] = f32_to_bf16_bits(np.float32([a]))[0]
    w = f32_to_bf16_bits(np.ones(n, dtype=np.float32))
    eps = 0.75  # exact in float32
    y = bf16_bits_to_f64(rmsnorm_fwd(x, w, eps))
    # a / sqrt(4/16 + 0.75) = 2 / 1 = 2 exactly
    assert y[0, 3] == 2.0
    assert np.all(y[0, np.arange(n) != 3] == 0.0)


@pytest.mark.parametrize("k", [-20, -7, 1, 9, 20])
def test_scale_invariance_eps_zero(k):
    """P3: with eps = 0, y(2^k x) == y(x) bit for bit."""
    rng = np.random.default_rng(12)
    x = random_bf16_bits(rng, (16, 256))
    w = random_bf16_bits(rng, (256,), lo=0.5, hi=1.5)
    xs = f32_to_bf16_bits(bf16_bits_to_f64(x).astype(np.float32) * np.float32(2.0**k))
    assert np.array_equal(rmsnorm_fwd(xs, w, 0.0), rmsnorm_fwd(x, w, 0.0))


def test_scale_invariance_as_eps_vanishes():
    """P3: for alpha = 2^k the outputs for alpha*x and x converge as eps -> 0."""
    rng = np.random.default_rng(13)
    x = random_bf16_bits(rng, (32, 512))
    w = random_bf16_bits(rng, (512,), lo=0.5, hi=1.5)
    xs = f32_to_bf16_bits(bf16_bits_to_f64(x).astype(np.float32) * np.float32(0.25))
    prev = None
    for eps in [1e-2, 1e-4, 1e-6, 1e-9, 1e-12]:
        d = np.count_nonzero(rmsnorm_fwd(xs, w, eps) != rmsnorm_fwd(x, w, eps))
        if prev is not None:
            assert d <= prev
        prev = d
    assert prev <= 2  # only near-midpoint cases may remain
    assert np.count_nonzero(rmsnorm_fwd(xs, w, 1e-2) != rmsnorm_fwd(x, w, 1e-2)) > 100


def test_unit_rms():
    """P4: with w = 1 the normalized row has RMS 1 (eps = 0) or sqrt(ms/(ms+eps))."""
    rng = np.random.default_rng(14)
    x = random_bf16_bits(rng, (64, 1024), scale=3.0)
    w = f32_to_bf16_bits(np.ones(1024, dtype=np.float32))
    y = rmsnorm_fwd_f64(x, w, 0.0)
    rms = np.sqrt(np.mean(y * y, axis=1))
    assert np.max(np.abs(rms - 1.0)) < 1e-14
    yb = bf16_bits_to_f64(rmsnorm_fwd(x, w, 0.0))
    rmsb = np.sqrt(np.mean(yb * yb, axis=1))
    assert np.max(np.abs(rmsb - 1.0)) <= 2.0**-9
    eps = 0.125
    xv = bf16_bits_to_f64(x)
    ms = np.mean(xv * xv, axis=1)
    y = rmsnorm_fwd_f64(x, w, eps)
    rms = np.sqrt(np.mean(y * y, axis=1))
    assert np.allclose(rms, np.sqrt(ms / (ms + eps)), rtol=1e-14, atol=0)


def test_odd_symmetry_and_weight_scaling():
    """P5: y(-x) = -y(x); w -> 2^k w gives y -> 2^k y (bit exact)."""
    rng = np.random.default_rng(15)
    x = random_bf16_bits(rng, (16, 384))
    w = random_bf16_bits(rng, (384,), lo=0.5, hi=1.5)
    y = rmsnorm_fwd(x, w, 1e-6)
    yn = rmsnorm_fwd(x ^ np.uint16(0x8000), w, 1e-6)
    assert np.array_equal(yn, y ^ np.uint16(0x8000))
    w4 = f32_to_bf16_bits(bf16_bits_to_f64(w).astype(np.float32) * np.float32(4.0))
    y4 = bf16_bits_to_f64(rmsnorm_fwd(x, w4, 1e-6))
    assert np.array_equal(y4, 4.0 * bf16_bits_to_f64(y))


def test_column_permutation_equivariance():
    """P6: permuting the columns of x and w together permutes y."""
    rng = np.random.default_rng(16)
    x = random_bf16_bits(rng, (32, 300))
    w = random_bf16_bits(rng, (300,), lo=0.5, hi=1.5)
    p = rng.permutation(300)
    y = rmsnorm_fwd(x, w, 1e-6)
    yp = rmsnorm_fwd(x[:, p], w[p], 1e-6)
    diff = np.count_nonzero(yp != y[:, p])
    assert diff <= 3  # summation order only moves near-midpoint cases


def test_n_equals_one_closed_form():
    """P7: N = 1 gives y = w * x / sqrt(x^2 + eps)."""
    for xv, wv, eps in [(0.5, 1.25, 1e-6), (-7.0, 0.75, 0.5), (1e-3, 1.0, 1e-6), (3.0, 2.0, 0.0)]:
        x = f32_to_bf16_bits(np.float32([[xv]]))
        w = f32_to_bf16_bits(np.float32([wv]))
        xe = bf16_fields_value(int(x[0, 0]))
        we = bf16_fields_value(int(w[0]))
        from exact import dec_sqrt

        ref = round_exact_to_bf16(xe * we / Fraction(dec_sqrt(xe * xe + Fraction(_eps32(eps)))))
        assert int(rmsnorm_fwd(x, w, eps)[0, 0]) == ref


def test_special_rows():
    """Zero, NaN and infinite rows follow the IEEE reading of the formula."""
    n = 32
    w = f32_to_bf16_bits(np.linspace(0.5, 1.5, n, dtype=np.float32))
    x = np.zeros((4, n), dtype=np.uint16)
    x[1, 5] = 0x7FC0  # NaN
    x[2] = f32_to_bf16_bits(np.linspace(-1, 1, n, dtype=np.float32))
    x[2, 7] = 0x7F80  # +inf
    x[3] = f32_to_bf16_bits(np.ones(n, dtype=np.float32))
    y = bf16_bits_to_f64(rmsnorm_fwd(x, w, 1e-6))
    assert np.all(y[0] == 0.0)
    assert np.all(np.isnan(y[1]))
    assert math.isnan(y[2, 7])
    others = np.arange(n) != 7
    assert np.all(y[2, others] == 0.0)
    y0 = bf16_bits_to_f64(rmsnorm_fwd(x[:1], w, 0.0))
    assert np.all(np.isnan(y0))


def test_empty_inputs():
    w = f32_to_bf16_bits(np.ones(8, dtype=np.float32))
    assert rmsnorm_fwd(np.zeros((0, 8), dtype=np.uint16), w, 1e-6).shape == (0, 8)


def test_rows_are_independent():
    rng = np.random.default_rng(17)
    x = random_bf16_bits(rng, (20, 128))
    w = random_bf16_bits(rng, (128,), lo=0.5, hi=1.5)
    y = rmsnorm_fwd(x, w, 1e-6)
    for i in [0, 7, 19]:
        assert np.array_equal(rmsnorm_fwd(x[i : i + 1], w, 1e-6)[0], y[i])
