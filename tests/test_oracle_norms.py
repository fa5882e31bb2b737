"""Pins for the add+RMSNorm, LayerNorm and L2Norm oracles (exact arithmetic,
closed forms and invariants; the pages print no worked example)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import (
    bf16_fields_value,
    exact_l2norm_row,
    exact_layernorm_row,
    exact_rmsnorm_row,
    midpoint_distance,
    round_exact_to_bf16,
)
from oracle import (
    add_rmsnorm_fwd,
    bf16_bits_to_f64,
    l2norm_fwd,
    l2norm_fwd_f64,
    layernorm_fwd,
    layernorm_fwd_f64,
    rmsnorm_fwd,
)
from workloads import f32_to_bf16_bits, random_bf16_bits


def _vals(bits):
    return [bf16_fields_value(int(b)) for b in np.asarray(bits).reshape(-1)]


def _eps32(e):
    return Fraction(float(np.float32(e)))


def _check_exact(got, exact_vals, slack=2):
    near = 0
    for g, v in zip(np.asarray(got).reshape(-1), exact_vals):
        if int(g) != round_exact_to_bf16(v):
            assert midpoint_distance(v) < Fraction(1, 10**14)
            near += 1
    assert near <= slack


# ---------------- residual add + RMSNorm ----------------

def test_add_is_single_rounding_of_exact_sum():
    rng = np.random.default_rng(40)
    x = random_bf16_bits(rng, (64, 64), scale=3.0)
    r = random_bf16_bits(rng, (64, 64), scale=0.01)
    h, _ = add_rmsnorm_fwd(x, r, f32_to_bf16_bits(np.ones(64, np.float32)), 1e-6)
    exact = [a + b for a, b in zip(_vals(x), _vals(r))]
    assert [int(v) for v in h.reshape(-1)] == [round_exact_to_bf16(v) for v in exact]
    # and agrees with torch's bf16 add (computed in fp32, rounded once)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
    assert np.array_equal(h, (tx + tr).view(torch.int16).numpy().view(np.uint16))


def test_add_rmsnorm_brute_force_4x8():
    rng = np.random.default_rng(41)
    for _ in range(20):
        x = random_bf16_bits(rng, (4, 8))
        r = random_bf16_bits(rng, (4, 8))
        w = random_bf16_bits(rng, (8,), lo=0.5, hi=1.5)
        h, y = add_rmsnorm_fwd(x, r, w, 1e-6)
        for i in range(4):
            hv = [bf16_fields_value(round_exact_to_bf16(a + b)) for a, b in zip(_vals(x[i]), _vals(r[i]))]
            _check_exact(y[i], exact_rmsnorm_row(hv, _vals(w), _eps32(1e-6)))


def test_add_rmsnorm_special_cases():
    rng = np.random.default_rng(42)
    x = random_bf16_bits(rng, (8, 256))
    w = random_bf16_bits(rng, (256,), lo=0.5, hi=1.5)
    zero = np.zeros_like(x)
    h, y = add_rmsnorm_fwd(x, zero, w, 1e-6)
    assert np.array_equal(h, x) and np.array_equal(y, rmsnorm_fwd(x, w, 1e-6))
    h, y = add_rmsnorm_fwd(x, x ^ np.uint16(0x8000), w, 1e-6)  # x + (-x) = 0
    assert np.all(bf16_bits_to_f64(h) == 0) and np.all(bf16_bits_to_f64(y) == 0)
    h1, y1 = add_rmsnorm_fwd(x, zero + 0x3F80, w, 1e-6)
    h2, y2 = add_rmsnorm_fwd(zero + 0x3F80, x, w, 1e-6)  # the add commutes
    assert np.array_equal(h1, h2) and np.array_equal(y1, y2)


# ---------------- LayerNorm ----------------

def test_layernorm_brute_force_4x8():
    rng = np.random.default_rng(43)
    for eps in (1e-5, 0.25):
        for _ in range(15):
            x = random_bf16_bits(rng, (4, 8), scale=float(rng.choice([0.1, 1.0, 20.0])))
            w = random_bf16_bits(rng, (8,), lo=0.5, hi=1.5)
            b = random_bf16_bits(rng, (8,), lo=-0.5, hi=0.5)
            y = layernorm_fwd(x, w, b, eps)
            for i in range(4):
                _check_exact(y[i], exact_layernorm_row(_vals(x[i]), _vals(w), _vals(b), _eps32(eps)))


def test_layernorm_constant_row_gives_bias():
    rng = np.random.default_rng(44)
    w = random_bf16_bits(rng, (64,), lo=0.5, hi=1.5)
    b = random_bf16_bits(rng, (64,), lo=-0.5, hi=0.5)
    x = np.full((3, 64), f32_to_bf16_bits(np.float32([2.5]))[0], dtype=np.uint16)
    assert np.array_equal(layernorm_fwd(x, w, b, 1e-5), np.tile(b, (3, 1)))
    # N = 1: x - mean = 0, so y = b
    assert np.array_equal(layernorm_fwd(x[:, :1], w[:1], b[:1], 1e-5)[:, 0], np.full(3, b[0]))


def test_layernorm_zero_mean_unit_variance():
    rng = np.random.default_rng(45)
    x = random_bf16_bits(rng, (32, 1000), scale=4.0)
    one = f32_to_bf16_bits(np.ones(1000, np.float32))
    zero = np.zeros(1000, np.uint16)
    y = layernorm_fwd_f64(x, one, zero, 0.0)
    assert np.max(np.abs(y.mean(axis=1))) < 1e-14
    assert np.max(np.abs(y.var(axis=1) - 1.0)) < 1e-13


def test_layernorm_shift_and_scale_invariance():
    rng = np.random.default_rng(46)
    xi = rng.integers(-100, 100, size=(16, 128)).astype(np.float32)
    x = f32_to_bf16_bits(xi)
    xs = f32_to_bf16_bits(xi + np.float32(64.0))  # exact in bf16 (|values| <= 164 < 256)
    w = random_bf16_bits(rng, (128,), lo=0.5, hi=1.5)
    b = random_bf16_bits(rng, (128,), lo=-0.5, hi=0.5)
    assert np.count_nonzero(layernorm_fwd(x, w, b, 0.0) != layernorm_fwd(xs, w, b, 0.0)) <= 2
    x4 = f32_to_bf16_bits(xi * np.float32(4.0))
    assert np.array_equal(layernorm_fwd(x4, w, b, 0.0), layernorm_fwd(x, w, b, 0.0))


def test_layernorm_weight_and_bias_roles():
    rng = np.random.default_rng(47)
    x = random_bf16_bits(rng, (8, 96))
    w = random_bf16_bits(rng, (96,), lo=0.5, hi=1.5)
    zero = np.zeros(96, np.uint16)
    one = f32_to_bf16_bits(np.ones(96, np.float32))
    base = layernorm_fwd_f64(x, one, zero, 1e-5)
    assert np.allclose(layernorm_fwd_f64(x, w, zero, 1e-5), base * bf16_bits_to_f64(w), rtol=1e-15, atol=0)
    assert np.allclose(layernorm_fwd_f64(x, one, one, 1e-5), base + 1.0, rtol=0, atol=1e-15)
    neg = layernorm_fwd(x ^ np.uint16(0x8000), w, zero, 1e-5)
    assert np.array_equal(neg, layernorm_fwd(x, w, zero, 1e-5) ^ np.uint16(0x8000))


def test_layernorm_special_rows():
    w = f32_to_bf16_bits(np.ones(16, np.float32))
    b = f32_to_bf16_bits(np.full(16, 0.25, np.float32))
    x = np.zeros((3, 16), np.uint16)
    x[1, 3] = 0x7FC0
    x[2, 4] = 0x7F80
    y = bf16_bits_to_f64(layernorm_fwd(x, w, b, 1e-5))
    assert np.all(y[0] == 0.25)  # zero row: (0 - 0) * rstd + b
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))


# ---------------- L2Norm ----------------

def test_l2norm_brute_force():
    rng = np.random.default_rng(48)
    for _ in range(25):
        x = random_bf16_bits(rng, (4, 8), scale=float(rng.choice([1e-3, 1.0, 50.0])))
        y = l2norm_fwd(x, 1e-12)
        for i in range(4):
            _check_exact(y[i], exact_l2norm_row(_vals(x[i]), _eps32(1e-12)))


def test_l2norm_unit_norm_and_scale_invariance():
    rng = np.random.default_rng(49)
    x = random_bf16_bits(rng, (32, 512), scale=7.0)
    y = l2norm_fwd_f64(x, 1e-12)
    assert np.max(np.abs(np.linalg.norm(y, axis=1) - 1)) < 1e-14
    x8 = f32_to_bf16_bits(bf16_bits_to_f64(x).astype(np.float32) * np.float32(8.0))
    assert np.array_equal(l2norm_fwd(x8, 1e-12), l2norm_fwd(x, 1e-12))


def test_l2norm_eps_guard_and_one_hot():
    x = np.zeros((3, 8), np.uint16)
    x[1, 2] = f32_to_bf16_bits(np.float32([-3.0]))[0]
    x[2, :] = f32_to_bf16_bits(np.full(8, 1e-3, np.float32))
    y = bf16_bits_to_f64(l2norm_fwd(x, 0.5))
    assert np.all(y[0] == 0.0)  # zero row: 0 / eps
    assert y[1, 2] == -1.0 and np.count_nonzero(y[1]) == 1
    xv = bf16_bits_to_f64(x[2])
    assert np.array_equal(l2norm_fwd(x[2:], 0.5)[0], f32_to_bf16_bits((xv / 0.5).astype(np.float32)))  # ||x|| < eps
