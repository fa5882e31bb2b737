"""Pins for the fused QK-norm + rotary oracle.

"[pretuned] Optimize fused_qk_norm_rope on B200" (Summary) fixes the dataflow:
full-head RMS, then the Q/K weights, then the rotary embedding of the two
halves, each half stored once. The rotary formula itself is not printed, so the
oracle is pinned to the textbook rotate-half rotation through properties a
rotation must have and through its matrix form.
"""

import math

import numpy as np
import pytest

from oracle import (
    bf16_bits_to_f64,
    qk_norm_rope_fwd,
    qk_norm_rope_fwd_f64,
    rmsnorm_fwd,
    rope_inv_freq,
    rope_rotate_neox,
)
from workloads import QK_WORKLOADS, f32_to_bf16_bits, make_qk_inputs, random_bf16_bits

D = 128


def _small_case(rng, t=8, hq=4, hk=2, d=D):
    qkv = random_bf16_bits(rng, (t, (hq + 2 * hk) * d))
    q_w = random_bf16_bits(rng, (d,), lo=0.5, hi=1.5)
    k_w = random_bf16_bits(rng, (d,), lo=0.5, hi=1.5)
    return qkv, q_w, k_w


def test_inverse_frequencies_closed_form():
    f = rope_inv_freq(D, 1e6)
    assert f[0] == 1.0
    assert abs(f[D // 4] - 1e-3) < 1e-18  # theta^(-1/2) = 1e-3
    r = f[1:] / f[:-1]
    assert np.allclose(r, 1e6 ** (-2.0 / D), rtol=1e-13, atol=0)
    assert abs(f[-1] / 1e6 ** (-(D - 2) / D) - 1) < 1e-14


def test_two_dimensional_textbook_rotation():
    """P12: D = 2 has one pair with inverse frequency 1: a plain 2-D rotation."""
    for a, b, p in [(1.0, 0.0, 1.0), (0.0, 1.0, 1.0), (0.3, -2.0, 5.0), (1.0, 0.0, math.pi / 2)]:
        o = rope_rotate_neox(np.array([a, b]), p, 1e6)
        assert abs(o[0] - (a * math.cos(p) - b * math.sin(p))) < 1e-15
        assert abs(o[1] - (b * math.cos(p) + a * math.sin(p))) < 1e-15
    # counter-clockwise by pi/2 maps (1, 0) to (0, 1)
    o = rope_rotate_neox(np.array([1.0, 0.0]), math.pi / 2, 1e6)
    assert abs(o[0]) < 1e-15 and abs(o[1] - 1.0) < 1e-15


def test_pairing_is_rotate_half():
    """A unit vector e_i (i < D/2) only reaches i and i + D/2."""
    f = rope_inv_freq(D, 1e6)
    p = 37.0
    for i in [0, 1, 5, 31, 63]:
        e = np.zeros(D)
        e[i] = 1.0
        o = rope_rotate_neox(e, p, 1e6)
        nz = set(np.nonzero(np.abs(o) > 1e-300)[0].tolist())
        assert nz <= {i, i + D // 2}
        assert abs(o[i] - math.cos(p * f[i])) < 1e-15
        assert abs(o[i + D // 2] - math.sin(p * f[i])) < 1e-15
        e2 = np.zeros(D)
        e2[i + D // 2] = 1.0
        o2 = rope_rotate_neox(e2, p, 1e6)
        assert abs(o2[i] + math.sin(p * f[i])) < 1e-15
        assert abs(o2[i + D // 2] - math.cos(p * f[i])) < 1e-15


def _rope_matrix(p, d, theta):
    """Block rotation matrix acting on the (i, i + d/2) planes."""
    h = d // 2
    r = np.zeros((d, d))
    for i in range(h):
        ang = p * math.pow(theta, -2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        r[i, i] = c
        r[i, i + h] = -s
        r[i + h, i] = s
        r[i + h, i + h] = c
    return r


def test_matches_matrix_form_and_is_orthogonal():
    rng = np.random.default_rng(20)
    u = rng.standard_normal((5, D))
    for p in [0.0, 1.0, 17.0, 255.0, 4096.0]:
        r = _rope_matrix(p, D, 1e6)
        assert np.allclose(r @ r.T, np.eye(D), atol=1e-14)
        # the two sides evaluate theta^(-2i/D) with different pow routines (1 ulp
        # apart), which moves the angle by about p * 1e-16
        assert np.allclose(rope_rotate_neox(u, p, 1e6), u @ r.T, rtol=0, atol=1e-13 * max(1.0, p / 64))


def test_rotation_preserves_pair_norms():
    """P9: o_i^2 + o_{i+D/2}^2 = u_i^2 + u_{i+D/2}^2."""
    rng = np.random.default_rng(21)
    u = rng.standard_normal((64, D))
    pos = rng.integers(0, 100000, size=64).astype(np.float64)
    o = rope_rotate_neox(u, pos, 1e6)
    h = D // 2
    assert np.allclose(o[:, :h] ** 2 + o[:, h:] ** 2, u[:, :h] ** 2 + u[:, h:] ** 2, rtol=1e-13, atol=1e-15)


def test_rotation_composition():
    """P10: R(p) R(q) = R(p + q)."""
    rng = np.random.default_rng(22)
    u = rng.standard_normal((16, D))
    for p, q in [(3, 4), (100, 155), (0, 9)]:
        a = rope_rotate_neox(rope_rotate_neox(u, q, 1e6), p, 1e6)
        b = rope_rotate_neox(u, p + q, 1e6)
        assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_relative_position_property():
    """P11: <R(m) a, R(n) b> depends only on m - n."""
    rng = np.random.default_rng(23)
    a = rng.standard_normal(D)
    b = rng.standard_normal(D)
    base = np.dot(rope_rotate_neox(a, 10, 1e6), rope_rotate_neox(b, 3, 1e6))
    for s in [1, 50, 200]:
        v = np.dot(rope_rotate_neox(a, 10 + s, 1e6), rope_rotate_neox(b, 3 + s, 1e6))
        assert abs(v - base) < 1e-11


def test_position_zero_reduces_to_per_head_rmsnorm():
    """P8: at position 0 the rotation is the identity: per-head RMSNorm."""
    rng = np.random.default_rng(24)
    t, hq, hk = 6, 4, 2
    qkv, q_w, k_w = _small_case(rng, t, hq, hk)
    pos = np.zeros(t, dtype=np.int64)
    out = qk_norm_rope_fwd(qkv, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6)
    heads = qkv[:, : (hq + hk) * D].reshape(t, hq + hk, D)
    ref_q = rmsnorm_fwd(heads[:, :hq].reshape(-1, D), q_w, 1e-6).reshape(t, hq * D)
    ref_k = rmsnorm_fwd(heads[:, hq:].reshape(-1, D), k_w, 1e-6).reshape(t, hk * D)
    assert np.array_equal(out[:, : hq * D], ref_q)
    assert np.array_equal(out[:, hq * D : (hq + hk) * D], ref_k)


def test_weights_go_to_their_heads():
    """q_w scales only q heads, k_w only k heads (power-of-two scaling is exact)."""
    rng = np.random.default_rng(25)
    t, hq, hk = 5, 3, 2
    qkv, _, _ = _small_case(rng, t, hq, hk)
    one = f32_to_bf16_bits(np.ones(D, dtype=np.float32))
    two = f32_to_bf16_bits(np.full(D, 2.0, dtype=np.float32))
    pos = np.arange(t, dtype=np.int64) * 11
    base = bf16_bits_to_f64(qk_norm_rope_fwd(qkv, one, one, pos, hq, hk, D, 1e-6, 1e6))
    kq = bf16_bits_to_f64(qk_norm_rope_fwd(qkv, one, two, pos, hq, hk, D, 1e-6, 1e6))
    qq = bf16_bits_to_f64(qk_norm_rope_fwd(qkv, two, one, pos, hq, hk, D, 1e-6, 1e6))
    nq, nk = hq * D, (hq + hk) * D
    assert np.array_equal(kq[:, :nq], base[:, :nq])
    assert np.array_equal(kq[:, nq:nk], 2 * base[:, nq:nk])
    assert np.array_equal(qq[:, :nq], 2 * base[:, :nq])
    assert np.array_equal(qq[:, nq:nk], base[:, nq:nk])


def test_unit_weights_unit_rms():
    """P9: with w = 1 and eps = 0 each output head has RMS 1 before rounding."""
    rng = np.random.default_rng(26)
    qkv, _, _ = _small_case(rng, 7, 4, 2)
    one = f32_to_bf16_bits(np.ones(D, dtype=np.float32))
    o = qk_norm_rope_fwd_f64(qkv, one, one, np.arange(7) * 31, 4, 2, D, 0.0, 1e6)
    assert np.max(np.abs(np.sqrt(np.mean(o * o, axis=-1)) - 1)) < 1e-14


def test_v_untouched_and_tokens_independent():
    """P13: v heads keep their bits; a token's output depends only on that token."""
    rng = np.random.default_rng(27)
    t, hq, hk = 9, 4, 2
    qkv, q_w, k_w = _small_case(rng, t, hq, hk)
    pos = np.arange(t, dtype=np.int64)
    out = qk_norm_rope_fwd(qkv, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6)
    nk = (hq + hk) * D
    assert np.array_equal(out[:, nk:], qkv[:, nk:])
    qkv2 = qkv.copy()
    qkv2[4] = random_bf16_bits(rng, (qkv.shape[1],))
    out2 = qk_norm_rope_fwd(qkv2, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6)
    same = np.arange(t) != 4
    assert np.array_equal(out2[same], out[same])
    assert not np.array_equal(out2[4, :nk], out[4, :nk])
    # a token's result depends on its own position only
    single = qk_norm_rope_fwd(qkv[5:6], q_w, k_w, pos[5:6], hq, hk, D, 1e-6, 1e6)
    assert np.array_equal(single[0], out[5])


def test_head_layout_brute_force_loop():
    """Pure-Python loop over tokens/heads/elements with the matrix form."""
    rng = np.random.default_rng(28)
    t, hq, hk, d = 3, 2, 1, 8
    qkv = random_bf16_bits(rng, (t, (hq + 2 * hk) * d))
    q_w = random_bf16_bits(rng, (d,), lo=0.5, hi=1.5)
    k_w = random_bf16_bits(rng, (d,), lo=0.5, hi=1.5)
    pos = np.array([0, 3, 200], dtype=np.int64)
    got = qk_norm_rope_fwd_f64(qkv, q_w, k_w, pos, hq, hk, d, 1e-6, 1e6)
    xv = bf16_bits_to_f64(qkv)
    qw = bf16_bits_to_f64(q_w)
    kw = bf16_bits_to_f64(k_w)
    eps = float(np.float32(1e-6))
    for ti in range(t):
        r = _rope_matrix(float(pos[ti]), d, 1e6)
        for h in range(hq + hk):
            seg = [xv[ti, h * d + j] for j in range(d)]
            ss = 0.0
            for v in seg:
                ss += v * v
            rstd = 1.0 / math.sqrt(ss / d + eps)
            w = qw if h < hq else kw
            u = np.array([seg[j] * rstd * w[j] for j in range(d)])
            ref = r @ u
            assert np.allclose(got[ti, h], ref, rtol=1e-13, atol=1e-15)


def test_workload_shape_and_runs():
    wl = QK_WORKLOADS["qk_256"]
    qkv, q_w, k_w, pos, eps, theta = make_qk_inputs(wl)
    assert qkv.shape == (256, 6144) and q_w.shape == (128,) and pos[-1] == 255
    out = qk_norm_rope_fwd(qkv, q_w, k_w, pos, 32, 8, 128, eps, theta)
    assert np.array_equal(out[:, 5120:], qkv[:, 5120:])
    assert np.all(np.isfinite(bf16_bits_to_f64(out)))


# ---------------- partial rotary ----------------

@pytest.mark.parametrize("rot", [16, 32, 64, 96])
def test_partial_rotary_tail_is_per_head_rmsnorm(rot):
    """The tail past rotary_dim is the plain weighted per-head RMSNorm."""
    rng = np.random.default_rng(60 + rot)
    t, hq, hk = 5, 3, 2
    qkv, q_w, k_w = _small_case(rng, t, hq, hk)
    pos = np.arange(t, dtype=np.int64) * 37 + 3
    out = qk_norm_rope_fwd(qkv, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6, rotary_dim=rot)
    heads = qkv[:, : (hq + hk) * D].reshape(t, hq + hk, D)
    oh = out[:, : (hq + hk) * D].reshape(t, hq + hk, D)
    ref_q = rmsnorm_fwd(heads[:, :hq].reshape(-1, D), q_w, 1e-6).reshape(t, hq, D)
    ref_k = rmsnorm_fwd(heads[:, hq:].reshape(-1, D), k_w, 1e-6).reshape(t, hk, D)
    assert np.array_equal(oh[:, :hq, rot:], ref_q[:, :, rot:])
    assert np.array_equal(oh[:, hq:, rot:], ref_k[:, :, rot:])
    # the rotary part differs from the plain norm (positions are not 0) ...
    assert not np.array_equal(oh[:, :hq, :rot], ref_q[:, :, :rot])
    # ... and preserves the norm of each rotated pair
    f = qk_norm_rope_fwd_f64(qkv, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6, rotary_dim=rot)
    u = qk_norm_rope_fwd_f64(qkv, q_w, k_w, np.zeros(t, np.int64), hq, hk, D, 1e-6, 1e6, rotary_dim=rot)
    h2 = rot // 2
    assert np.allclose(f[..., :h2] ** 2 + f[..., h2:rot] ** 2, u[..., :h2] ** 2 + u[..., h2:rot] ** 2,
                       rtol=1e-13, atol=1e-15)


def test_partial_rotary_uses_its_own_frequencies():
    """Pairing (i, i + R/2) with angle p * theta^(-2i/R), via the matrix form at D = R."""
    rng = np.random.default_rng(70)
    rot = 32
    qkv, q_w, k_w = _small_case(rng, 3, 1, 0)
    pos = np.array([0, 5, 211], dtype=np.int64)
    f = qk_norm_rope_fwd_f64(qkv, q_w, k_w, pos, 1, 0, D, 1e-6, 1e6, rotary_dim=rot)
    u = qk_norm_rope_fwd_f64(qkv, q_w, k_w, np.zeros(3, np.int64), 1, 0, D, 1e-6, 1e6, rotary_dim=rot)
    for ti in range(3):
        r = _rope_matrix(float(pos[ti]), rot, 1e6)
        assert np.allclose(f[ti, 0, :rot], r @ u[ti, 0, :rot], rtol=0, atol=1e-13)
        assert np.array_equal(f[ti, 0, rot:], u[ti, 0, rot:])


def test_full_rotary_dim_is_the_default():
    rng = np.random.default_rng(71)
    qkv, q_w, k_w = _small_case(rng, 4, 2, 1)
    pos = np.arange(4, dtype=np.int64) * 9
    a = qk_norm_rope_fwd(qkv, q_w, k_w, pos, 2, 1, D, 1e-6, 1e6)
    b = qk_norm_rope_fwd(qkv, q_w, k_w, pos, 2, 1, D, 1e-6, 1e6, rotary_dim=D)
    assert np.array_equal(a, b)
