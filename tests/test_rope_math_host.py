"""CPU tests of the QK kernel's rotary-angle arithmetic (csrc/rope_math.h),
built for the host (tests/c_abi/librope_math_host.so): the Cody-Waite + Taylor
sine / cosine and the inverse frequencies theta^(-2i/R) formed from six
host-evaluated powers, against 60-digit values from mpmath.

Bounds pinned here: |sin - exact|, |cos - exact| <= 1.5e-16 for every angle
tried (0.68 ulp of 1; the measured worst is 1.33e-16), on both sides of the
|phi| = 2^40 switch to the library routine; inverse frequencies within 5e-16
relative (measured worst 3.3e-16), far inside the 1e-15 the angle-precision
reading of the rotary embedding ("[pretuned] Optimize fused_qk_norm_rope on
B200", Summary: the angles and sin / cos are fp64) relies on.
"""

import ctypes
import os
import zlib

import numpy as np
import pytest

mpmath = pytest.importorskip("mpmath")

from memory_bound_normalization_amd import build as mbn_build  # noqa: E402

SIN_COS_ABS = 1.5e-16
INV_FREQ_REL = 5e-16


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mbn_build.ROPE_HOST_LIB):
        mbn_build.build_rope_host()
    h = ctypes.CDLL(mbn_build.ROPE_HOST_LIB)
    h.mbn_test_sincos.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    h.mbn_test_sincos.restype = None
    h.mbn_test_inv_freq.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    h.mbn_test_inv_freq.restype = None
    return h


def _sincos(lib, phi):
    phi = np.ascontiguousarray(phi, dtype=np.float64)
    s, c = np.empty_like(phi), np.empty_like(phi)
    lib.mbn_test_sincos(phi.ctypes.data, s.ctypes.data, c.ctypes.data, phi.size)
    return s, c


def _max_abs_err(phi, s, c):
    mpmath.mp.dps = 60
    es = ec = 0.0
    for p, sv, cv in zip(phi.tolist(), s.tolist(), c.tolist()):
        x = mpmath.mpf(p)
        es = max(es, abs(float(mpmath.sin(x) - mpmath.mpf(sv))))
        ec = max(ec, abs(float(mpmath.cos(x) - mpmath.mpf(cv))))
    return es, ec


def _near_multiples_of_half_pi(rng, n, kmax):
    """fp64 nearest to k * pi/2 (exactly rounded), and its two neighbours."""
    mpmath.mp.dps = 60
    k = rng.integers(-kmax, kmax, n)
    base = np.array([float(mpmath.mpf(int(v)) * mpmath.pi / 2) for v in k])
    return np.concatenate([base, np.nextafter(base, np.inf), np.nextafter(base, -np.inf)])


CASES = {
    "uniform in [-1e9, 1e9]": lambda rng: rng.uniform(-1e9, 1e9, 2000),
    "uniform in [-4, 4]": lambda rng: rng.uniform(-4.0, 4.0, 2000),
    "negative angles to -1e6": lambda rng: -rng.uniform(0.0, 1e6, 1000),
    "near multiples of pi/2 (|k| < 2^28)": lambda rng: _near_multiples_of_half_pi(rng, 600, 1 << 28),
    "near multiples of pi/2 (|k| < 64)": lambda rng: _near_multiples_of_half_pi(rng, 200, 64),
    # the quadrant decision: odd multiples of pi/4, where rint(phi * 2/pi) flips
    "near odd multiples of pi/4": lambda rng: _near_multiples_of_half_pi(rng, 300, 1 << 20) + np.pi / 4,
    "tiny and zero": lambda rng: np.array([0.0, -0.0, 1e-300, -1e-300, 5e-324, 1e-8, -3e-5, 2.0**-30]),
    # the switch to the library's sincos at |phi| = 2^40
    "across the 2^40 switch": lambda rng: np.array([2.0**40 * (1 - 2.0**-52), 2.0**40, -2.0**40,
                                                     -(2.0**40) * (1 - 2.0**-52), 2.0**40 + 1.0, 2.0**41,
                                                     1e13, -3e15, 2.0**39 * 1.999, 2.0**39]),
    # the workload's angles: positions 0 ... 1.23e8 times theta^(-2i/128), theta = 1e6
    "rotary angles, theta 1e6": lambda rng: np.array([p * 1e6 ** (-2.0 * i / 128) for p in
                                                      (1.0, 255.0, 4095.0, 1e6, 1.23e8) for i in range(0, 64, 3)]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_sincos_against_60_digits(lib, name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    phi = CASES[name](rng)
    s, c = _sincos(lib, phi)
    es, ec = _max_abs_err(phi, s, c)
    assert es <= SIN_COS_ABS and ec <= SIN_COS_ABS, (name, es, ec)


def test_sincos_symmetries(lib):
    """sin is odd and cos even in this routine as well (the reduction is
    symmetric: rint ties and the three-part pi/2 are sign-independent)."""
    phi = np.random.default_rng(3).uniform(0.0, 1e7, 2000)
    s1, c1 = _sincos(lib, phi)
    s2, c2 = _sincos(lib, -phi)
    assert np.array_equal(s1, -s2) and np.array_equal(c1, c2)


@pytest.mark.parametrize("theta", [2.0, 1e4, 5e5, 1e6])
def test_inverse_frequencies(lib, theta):
    """theta^(-2i/R) for every pair i < R/2, R = 16 ... 128 (the partial and
    full rotary dimensions the kernel takes), within 5e-16 relative."""
    mpmath.mp.dps = 60
    worst = 0.0
    for R in range(16, 129, 16):
        out = np.empty(R // 2)
        lib.mbn_test_inv_freq(theta, R, out.ctypes.data)
        assert out[0] == 1.0
        for i in range(R // 2):
            exact = mpmath.mpf(theta) ** (mpmath.mpf(-2 * i) / R)
            worst = max(worst, abs(float((mpmath.mpf(float(out[i])) - exact) / exact)))
    assert worst <= INV_FREQ_REL, (theta, worst)
