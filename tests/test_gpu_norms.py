"""GPU parity of add_rmsnorm_fwd, layernorm_fwd and l2norm_fwd (HIP, through
the C ABI) against the fp64 oracle; every output compared, on small and ragged
shapes and on the full-size workload shapes."""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import add_rmsnorm_fwd as o_add, l2norm_fwd as o_l2, layernorm_fwd as o_ln
from parity import assert_parity, assert_parity_rows, from_gpu_bf16, to_gpu_bf16
from workloads import RMS_WORKLOADS, f32_to_bf16_bits, make_norm_family_inputs, random_bf16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

WIDTHS = [8, 24, 512, 520, 1024, 2056, 4096, 4104, 8192, 8200, 16384, 16392, 32768, 32776, 65536]


def _inputs(M, N, seed, scale=1.0, shift=0.0):
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32) * np.float32(scale) + np.float32(shift))
    r = random_bf16_bits(rng, (M, N), scale=scale)
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    b = random_bf16_bits(rng, (N,), lo=-0.5, hi=0.5)
    return x, r, w, b


def _add(x, r, w, eps, alias=None):
    xg, rg, wg = to_gpu_bf16(x), to_gpu_bf16(r), to_gpu_bf16(w)
    h = rg if alias in ("h=r",) else (xg if alias == "h=x" else None)
    y = xg if alias in ("h=r",) else (rg if alias == "h=x" else None)
    h, y = mbn.add_rmsnorm_fwd(xg, rg, wg, h=h, y=y, eps=eps)
    torch.cuda.synchronize()
    return from_gpu_bf16(h), from_gpu_bf16(y)


def _assert_h_exact(h, rh, what):
    """h = bf16(x + r) is one rounding of a sum: bit-exact, NaN positions equal."""
    nan_g = (h & 0x7FFF) > 0x7F80
    nan_r = (rh & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions of h differ"
    assert np.array_equal(h[~nan_g], rh[~nan_r]), f"{what}: h = bf16(x + r) not bit-exact"


def _check_add(x, r, w, eps, what, alias=None):
    h, y = _add(x, r, w, eps, alias)
    rh, ry = o_add(x, r, w, eps)
    _assert_h_exact(h, rh, what)
    assert_parity(y, ry, what)


@pytest.mark.parametrize("N", WIDTHS)
def test_add_rmsnorm_widths(N):
    M = 23 if N <= 16392 else 5
    print(f"[add_rmsnorm] M={M} N={N}", flush=True)
    x, r, w, _ = _inputs(M, N, N)
    _check_add(x, r, w, 1e-6, f"add M={M} N={N}")


@pytest.mark.parametrize("alias", ["h=r", "h=x"])
def test_add_rmsnorm_in_place(alias):
    x, r, w, _ = _inputs(37, 16384, 5)
    _check_add(x, r, w, 1e-6, f"add {alias}", alias=alias)


def test_add_rmsnorm_special():
    x, r, w, _ = _inputs(5, 4096, 6)
    r[0] = x[0] ^ np.uint16(0x8000)  # h = 0
    x[1, 3] = 0x7FC0
    r[2, 9] = 0x7F80
    x[3, 9] = 0xFF80
    r[3, 9] = 0x7F80  # inf + -inf = NaN
    _check_add(x, r, w, 1e-6, "add special")


@pytest.mark.parametrize("N", WIDTHS)
def test_layernorm_widths(N):
    M = 23 if N <= 16392 else 5
    print(f"[layernorm] M={M} N={N}", flush=True)
    x, _, w, b = _inputs(M, N, N + 1)
    xg = to_gpu_bf16(x)
    y = mbn.layernorm_fwd(xg, to_gpu_bf16(w), to_gpu_bf16(b), eps=1e-5)
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), o_ln(x, w, b, 1e-5), f"layernorm N={N}")


@pytest.mark.parametrize("scale,shift", [(1.0, 0.0), (0.01, 0.0), (1.0, 100.0), (30.0, -5.0)])
def test_layernorm_scale_and_offset(scale, shift):
    x, _, w, b = _inputs(19, 8192, 7, scale=scale, shift=shift)
    for eps in (1e-5, 0.0):
        y = mbn.layernorm_fwd(to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(b), eps=eps)
        torch.cuda.synchronize()
        assert_parity(from_gpu_bf16(y), o_ln(x, w, b, eps), f"layernorm scale={scale} shift={shift} eps={eps}")


def test_layernorm_special_and_in_place():
    x, _, w, b = _inputs(6, 2048, 8)
    x[0] = f32_to_bf16_bits(np.full(2048, 3.0, np.float32))  # constant row -> b
    x[1, 5] = 0x7FC0
    x[2, 6] = 0x7F80
    xg = to_gpu_bf16(x)
    ref = o_ln(x, w, b, 1e-5)
    y = mbn.layernorm_fwd(xg, to_gpu_bf16(w), to_gpu_bf16(b), eps=1e-5)
    mbn.layernorm_fwd(xg, to_gpu_bf16(w), to_gpu_bf16(b), y=xg, eps=1e-5)
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), ref, "layernorm special")
    assert np.array_equal(from_gpu_bf16(xg), from_gpu_bf16(y)), "in place differs"


@pytest.mark.parametrize("N", WIDTHS)
def test_l2norm_widths(N):
    M = 23 if N <= 16392 else 5
    print(f"[l2norm] M={M} N={N}", flush=True)
    x, _, _, _ = _inputs(M, N, N + 2)
    y = mbn.l2norm_fwd(to_gpu_bf16(x), eps=1e-12)
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), o_l2(x, 1e-12), f"l2norm N={N}")


def test_l2norm_eps_and_special():
    x, _, _, _ = _inputs(8, 1024, 9, scale=1e-4)
    x[0] = 0
    x[1, 3] = 0x7FC0
    x[2, 4] = 0x7F80
    for eps in (1e-12, 0.5):
        xg = to_gpu_bf16(x)
        y = mbn.l2norm_fwd(xg, eps=eps)
        mbn.l2norm_fwd(xg, y=xg, eps=eps)
        torch.cuda.synchronize()
        assert_parity(from_gpu_bf16(y), o_l2(x, eps), f"l2norm eps={eps}")
        assert np.array_equal(from_gpu_bf16(xg), from_gpu_bf16(y))


@pytest.mark.parametrize("name", list(RMS_WORKLOADS))
def test_family_workloads(name):
    """Every output of the residual add + RMSNorm (h bit-exact, y within
    tolerance), LayerNorm and L2Norm on the full-size workload shapes (the
    oracle run in row blocks on host threads)."""
    wl = RMS_WORKLOADS[name]
    print(f"[norm family] workload {name}", flush=True)
    x, w, r, b, eps = make_norm_family_inputs(wl)
    xg, wg, rg, bg = to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(r), to_gpu_bf16(b)
    h, y = mbn.add_rmsnorm_fwd(xg, rg, wg, eps=eps)
    torch.cuda.synchronize()
    hb, yb = from_gpu_bf16(h), from_gpu_bf16(y)
    del h, y

    def add_block(lo, hi):
        rh, ry = o_add(x[lo:hi], r[lo:hi], w, eps)
        _assert_h_exact(hb[lo:hi], rh, f"add {name} rows [{lo}, {hi})")
        return ry

    assert assert_parity_rows(yb, add_block, f"add {name}") == wl.M * wl.N
    del hb, yb, rg
    y = mbn.layernorm_fwd(xg, wg, bg, eps=eps)
    torch.cuda.synchronize()
    assert_parity_rows(from_gpu_bf16(y), lambda lo, hi: o_ln(x[lo:hi], w, b, eps), f"layernorm {name}")
    y = mbn.l2norm_fwd(xg, y=y, eps=1e-12)
    torch.cuda.synchronize()
    assert_parity_rows(from_gpu_bf16(y), lambda lo, hi: o_l2(x[lo:hi], 1e-12), f"l2norm {name}")
