"""GPU parity of the fp16 entry points (HIP, through the C ABI) against the
fp64 oracle evaluated on binary16 data; every output compared."""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import add_rmsnorm_fwd as o_add, l2norm_fwd as o_l2, layernorm_fwd as o_ln
from oracle import qk_norm_rope_fwd as o_qk, rmsnorm_fwd as o_rms
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
F16 = "f16"


def _bits(rng, shape, scale=1.0, lo=None, hi=None):
    v = lo + (hi - lo) * rng.random(shape) if lo is not None else rng.standard_normal(shape) * scale
    return v.astype(np.float16).view(np.uint16)


def up(bits):
    return to_gpu_bf16(bits, dtype=F16)


@pytest.mark.parametrize("N", [8, 520, 4096, 8200, 16384, 32768, 65536])
def test_rmsnorm_f16(N):
    print(f"[f16] rmsnorm N={N}", flush=True)
    rng = np.random.default_rng(N)
    M = 13 if N <= 16384 else 5
    x = _bits(rng, (M, N), scale=float(rng.choice([0.01, 1.0, 300.0])))
    w = _bits(rng, (N,), lo=0.5, hi=1.5)
    y = mbn.rmsnorm_fwd(up(x), up(w), eps=1e-6)
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    assert_parity(from_gpu_bf16(y), o_rms(x, w, 1e-6, dtype=F16), f"rmsnorm f16 N={N}", dtype=F16)


@pytest.mark.parametrize("N", [520, 8192, 16384])
def test_family_f16(N):
    print(f"[f16] family N={N}", flush=True)
    rng = np.random.default_rng(N + 1)
    M = 11
    x = _bits(rng, (M, N), scale=2.0)
    r = _bits(rng, (M, N), scale=2.0)
    w = _bits(rng, (N,), lo=0.5, hi=1.5)
    b = _bits(rng, (N,), lo=-0.5, hi=0.5)
    x[0, 3] = np.float16(60000.0).view(np.uint16)
    r[0, 3] = np.float16(30000.0).view(np.uint16)  # h overflows to inf in fp16
    h, y = mbn.add_rmsnorm_fwd(up(x), up(r), up(w), eps=1e-6)
    rh, ry = o_add(x, r, w, 1e-6, dtype=F16)
    torch.cuda.synchronize()
    assert np.array_equal(from_gpu_bf16(h), rh), "h = f16(x + r) not bit-exact"
    assert_parity(from_gpu_bf16(y), ry, f"add f16 N={N}", dtype=F16)
    y = mbn.layernorm_fwd(up(x[1:]), up(w), up(b), eps=1e-5)
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), o_ln(x[1:], w, b, 1e-5, dtype=F16), f"layernorm f16 N={N}", dtype=F16)
    y = mbn.l2norm_fwd(up(x), eps=1e-12)
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), o_l2(x, 1e-12, dtype=F16), f"l2norm f16 N={N}", dtype=F16)


@pytest.mark.parametrize("rot", [None, 64, 32])
def test_qk_f16(rot):
    print(f"[f16] qk rotary_dim={rot}", flush=True)
    rng = np.random.default_rng(7 if rot is None else rot)
    T, hq, hk, D = 300, 32, 8, 128
    qkv = _bits(rng, (T, (hq + 2 * hk) * D))
    q_w = _bits(rng, (D,), lo=0.5, hi=1.5)
    k_w = _bits(rng, (D,), lo=0.5, hi=1.5)
    pos = np.arange(T, dtype=np.int64) * 7
    g = up(qkv)
    mbn.qk_norm_rope_fwd(g, up(q_w), up(k_w), torch.from_numpy(pos).cuda(), hq, hk, D, eps=1e-6, theta=1e6,
                         rotary_dim=rot)
    torch.cuda.synchronize()
    got = from_gpu_bf16(g)
    ref = o_qk(qkv, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6, rotary_dim=rot, dtype=F16)
    assert np.array_equal(got[:, (hq + hk) * D:], qkv[:, (hq + hk) * D:])
    assert_parity(got, ref, f"qk f16 rot={rot}", dtype=F16)


def test_mixed_dtypes_are_rejected():
    x = torch.zeros(2, 64, dtype=torch.float16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        mbn.rmsnorm_fwd(x, w)
