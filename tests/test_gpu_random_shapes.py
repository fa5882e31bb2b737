"""Randomized GPU parity over the row norms: a fixed-seed draw of op (RMSNorm,
residual add + RMSNorm, LayerNorm, L2Norm), storage type (bf16, fp16), width
(any N up to 20000, biased to multiples of 8 and common model widths), row
count, and element offsets of every row tensor (views that start inside a
16-byte block, the same or different offsets per tensor), so that launch-table
selection and every kernel path (row windows, sub-bands, exact widths,
persistent, per-chunk waits, the 16-byte staged and element-group any-width
kernels) meet in combinations the targeted tests do not spell out. Every
output is compared against the fp64 oracle; h of the residual add bit for bit."""

import numpy as np
import pytest

from parity import assert_parity, from_gpu_bf16
from workloads import random_bf16_bits, random_f16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import memory_bound_normalization_amd as mbn  # noqa: E402
from oracle import add_rmsnorm_fwd as o_add, l2norm_fwd as o_l2, layernorm_fwd as o_ln, rmsnorm_fwd as o_rms  # noqa: E402

COMMON = [1024, 2048, 2560, 3072, 4096, 5120, 6144, 7168, 8192, 10240, 12288, 14336, 16384, 18432]


def _cases(n=160, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        op = ["rms", "add", "layer", "l2"][i % 4]
        dtype = "f16" if rng.random() < 0.3 else "bf16"
        kind = rng.random()
        if kind < 0.35:
            N = int(rng.choice(COMMON))
        elif kind < 0.7:
            N = 8 * int(rng.integers(1, 2500))
        else:
            N = int(rng.integers(1, 20000))
        M = int(rng.integers(1, max(2, min(3000, (8 << 20) // N))))
        if rng.random() < 0.25:
            M = int(rng.choice([1, 2, 3, 7, 255, 256, 257, 1023, 1024, 1025, 2048, 2049]))
            M = min(M, max(1, (8 << 20) // N))
        offs = [0, 0, 0, 0]
        r = rng.random()
        if r < 0.25:
            o = int(rng.integers(1, 8))
            offs = [o, o, o, o]  # every tensor at the same offset
        elif r < 0.4:
            offs = [int(v) for v in rng.integers(0, 8, 4)]
        out.append((i, op, dtype, M, N, tuple(offs)))
    return out


CASES = _cases()


def _view(bits, off, dtype):
    """A contiguous GPU tensor holding `bits` that starts `off` elements into
    a fresh allocation (so off % 8 != 0 is not 16-byte aligned)."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    flat = np.ascontiguousarray(bits).reshape(-1).view(np.int16)
    buf = torch.empty(flat.size + off + 8, dtype=torch.int16, device="cuda")
    buf[off:off + flat.size].copy_(torch.from_numpy(flat))
    return buf[off:off + flat.size].view(tdt).view(bits.shape)


def _empty_view(shape, off, dtype):
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    n = int(np.prod(shape))
    buf = torch.empty(n + off + 8, dtype=tdt, device="cuda")
    return buf[off:off + n].view(shape)


@pytest.mark.parametrize("i,op,dtype,M,N,offs", CASES)
def test_random_shape(i, op, dtype, M, N, offs):
    label = f"case {i}: {op} {dtype} M={M} N={N} offsets={offs}"
    print(f"[random] {label}", flush=True)
    rng = np.random.default_rng(1000 + i)
    gen = random_f16_bits if dtype == "f16" else random_bf16_bits
    x = gen(rng, (M, N), scale=float(rng.choice([0.05, 1.0, 20.0])))
    w = gen(rng, (N,), lo=0.5, hi=1.5)
    xo, ro, ho, yo = offs
    xg = _view(x, xo, dtype)
    y = _empty_view((M, N), yo, dtype)
    if op == "rms":
        mbn.rmsnorm_fwd(xg, _view(w, 0, dtype), y, eps=1e-6)
        ref = o_rms(x, w, 1e-6, dtype=dtype)
    elif op == "layer":
        b = gen(rng, (N,), lo=-0.5, hi=0.5)
        mbn.layernorm_fwd(xg, _view(w, 0, dtype), _view(b, 0, dtype), y, eps=1e-5)
        ref = o_ln(x, w, b, 1e-5, dtype=dtype)
    elif op == "l2":
        mbn.l2norm_fwd(xg, y, eps=1e-12)
        ref = o_l2(x, 1e-12, dtype=dtype)
    else:
        r = gen(rng, (M, N))
        h = _empty_view((M, N), ho, dtype)
        mbn.add_rmsnorm_fwd(xg, _view(r, ro, dtype), _view(w, 0, dtype), h=h, y=y, eps=1e-6)
        rh, ref = o_add(x, r, w, 1e-6, dtype=dtype)
        torch.cuda.synchronize()
        assert np.array_equal(from_gpu_bf16(h), rh), f"{label}: h not bit-exact"
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), ref, label, dtype=dtype)
