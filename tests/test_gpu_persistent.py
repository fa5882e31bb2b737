"""GPU parity of the persistent row-norm kernel against the fp64 oracle.

For RMSNorm, LayerNorm and L2Norm with 2048 < N <= 8192 the launcher runs, at
the row counts its tables name, a persistent grid of 1024 to 2048 workgroups,
each looping over rows with two LDS buffers (the next row's copy in flight
while the current one is normalized). The row counts below are read from the
tables: the top of every row window (workgroups loop up to eight times, the
last iteration on a partial set of workgroups), both edges of every window
(one-shot kernel just outside), a small launch, at both edges of each width
band, ragged widths and both storage types. Every output is compared.
"""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import l2norm_fwd as o_l2, layernorm_fwd as o_ln, rmsnorm_fwd as o_rms
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from tables import persistent_windows
from workloads import f32_to_bf16_bits, random_bf16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# band edges (2056: 257 chunks, 3072, 3080, 4096, 4104, 6144, 6152, 8192) and
# ragged widths inside
WIDTHS = [2056, 3000, 3072, 3080, 4096, 4104, 6144, 6152, 8184, 8192]


def _rows(op, N):
    # a small launch, and the top of each row window of this width (several
    # loops per workgroup where it exceeds the grid, ragged last loop)
    return [200] + [hi for _, _, hi in persistent_windows(op, N // 8)]


def _edges(op, N):
    rows = set()
    for _, lo, hi in persistent_windows(op, N // 8):
        rows |= {m for m in (lo - 1, lo, hi, hi + 1) if m >= 1}
    return sorted(rows)


def _inputs(M, N, seed, dtype):
    rng = np.random.default_rng(seed)
    if dtype == "f16":
        x = rng.standard_normal((M, N)).astype(np.float16).view(np.uint16)
        w = rng.uniform(0.5, 1.5, N).astype(np.float16).view(np.uint16)
        b = rng.uniform(-0.5, 0.5, N).astype(np.float16).view(np.uint16)
    else:
        x = random_bf16_bits(rng, (M, N))
        w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
        b = random_bf16_bits(rng, (N,), lo=-0.5, hi=0.5)
    return x, w, b


def _run(op, x, w, b, eps, dtype):
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    xg = to_gpu_bf16(x, dtype=dtype)
    wg = to_gpu_bf16(w, dtype=dtype)
    bg = to_gpu_bf16(b, dtype=dtype)
    assert xg.dtype == tdt
    if op == "rms":
        y = mbn.rmsnorm_fwd(xg, wg, eps=eps)
    elif op == "layer":
        y = mbn.layernorm_fwd(xg, wg, bg, eps=eps)
    else:
        y = mbn.l2norm_fwd(xg, eps=eps)
    torch.cuda.synchronize()
    return from_gpu_bf16(y)


def _oracle(op, x, w, b, eps, dtype):
    if op == "rms":
        return o_rms(x, w, eps, dtype=dtype)
    if op == "layer":
        return o_ln(x, w, b, eps, dtype=dtype)
    return o_l2(x, eps, dtype=dtype)


@pytest.mark.parametrize("op", ["rms", "layer", "l2"])
@pytest.mark.parametrize("N", WIDTHS)
def test_persistent_widths(op, N):
    for M in _rows(op, N):
        print(f"[persistent {op}] M={M} N={N}", flush=True)
        x, w, b = _inputs(M, N, seed=M + N, dtype="bf16")
        assert_parity(_run(op, x, w, b, 1e-6, "bf16"), _oracle(op, x, w, b, 1e-6, "bf16"), f"{op} M={M} N={N}")


@pytest.mark.parametrize("op", ["rms", "layer", "l2"])
@pytest.mark.parametrize("N", [3000, 6144])
def test_persistent_f16(op, N):
    M = max([200] + [hi for _, _, hi in persistent_windows(op, N // 8)])
    print(f"[persistent {op} f16] M={M} N={N}", flush=True)
    x, w, b = _inputs(M, N, seed=N, dtype="f16")
    assert_parity(_run(op, x, w, b, 1e-5, "f16"), _oracle(op, x, w, b, 1e-5, "f16"), f"{op} f16 M={M} N={N}",
                  dtype="f16")


@pytest.mark.parametrize("op", ["rms", "layer", "l2"])
@pytest.mark.parametrize("N", [3072, 4096, 6144, 8192])
def test_row_window_edges(op, N):
    """Either side of each row window of the persistent tables (persistent
    inside, one-shot outside), at the top width of each band."""
    for M in _edges(op, N):
        print(f"[persistent {op} edge] M={M} N={N}", flush=True)
        x, w, b = _inputs(M, N, seed=M, dtype="bf16")
        assert_parity(_run(op, x, w, b, 1e-6, "bf16"), _oracle(op, x, w, b, 1e-6, "bf16"), f"{op} M={M} N={N}")


def test_every_band_has_a_window():
    """The tables above still reach the persistent kernel in every band the
    tests name (so the parity cases exercise it)."""
    for op, widths in (("rms", (3072, 4096, 6144, 8192)), ("layer", (3072, 4096, 6144, 8192)), ("l2", (3072, 6144))):
        for N in widths:
            assert persistent_windows(op, N // 8), (op, N)


def test_special_rows_between_normal_ones():
    """NaN, infinite and zero rows inside a persistent loop leave the other
    rows untouched (per-row partials do not leak across iterations)."""
    M, N = 4096, 4096
    rng = np.random.default_rng(9)
    x = random_bf16_bits(rng, (M, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    b = random_bf16_bits(rng, (N,), lo=-0.5, hi=0.5)
    x[5, 17] = 0x7FC0
    x[1029, :] = 0
    x[2048, 100] = 0x7F80
    # large but inside the float32 range of the sum of squares (|x| < ~1.8e19)
    x[4095, :] = f32_to_bf16_bits(np.full(N, 1e15, dtype=np.float32))
    for op in ("rms", "layer", "l2"):
        print(f"[persistent special {op}] M={M} N={N}", flush=True)
        assert_parity(_run(op, x, w, b, 1e-6, "bf16"), _oracle(op, x, w, b, 1e-6, "bf16"), f"special {op}")
