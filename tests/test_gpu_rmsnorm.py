"""GPU parity of rmsnorm_fwd (HIP, through the C ABI) against the fp64 oracle.

Every output is compared: small and ragged shapes, and the full-size
workloads (the oracle run in row blocks on host threads).
"""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import rmsnorm_fwd as oracle_rmsnorm
from parity import assert_parity, assert_parity_rows, from_gpu_bf16, to_gpu_bf16
from workloads import RMS_WORKLOADS, f32_to_bf16_bits, make_rms_inputs, outlier_rows, random_bf16_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(x_bits, w_bits, eps, inplace=False):
    x = to_gpu_bf16(x_bits)
    w = to_gpu_bf16(w_bits)
    y = mbn.rmsnorm_fwd(x, w, x if inplace else None, eps=eps)
    torch.cuda.synchronize()
    return from_gpu_bf16(y)


def _check(M, N, eps=1e-6, seed=0, scale=1.0):
    print(f"[rmsnorm] M={M} N={N} eps={eps} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    x = random_bf16_bits(rng, (M, N), scale=scale)
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    assert_parity(_run(x, w, eps), oracle_rmsnorm(x, w, eps), f"M={M} N={N}")


# every band of the launch table, its edges, and ragged widths inside it
WIDTHS = [8, 16, 24, 504, 512, 520, 1024, 1032, 2040, 2048, 2056, 4096, 4104, 6144, 8192, 8200,
          12288, 16384, 16392, 24576, 32768, 32776, 65528, 65536]


@pytest.mark.parametrize("N", WIDTHS)
def test_widths(N):
    M = 37 if N <= 16384 else 9  # not a multiple of the rows per workgroup
    _check(M, N, seed=N)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 65, 1023])
def test_row_counts(M):
    _check(M, 256, seed=M)
    _check(M, 4096, seed=M + 1)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-5, 0.5])
def test_eps(eps):
    _check(16, 2048, eps=eps, seed=3)


@pytest.mark.parametrize("scale", [1e-3, 30.0, 1e4])
def test_scales(scale):
    _check(16, 8192, seed=4, scale=scale)


def test_empty():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    assert mbn.rmsnorm_fwd(x, w).shape == (0, 64)


def test_special_rows():
    N = 4096
    rng = np.random.default_rng(5)
    x = random_bf16_bits(rng, (6, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    x[0] = 0  # zero row
    x[1, 100] = 0x7FC0  # NaN
    x[2, 7] = 0x7F80  # +inf
    x[3, 9] = 0xFF80  # -inf
    x[4] = f32_to_bf16_bits(np.full(N, -2.5, dtype=np.float32))  # constant row
    for eps in (1e-6, 0.0):
        assert_parity(_run(x, w, eps), oracle_rmsnorm(x, w, eps), f"special eps={eps}")


def test_in_place_equals_out_of_place_and_deterministic():
    rng = np.random.default_rng(6)
    for M, N in [(33, 4096), (17, 16384), (5, 32768), (64, 1000 * 8)]:
        x = random_bf16_bits(rng, (M, N))
        w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
        a = _run(x, w, 1e-6)
        b = _run(x, w, 1e-6)
        c = _run(x, w, 1e-6, inplace=True)
        assert np.array_equal(a, b), "not deterministic"
        assert np.array_equal(a, c), "in place differs"


def test_non_default_stream():
    rng = np.random.default_rng(7)
    x = random_bf16_bits(rng, (64, 8192))
    w = random_bf16_bits(rng, (8192,), lo=0.5, hi=1.5)
    s = torch.cuda.Stream()
    xg, wg = to_gpu_bf16(x), to_gpu_bf16(w)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = mbn.rmsnorm_fwd(xg, wg, eps=1e-6)
    s.synchronize()
    assert_parity(from_gpu_bf16(y), oracle_rmsnorm(x, w, 1e-6), "side stream")


def test_misaligned_pointer_takes_the_any_width_path():
    """x and y at a 2-byte offset (not 16-byte aligned): served element-wise,
    correct, and nothing outside the rows is written."""
    rng = np.random.default_rng(8)
    M, N = 4, 64
    x = random_bf16_bits(rng, (M, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    xb = torch.zeros(M * N + 8, dtype=torch.bfloat16, device="cuda")
    yb = torch.full((M * N + 8,), 7.0, dtype=torch.bfloat16, device="cuda")
    xb[1 : 1 + M * N] = to_gpu_bf16(x).view(-1)
    xv = xb[1 : 1 + M * N].view(M, N)
    yv = yb[3 : 3 + M * N].view(M, N)
    mbn.rmsnorm_fwd(xv, to_gpu_bf16(w), yv)
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(yv), oracle_rmsnorm(x, w, 1e-6), "misaligned x, y")
    guard = torch.cat([yb[:3], yb[3 + M * N :]])
    assert bool((guard == 7.0).all()), "wrote outside y"


@pytest.mark.parametrize("name", list(RMS_WORKLOADS))
def test_workloads(name):
    """Every output of the full-size workload against the oracle (row blocks on
    host threads), the launch run twice (bit-identical) and in place."""
    wl = RMS_WORKLOADS[name]
    print(f"[rmsnorm] workload {name}", flush=True)
    x_bits, w_bits, eps = make_rms_inputs(wl)
    x = to_gpu_bf16(x_bits)
    w = to_gpu_bf16(w_bits)
    y = mbn.rmsnorm_fwd(x, w, eps=eps)
    y2 = mbn.rmsnorm_fwd(x, w, eps=eps)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not deterministic"
    got = from_gpu_bf16(y)
    n = assert_parity_rows(got, lambda lo, hi: oracle_rmsnorm(x_bits[lo:hi], w_bits, eps), name)
    assert n == wl.M * wl.N
    # the outlier rows are among the compared rows; check they were drawn
    if wl.outlier_frac:
        assert len(outlier_rows(wl)) == int(wl.M * wl.outlier_frac)
    # in place on the full workload matches
    mbn.rmsnorm_fwd(x, w, x, eps=eps)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "in place differs"


def test_many_rows():
    """262144 rows (grids far beyond 65535 workgroups): every output against the oracle."""
    M, N = 262144, 2048
    print(f"[rmsnorm] large M={M} N={N}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    x = (torch.randn(M, N, device="cuda", generator=g) * 2).to(torch.bfloat16)
    w = (torch.rand(N, device="cuda", generator=g) + 0.5).to(torch.bfloat16)
    y = mbn.rmsnorm_fwd(x, w, eps=1e-6)
    torch.cuda.synchronize()
    xb, wb, yb = from_gpu_bf16(x), from_gpu_bf16(w), from_gpu_bf16(y)
    del x, y
    assert assert_parity_rows(yb, lambda lo, hi: oracle_rmsnorm(xb[lo:hi], wb, 1e-6), "large M",
                              block=4096) == M * N
