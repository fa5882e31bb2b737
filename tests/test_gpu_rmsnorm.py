"""GPU parity of rmsnorm_fwd (HIP, through the C ABI) against the fp64 oracle.

Small and ragged shapes are compared on every output; the full-size workloads
are compared on sampled rows (first, last, outlier and random rows, the oracle
computing only those rows) plus properties checked on every row.
"""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import rmsnorm_fwd as oracle_rmsnorm
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
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


def _sample_rows(M, rng, extra=()):
    rows = {0, 1, M // 2, M - 2, M - 1, *[int(r) for r in extra]}
    rows.update(int(r) for r in rng.choice(M, size=min(M, 192), replace=False))
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", list(RMS_WORKLOADS))
def test_workloads(name):
    wl = RMS_WORKLOADS[name]
    print(f"[rmsnorm] workload {name}", flush=True)
    x_bits, w_bits, eps = make_rms_inputs(wl)
    x = to_gpu_bf16(x_bits)
    w = to_gpu_bf16(w_bits)
    y = mbn.rmsnorm_fwd(x, w, eps=eps)
    y2 = mbn.rmsnorm_fwd(x, w, eps=eps)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not deterministic"
    rng = np.random.default_rng(123)
    rows = _sample_rows(wl.M, rng, extra=outlier_rows(wl))
    got = from_gpu_bf16(y[torch.from_numpy(rows).cuda()])
    assert_parity(got, oracle_rmsnorm(x_bits[rows], w_bits, eps), name)
    # every row: finite output, and with w in [0.5, 1.5] the row RMS of y/w is 1
    yf = y.float()
    assert torch.isfinite(yf).all()
    rms = torch.sqrt(torch.mean((yf / w.float()) ** 2, dim=1))
    assert torch.all(torch.abs(rms - 1) < 2e-3), float(torch.max(torch.abs(rms - 1)))
    # in place on the full workload matches
    mbn.rmsnorm_fwd(x, w, x, eps=eps)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16)), "in place differs"


def test_many_rows_sampled():
    """262144 rows (grids far beyond 65535 workgroups): sampled rows against the oracle."""
    M, N = 262144, 2048
    print(f"[rmsnorm] large M={M} N={N}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    x = (torch.randn(M, N, device="cuda", generator=g) * 2).to(torch.bfloat16)
    w = (torch.rand(N, device="cuda", generator=g) + 0.5).to(torch.bfloat16)
    y = mbn.rmsnorm_fwd(x, w, eps=1e-6)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 4095, 65535, 65536, 131071, 200000, M - 2, M - 1], device="cuda")
    xb, wb = from_gpu_bf16(x[rows]), from_gpu_bf16(w)
    assert_parity(from_gpu_bf16(y[rows]), oracle_rmsnorm(xb, wb, 1e-6), "large M")
    assert torch.isfinite(y.float()).all()
