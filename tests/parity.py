"""Helpers shared by the GPU parity tests: bit transfer and the tolerance check.

Tolerance (elementwise, on every compared output): with y_ref the oracle's
bf16 value widened to float64,

    |y_gpu - y_ref| <= 2^-7 * |y_ref| + 1e-6

i.e. one bf16 ulp relative plus an absolute floor for outputs near zero; for
fp16 data the relative term is one fp16 ulp, 2^-10 * |y_ref|. NaN positions
must match exactly; infinities must match exactly.
"""

from __future__ import annotations

import numpy as np

from oracle import bf16_bits_to_f64, widen

REL_TOL = 2.0**-7
REL_TOL_F16 = 2.0**-10
ABS_TOL = 1e-6


def to_gpu_bf16(bits: np.ndarray, device="cuda", dtype="bf16"):
    import torch

    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(device)


def from_gpu_bf16(t) -> np.ndarray:
    import torch

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def tolerance_violations(got_bits, ref_bits, dtype="bf16"):
    """Return a boolean mask of outputs outside the tolerance (NaN/inf aware)."""
    g = widen(got_bits, dtype)
    r = widen(ref_bits, dtype)
    rel = REL_TOL_F16 if dtype == "f16" else REL_TOL
    nan_r, nan_g = np.isnan(r), np.isnan(g)
    with np.errstate(invalid="ignore"):
        ok = (np.abs(g - r) <= rel * np.abs(r) + ABS_TOL) | (g == r)
    ok = np.where(nan_r | nan_g, nan_r & nan_g, ok)
    return ~ok


def assert_parity(got_bits, ref_bits, what: str = "", dtype="bf16"):
    got_bits = np.asarray(got_bits)
    ref_bits = np.asarray(ref_bits)
    assert got_bits.shape == ref_bits.shape, (got_bits.shape, ref_bits.shape)
    bad = tolerance_violations(got_bits, ref_bits, dtype)
    n = int(np.count_nonzero(bad))
    if n:
        idx = np.argwhere(bad)[:8]
        g = widen(got_bits, dtype)
        r = widen(ref_bits, dtype)
        rows = [f"  at {tuple(int(v) for v in i)}: gpu {g[tuple(i)]!r} oracle {r[tuple(i)]!r}" for i in idx]
        raise AssertionError(f"{what}: {n} of {bad.size} outputs outside tolerance\n" + "\n".join(rows))


def ulp_stats(got_bits, ref_bits) -> dict:
    """How far the GPU is from the oracle, in bf16 ulps of the oracle value (finite only)."""
    g = bf16_bits_to_f64(got_bits)
    r = bf16_bits_to_f64(ref_bits)
    fin = np.isfinite(r) & np.isfinite(g)
    same = int(np.count_nonzero((got_bits == ref_bits) & fin))
    return {"compared": int(fin.sum()), "bit_equal": same, "frac_bit_equal": same / max(1, int(fin.sum()))}


def host_threads() -> int:
    """Threads for host-side oracle work: the CPUs this process may use, at most 16."""
    import os

    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def assert_parity_rows(got_bits, ref_rows, what: str = "", dtype="bf16", block: int = 512):
    """Compare every row of ``got_bits`` [M, ...] with the oracle.

    ``ref_rows(lo, hi)`` returns the oracle's output bits for rows [lo, hi).
    The oracle runs in row blocks (bounded float64 temporaries) on host threads
    (NumPy releases the GIL inside its array operations); every block is checked
    with the same elementwise tolerance as assert_parity. Returns the number of
    outputs compared.
    """
    from concurrent.futures import ThreadPoolExecutor

    got_bits = np.asarray(got_bits)
    m = got_bits.shape[0]

    def one(lo):
        hi = min(m, lo + block)
        assert_parity(got_bits[lo:hi], ref_rows(lo, hi), f"{what} rows [{lo}, {hi})", dtype)
        return got_bits[lo:hi].size

    with ThreadPoolExecutor(host_threads()) as pool:
        return sum(pool.map(one, range(0, m, block)))
