"""GPU parity of the launch-table entries with register-resident rows (the _R
entries: rownorm_regs_kernel, each lane's chunks of the row held in VGPRs
instead of LDS, exact widths only). Each is reached at its width with one
row, with a row count that is no multiple of anything in the kernel, and with
a few hundred rows, in both storage types, every output compared against the
fp64 oracle; at the 4096 x 32768 workload ten launches must give identical
bits, and the in-place call (y aliasing x) the same output."""

import numpy as np
import pytest

from tables import TABLES

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from norm_ops import TABLE_OPS, check_norm  # noqa: E402  (needs torch)

ENTRIES = [(TABLE_OPS[t], e) for t in TABLE_OPS for e in TABLES[t] if e.regs]
CASES = [(op, M, e.top * 8) for op, e in ENTRIES for M in (1, 37, 515)]


def test_register_entries_present():
    assert len(ENTRIES) >= 2 and all(e.exact and e.rpl == 1 for _, e in ENTRIES)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op,M,N", CASES)
def test_register_entry(op, M, N, dtype):
    print(f"[register rows {op} {dtype}] M={M} N={N}", flush=True)
    check_norm(op, M, N, M * 5 + N, f"{op} {dtype} M={M} N={N}", dtype=dtype)


def test_register_rows_repeat_and_in_place():
    M, N = 4096, 32768
    print(f"[register rows repeat] M={M} N={N}", flush=True)
    from oracle import rmsnorm_fwd as o_rms
    from parity import assert_parity_rows, from_gpu_bf16, to_gpu_bf16
    from workloads import random_bf16_bits

    import memory_bound_normalization_amd as mbn

    rng = np.random.default_rng(M ^ N ^ 5)
    block = random_bf16_bits(rng, (1024, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    x = to_gpu_bf16(block).repeat(M // 1024, 1).contiguous()
    wg = to_gpu_bf16(w)
    y = torch.empty_like(x)
    mbn.rmsnorm_fwd(x, wg, y, eps=1e-5)
    first = y.clone()
    for _ in range(9):
        mbn.rmsnorm_fwd(x, wg, y, eps=1e-5)
        assert torch.equal(y.view(torch.int16), first.view(torch.int16)), "run-to-run difference"
    mbn.rmsnorm_fwd(x, wg, x, eps=1e-5)  # in place
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), first.view(torch.int16)), "in-place output differs"
    ref = o_rms(block, w, 1e-5)
    got = from_gpu_bf16(first)
    assert assert_parity_rows(got, lambda lo, hi: ref[np.arange(lo, hi) % 1024], f"rms M={M} N={N}") == M * N
