"""GPU parity of the launch-table entries whose kernels load the weight after
the reduction (the _LW entries: rownorm_lw_kernel). Each is reached at its
full width and at a ragged width inside its band, with a row count just above
every row window and persistent window that would take the launch, in both
storage types, every output compared against the fp64 oracle; at the
8192 x 8192 workload shape ten launches must give identical bits."""

import numpy as np
import pytest

from tables import TABLES, persistent_windows

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from norm_ops import TABLE_OPS, check_norm  # noqa: E402  (needs torch)


def _cases():
    out = []
    for tname, op in TABLE_OPS.items():
        entries = TABLES[tname]
        prev = 0
        for e in entries:
            if e.late_w:
                windows = [f.max_rows for f in entries if f.max_rows and f.top == e.top]
                for nchunk in (e.top, (prev + 1 + e.top) // 2 | 1):
                    pers = [hi for _, _, hi in persistent_windows(op, nchunk)] if op != "add" else []
                    out.append((op, max(windows + pers + [0]) + 41, nchunk * 8))
            if not (e.max_rows or e.exact or e.sub):
                prev = e.top
    return out


CASES = _cases()


def test_late_weight_entries_present():
    assert len(CASES) == 2 * sum(1 for v in TABLES.values() for e in v if e.late_w) >= 2


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op,M,N", CASES)
def test_late_weight_entry(op, M, N, dtype):
    print(f"[late weights {op} {dtype}] M={M} N={N}", flush=True)
    check_norm(op, M, N, M * 7 + N, f"{op} {dtype} M={M} N={N}", dtype=dtype)


def test_late_weights_repeat():
    M, N = 8192, 8192
    print(f"[late weights repeat] M={M} N={N}", flush=True)
    from oracle import rmsnorm_fwd as o_rms
    from parity import assert_parity_rows, from_gpu_bf16, to_gpu_bf16
    from workloads import random_bf16_bits

    import memory_bound_normalization_amd as mbn

    rng = np.random.default_rng(M ^ N ^ 7)
    block = random_bf16_bits(rng, (1024, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    x = to_gpu_bf16(block).repeat(M // 1024, 1).contiguous()
    wg = to_gpu_bf16(w)
    y = torch.empty_like(x)
    mbn.rmsnorm_fwd(x, wg, y, eps=1e-6)
    first = y.clone()
    for _ in range(9):
        mbn.rmsnorm_fwd(x, wg, y, eps=1e-6)
        assert torch.equal(y.view(torch.int16), first.view(torch.int16)), "run-to-run difference"
    torch.cuda.synchronize()
    ref = o_rms(block, w, 1e-6)
    got = from_gpu_bf16(first)
    assert assert_parity_rows(got, lambda lo, hi: ref[np.arange(lo, hi) % 1024], f"rms M={M} N={N}") == M * N
