"""GPU parity of the per-chunk-wait kernels: the _W entries of the launch
tables carry a second full-width kernel whose first pass takes each staged
chunk as it lands (s_waitcnt on the count of copies still outstanding), used
for grids of at least 1024 workgroups. Each such entry is reached at its full
width with the smallest row count that selects it plus a remainder, so the
grid's last workgroup has rows past M (the path that waits for every load);
every output is compared against the fp64 oracle, in both storage types."""

import pytest

from tables import TABLES, persistent_windows

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from norm_ops import TABLE_OPS, check_norm  # noqa: E402  (needs torch)

MIN_BLOCKS = 1024  # the launcher's threshold for the per-chunk-wait kernel


def _cases():
    out = []
    for tname, op in TABLE_OPS.items():
        entries = TABLES[tname]
        for e in entries:
            if not e.chunk_wait:
                continue
            nchunk = e.capacity  # the full-width kernel
            band_top = e.top if not (e.sub or e.exact) else next(
                f.top for f in entries[entries.index(e) + 1:] if not f.sub and not f.max_rows and not f.exact)
            windows = [f.max_rows for f in entries if f.max_rows and f.top == band_top]
            pers = [hi for _, _, hi in persistent_windows(op, nchunk)] if op != "add" else []
            rows_per_wg = e.rows * e.rpl
            if e.max_rows:  # a row window: just below its top row count
                M = e.max_rows - 1
                assert M > max([w for w in windows if w < e.max_rows] + pers + [MIN_BLOCKS * rows_per_wg - 1])
            else:
                M = max(windows + pers + [MIN_BLOCKS * rows_per_wg]) + 1
            if M % rows_per_wg == 0 and rows_per_wg > 1:
                M += 1  # the last workgroup has rows past M
            out.append((op, M, nchunk * 8))
    return out


CASES = _cases()


def test_every_chunk_wait_entry_reached():
    assert len(CASES) == sum(1 for v in TABLES.values() for e in v if e.chunk_wait) >= 5


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op,M,N", CASES)
def test_chunk_wait_entry(op, M, N, dtype):
    print(f"[chunk wait {op} {dtype}] M={M} N={N}", flush=True)
    check_norm(op, M, N, M + N, f"{op} {dtype} M={M} N={N}", dtype=dtype)


def _repeat_equal(fn, reps):
    first = fn().clone()
    for _ in range(reps - 1):
        assert torch.equal(fn().view(torch.int16), first.view(torch.int16)), "run-to-run difference"
    return first


@pytest.mark.parametrize("op,M,N", [("rms", 16384, 16384), ("rms", 4096, 32768), ("rms", 8193, 4096),
                                    ("layer", 16384, 16384), ("rms", 6143, 16384)])
def test_chunk_wait_deterministic_at_size(op, M, N):
    """A chunk taken before it landed would read stale LDS and show up as a
    run-to-run difference: the per-chunk-wait kernels at full size (the
    headline shape among them), ten launches each, every output bit-identical,
    and every output checked against the oracle."""
    print(f"[chunk wait repeat {op}] M={M} N={N}", flush=True)
    import numpy as np

    from oracle import layernorm_fwd as o_ln, rmsnorm_fwd as o_rms
    from parity import assert_parity_rows, from_gpu_bf16, to_gpu_bf16
    from workloads import random_bf16_bits

    import memory_bound_normalization_amd as mbn

    rng = np.random.default_rng(M ^ N)
    block = random_bf16_bits(rng, (1024, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    b = random_bf16_bits(rng, (N,), lo=-0.5, hi=0.5)
    x = to_gpu_bf16(block).repeat(-(-M // 1024), 1)[:M].contiguous()
    wg, bg = to_gpu_bf16(w), to_gpu_bf16(b)
    y = torch.empty_like(x)
    if op == "rms":
        fn = lambda: mbn.rmsnorm_fwd(x, wg, y, eps=1e-6)  # noqa: E731
    else:
        fn = lambda: mbn.layernorm_fwd(x, wg, bg, y, eps=1e-5)  # noqa: E731
    out = _repeat_equal(fn, 10)
    torch.cuda.synchronize()
    ref = o_rms(block, w, 1e-6) if op == "rms" else o_ln(block, w, b, 1e-5)
    got = from_gpu_bf16(out)
    # the input repeats one 1024-row block, so row i's oracle output is that of block row i % 1024
    assert assert_parity_rows(got, lambda lo, hi: ref[np.arange(lo, hi) % 1024], f"{op} M={M} N={N}") == M * N
