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
