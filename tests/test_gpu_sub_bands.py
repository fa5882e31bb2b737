"""GPU parity of the entries of the one-shot launch tables that serve widths
between powers of two: sub-bands (part of a band, served by a configuration
of its own) and exact widths, at the row counts the band's row windows and
the persistent windows leave. Each sub-band is reached at its lowest width, at
a ragged width inside it and at its top width, each exact entry at its width,
with a row count just above every window that would take the launch and not a
multiple of the rows per workgroup, in both storage types; every output is
compared against the fp64 oracle."""

import pytest

from tables import TABLES, persistent_windows

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from norm_ops import TABLE_OPS, check_norm  # noqa: E402  (needs torch)


def _band_entry(entries, i):
    return next(f for f in entries[i + 1:] if not f.sub and not f.max_rows and not f.exact)


def _rows(op, entries, band, nchunk):
    windows = [f.max_rows for f in entries if f.max_rows and f.top == band.top]
    pers = [hi for _, _, hi in persistent_windows(op, nchunk)] if op != "add" else []
    return max(windows + pers + [0]) + 37


def _cases():
    out = []
    for tname, op in TABLE_OPS.items():
        entries = TABLES[tname]
        prev = 0
        for i, e in enumerate(entries):
            if e.sub:
                band = _band_entry(entries, i)
                for nchunk in (prev + 1, (prev + 1 + e.top) // 2 | 1, e.top):
                    out.append((op, _rows(op, entries, band, nchunk), nchunk * 8))
                prev = e.top
            elif e.exact:
                out.append((op, _rows(op, entries, _band_entry(entries, i), e.top), e.top * 8))
            elif not e.max_rows:
                prev = e.top
    return out


CASES = _cases()


def test_every_entry_reached():
    n = sum(3 if e.sub else 1 for entries in TABLES.values() for e in entries if e.sub or e.exact)
    assert n >= 4 and len(CASES) == n


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("op,M,N", CASES)
def test_between_powers_of_two(op, M, N, dtype):
    print(f"[between powers of two {op} {dtype}] M={M} N={N}", flush=True)
    check_norm(op, M, N, M * 3 + N, f"{op} {dtype} M={M} N={N}", dtype=dtype)
