"""Host-side checks of the row-norm launch tables in rownorm.hip (no GPU):
bands cover every width up to MBN_RMSNORM_MAX_N in increasing order, every
entry with several waves per row serves only widths of at least 64 * WPR chunks
(each wave parks its partial sum in its own first chunk), workgroups stay within
1024 threads and the staged rows within the 160 KiB of LDS of a CU, and the
row windows of a band precede its entry for any row count, in increasing order
and with its width, and sub-band entries come between a band's windows and
its entry, in increasing width; the persistent tables serve only widths their kernel
covers, with sane row windows and double buffers that fit in LDS."""

import pytest

from tables import PERSISTENT, TABLES


def test_all_four_tables_found():
    assert set(TABLES) == {"kRmsTable", "kAddRmsTable", "kLayerTable", "kL2Table"}


@pytest.mark.parametrize("name", sorted(TABLES))
def test_table_invariants(name):
    prev = 0  # widest row of the previous band
    band_top = None  # top width of the current band's row windows
    windows = []  # (exact, max_rows) of the current band's row windows, in table order
    sub_top = 0  # widest row of the last sub-band of the current band
    for e in TABLES[name]:
        top = e.top
        lowest = top if e.exact else max(prev, sub_top) + 1
        assert e.wpr == 1 or lowest >= 64 * e.wpr, (name, e)
        assert 64 * e.wpr * e.rows <= 1024
        assert e.rows * e.rpl * e.capacity * 16 <= 160 * 1024
        assert e.cap >= 0 and e.grp >= 0
        assert top <= e.capacity, (name, e)
        if e.max_rows:
            assert not e.sub and top > prev, (name, e)  # exact windows serve the band's top width
            assert not sub_top, (name, e)  # windows precede the band's sub-bands
            assert band_top is None or band_top == top, (name, top)  # the previous band closed
            band_top = top
            # first match wins: an exact window must be reached at the top width
            # past every window before it, a window of the whole band at the
            # widths below the top past the band's windows before it
            if e.exact:
                assert all(e.max_rows > m for _, m in windows), (name, e)
            else:
                assert all(e.max_rows > m for x, m in windows if not x), (name, e)
            windows.append((e.exact, e.max_rows))
        elif e.sub:
            assert top > max(prev, sub_top), (name, e)  # increasing sub-bands
            sub_top = top
        elif not e.exact:
            assert top > max(prev, sub_top)
            assert band_top is None or band_top == top, (name, top)  # windows end in their band's entry
            band_top = None
            windows = []
            sub_top = 0
            prev = top
    assert band_top is None and not windows and not sub_top
    assert prev * 8 == 65536  # the widest band reaches MBN_RMSNORM_MAX_N


def test_sub_bands_inside_their_band():
    """A sub-band entry serves part of the band whose entry follows it, never
    the band's top width (which the band entry keeps)."""
    for name, entries in TABLES.items():
        for i, e in enumerate(entries):
            if e.sub:
                band = next(f for f in entries[i + 1:] if not f.sub and not f.max_rows and not f.exact)
                assert e.top < band.top, (name, e)


def test_chunk_wait_entries():
    """Per-chunk waits are never asked of the residual add (its first pass
    also stores), and a row window asks for them only at its exact width."""
    n = 0
    for name, entries in TABLES.items():
        for e in entries:
            if e.chunk_wait:
                n += 1
                assert name != "kAddRmsTable", (name, e)
                assert not e.max_rows or e.exact, (name, e)
                assert e.rpl * e.maxc <= 63  # one vmcnt immediate per staged chunk
    assert n >= 5


def test_row_windows_present():
    """Every table has row windows for the small launches of its middle bands."""
    for name, entries in TABLES.items():
        assert sum(1 for e in entries if e.max_rows) >= 5, name


def test_persistent_tables_found():
    assert set(PERSISTENT) == {"kRmsPersistent", "kLayerPersistent", "kL2Persistent"}
    assert all(PERSISTENT.values())


@pytest.mark.parametrize("name", sorted(PERSISTENT))
def test_persistent_invariants(name):
    for lo, hi, wpr, rpl, maxc, grid, min_rows, max_rows in PERSISTENT[name]:
        assert 1 <= lo <= hi <= 64 * wpr * maxc, (name, lo, hi)
        assert 64 * wpr * (maxc // 2) < hi or maxc == 1  # no narrower kernel would do
        assert 64 * wpr <= 1024 and rpl >= 1
        # two buffers of rpl rows plus the partial sums
        assert 2 * rpl * hi * 16 + 4 * rpl * wpr * 4 <= 160 * 1024
        assert 256 <= grid <= 8 * 256
        assert 1 <= min_rows <= max_rows


@pytest.mark.parametrize("name", sorted(PERSISTENT))
def test_persistent_windows_do_not_overlap(name):
    """Within one width band the row windows are disjoint, so the first match
    is the only match."""
    bands = {}
    for lo, hi, *_, min_rows, max_rows in PERSISTENT[name]:
        bands.setdefault((lo, hi), []).append((min_rows, max_rows))
    spans = sorted(bands)
    for (a_lo, a_hi), (b_lo, b_hi) in zip(spans, spans[1:]):
        assert a_hi < b_lo  # bands are disjoint too
    for windows in bands.values():
        windows.sort()
        for (_, a_max), (b_min, _) in zip(windows, windows[1:]):
            assert a_max < b_min


def test_register_windows_precede_the_persistent_table():
    """An exact-width register-row window serves its launches even where a
    persistent entry covers the same width and row count; past the window the
    persistent kernel serves them again."""
    from tables import pick_entry, serves_persistent

    assert pick_entry("kRmsTable", 512, 3000).regs and not serves_persistent("kRmsTable", "rms", 512, 3000)
    assert serves_persistent("kRmsTable", "rms", 512, 5000)
    assert pick_entry("kLayerTable", 512, 1000).regs and not serves_persistent("kLayerTable", "layer", 512, 1000)
    assert serves_persistent("kLayerTable", "layer", 512, 4000)
    # a ragged width of the same band has no exact window: persistent
    assert serves_persistent("kRmsTable", "rms", 500, 3000)
    # the residual add has no persistent kernel
    assert not serves_persistent("kAddRmsTable", "add", 512, 3000)
