"""Host-side checks of the row-norm launch tables in rownorm.hip (no GPU):
bands cover every width up to MBN_RMSNORM_MAX_N in increasing order, every
entry with several waves per row serves only widths of at least 64 * WPR chunks
(each wave parks its partial sum in its own first chunk), workgroups stay within
1024 threads and the staged rows within the 160 KiB of LDS of a CU; the
persistent tables serve only widths their kernel covers, with sane row windows
and double buffers that fit in LDS."""

import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "memory_bound_normalization_amd", "csrc", "rownorm.hip")
CFG = r"MBN_CFG(_EXACT)?\((?:MODE|Norm::\w+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)"


def _tables():
    s = open(SRC).read()
    macros = {}
    for name in ("MBN_FIRST_BAND",):
        body = s[s.index("#define " + name):].split("\n")[0]
        macros[name] = re.findall(CFG, body)
    out = {}
    for tname, body in re.findall(r"const RowNormCfg (k\w+)\[\] = \{(.*?)\n\};", s, re.S):
        entries = []
        for line in body.split("\n"):
            line = line.strip()
            found = macros.get(line.split("(")[0], None) if line.startswith("MBN_FIRST_BAND") else None
            for e in (found if found is not None else re.findall(CFG, line)):
                exact, *nums = e
                entries.append((exact == "_EXACT", *map(int, nums)))
        out[tname] = entries
    return out


TABLES = _tables()


def test_all_four_tables_found():
    assert set(TABLES) == {"kRmsTable", "kAddRmsTable", "kLayerTable", "kL2Table"}


@pytest.mark.parametrize("name", sorted(TABLES))
def test_table_invariants(name):
    prev = 0
    for exact, wpr, rows, rpl, maxc, cap, grp in TABLES[name]:
        top = 64 * wpr * maxc
        lowest = top if exact else prev + 1
        assert wpr == 1 or lowest >= 64 * wpr, (name, wpr, maxc)
        assert 64 * wpr * rows <= 1024
        assert rows * rpl * top * 16 <= 160 * 1024
        assert cap >= 0 and grp >= 0
        if not exact:
            assert top > prev
            prev = top
    assert prev * 8 == 65536  # the widest band reaches MBN_RMSNORM_MAX_N


PCFG = r"MBN_PCFG\(Norm::(\w+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)"


def _persistent():
    s = open(SRC).read()
    out = {}
    for tname, body in re.findall(r"const PersistentCfg (k\w+)\[\] = \{(.*?)\n\};", s, re.S):
        out[tname] = [tuple(map(int, e[1:])) for e in re.findall(PCFG, body)]
    return out


PERSISTENT = _persistent()


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
