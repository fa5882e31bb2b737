"""Parser of the row-norm launch tables in rownorm.hip, shared by the host-side
table checks and the GPU tests that must reach every table entry (no GPU
needed here)."""

import os
import re
from collections import namedtuple

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "memory_bound_normalization_amd", "csrc", "rownorm.hip")
CFG = r"MBN_CFG(_EXACT|_ROWS_EXACT|_ROWS|_UPTO)?(_W|_LW)?\((?:MODE|Norm::\w+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)(?:, (\d+))?\)"
# exact-width entries with register-resident rows: WPR, ROWS, MAXC, CAP, GROUP (RPL = 1)
CFG_R = r"MBN_CFG_EXACT_R\((?:MODE|Norm::\w+), (\d+), (\d+), (\d+), (\d+), (\d+)\)"
# row windows with register-resident rows at one exact width: MAXROWS, WPR, ROWS, MAXC, CAP, GROUP
CFG_ROWS_R = r"MBN_CFG_ROWS_EXACT_R\((?:MODE|Norm::\w+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)"


class Entry(namedtuple("Entry", "exact max_rows wpr rows rpl maxc cap grp upto chunk_wait regs late_w",
                       defaults=(False, False))):
    """One launch-table entry. `upto` is the widest row (chunks) a sub-band
    entry (MBN_CFG_UPTO) serves, 0 for the other kinds; `chunk_wait`: a _W
    entry (per-chunk waits in its full-width kernel); `regs`: an _R entry
    (register-resident rows, exact width only); `late_w`: an _LW entry (weight
    loaded after the reduction); `top` is the widest row any entry serves and
    `capacity` its kernel's 64 * wpr * maxc chunks."""

    @property
    def capacity(self):
        return 64 * self.wpr * self.maxc

    @property
    def top(self):
        return self.upto or self.capacity

    @property
    def sub(self):
        return self.upto > 0


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
            for wpr, rows, maxc, cap, grp in re.findall(CFG_R, line):
                entries.append(Entry(True, 0, int(wpr), int(rows), 1, int(maxc), int(cap), int(grp), 0, False, True))
            for max_rows, wpr, rows, maxc, cap, grp in re.findall(CFG_ROWS_R, line):
                entries.append(Entry(True, int(max_rows), int(wpr), int(rows), 1, int(maxc), int(cap), int(grp), 0,
                                     False, True))
            if re.search(CFG_R, line) or re.search(CFG_ROWS_R, line):
                continue
            for e in (found if found is not None else re.findall(CFG, line)):
                kind, w, *nums = e
                nums = [int(v) for v in nums if v != ""]
                max_rows = 0
                upto = 0
                if kind in ("_ROWS", "_ROWS_EXACT"):
                    max_rows, nums = nums[0], nums[1:]
                elif kind == "_UPTO":
                    assert nums[0] % 8 == 0, line
                    upto, nums = nums[0] // 8, nums[1:]
                entries.append(Entry(kind in ("_EXACT", "_ROWS_EXACT"), max_rows, *nums, upto, w == "_W", False,
                                     w == "_LW"))
        out[tname] = entries
    return out


PCFG = r"MBN_PCFG\(Norm::(\w+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)"


def _persistent():
    s = open(SRC).read()
    out = {}
    for tname, body in re.findall(r"const PersistentCfg (k\w+)\[\] = \{(.*?)\n\};", s, re.S):
        out[tname] = [tuple(map(int, e[1:])) for e in re.findall(PCFG, body)]
    return out



TABLES = _tables()
PERSISTENT = _persistent()

PERSISTENT_TABLE = {"rms": "kRmsPersistent", "layer": "kLayerPersistent", "l2": "kL2Persistent"}


def persistent_windows(op, nchunk):
    """(grid, min_rows, max_rows) of the persistent entries of `op` that serve
    rows of `nchunk` 16-byte chunks."""
    return [(grid, lo_r, hi_r) for lo, hi, wpr, rpl, maxc, grid, lo_r, hi_r in PERSISTENT[PERSISTENT_TABLE[op]]
            if lo <= nchunk <= hi]


def pick_entry(tname, nchunk, M):
    """The one-shot table entry the launcher picks for rows of `nchunk`
    16-byte chunks and M rows (the first that serves both), or None."""
    for e in TABLES[tname]:
        if (nchunk == e.top if e.exact else nchunk <= e.top) and (e.max_rows == 0 or M <= e.max_rows):
            return e
    return None


def serves_persistent(tname, op, nchunk, M):
    """Whether the launcher runs the persistent kernel for this launch: a
    persistent entry covers it and no exact-width register-row window (which
    takes precedence) does."""
    e = pick_entry(tname, nchunk, M)
    if e is not None and e.regs and e.max_rows:
        return False
    return op in PERSISTENT_TABLE and any(lo <= M <= hi for _, lo, hi in persistent_windows(op, nchunk))

