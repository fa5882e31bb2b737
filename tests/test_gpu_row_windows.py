"""GPU parity of the row-window entries of the one-shot launch tables: small
launches (a few hundred to a few thousand rows) use configurations of their
own, one per window. Every windowed entry of the four tables is reached here
at the lowest row count that selects it (the window's lower edge), at the
band's top width (the fixed-width kernel) and at a ragged width inside the band
(the general kernel; windows of one exact width only at that width), and at
the top row count of its window where that launch stays within 16M elements; against the fp64 oracle, every output compared."""

import pytest

from tables import TABLES, serves_persistent

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from norm_ops import TABLE_OPS as OPS, check_norm  # noqa: E402  (needs torch)


def _cases():
    out = []
    for tname, op in OPS.items():
        prev = 0
        pending = []
        for e in TABLES[tname]:
            top = e.top
            if e.max_rows:
                pending.append((e.max_rows, top, e.exact))
                continue
            if not e.exact and not e.sub:
                # lowest row count that selects a window: past every earlier
                # window for an exact one (top width only), past the earlier
                # windows of the whole band for the others
                below_all = below_band = 0
                for max_rows_w, top_w, exact in pending:
                    assert top_w == top
                    below = below_all if exact else below_band
                    lo = below + 1 if below else min(max_rows_w, 100)
                    for nchunk in (top,) if exact else (top, (prev + 1 + top) // 2):
                        out.append((op, lo, nchunk * 8))
                    if max_rows_w != lo and max_rows_w * top * 8 <= 16 << 20:
                        out.append((op, max_rows_w, top * 8))
                    below_all = max(below_all, max_rows_w)
                    if not exact:
                        below_band = max(below_band, max_rows_w)
                pending = []
                prev = top
    return out


CASES = _cases()


def test_every_window_reached():
    assert len(CASES) >= 2 * 30


_TABLE_OF = {op: t for t, op in OPS.items()}


def _persistent_here(op, M, N):
    return serves_persistent(_TABLE_OF[op], op, N // 8, M)


@pytest.mark.parametrize("op,M,N", CASES)
def test_row_window_entry(op, M, N):
    if _persistent_here(op, M, N):
        pytest.skip("the persistent kernel serves this launch")  # covered by test_gpu_persistent
    print(f"[row window {op}] M={M} N={N}", flush=True)
    check_norm(op, M, N, M * 7 + N, f"{op} M={M} N={N}")
