"""GPU parity of the sub-band entries of the one-shot launch tables: between
powers of two, part of a band is served by a configuration of its own (fewer
chunks per lane) at the row counts the band's row windows and the persistent
windows leave. Each sub-band is reached at its lowest width, at a ragged width
inside it and at its top width, with a row count just above every window that
would take the launch and not a multiple of the rows per workgroup; every
output is compared against the fp64 oracle."""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import rmsnorm_fwd as o_rms
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from tables import TABLES, persistent_windows
from workloads import random_bf16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

OPS = {"kRmsTable": "rms"}


def _cases():
    out = []
    for tname, op in OPS.items():
        entries = TABLES[tname]
        prev = 0
        for i, e in enumerate(entries):
            if e.sub:
                band = next(f for f in entries[i + 1:] if not f.sub and not f.max_rows and not f.exact)
                windows = [f.max_rows for f in entries if f.max_rows and f.top == band.top]
                for nchunk in (prev + 1, (prev + 1 + e.top) // 2 | 1, e.top):
                    pers = [hi for _, _, hi in persistent_windows(op, nchunk)]
                    M = max(windows + pers + [0]) + 37
                    out.append((op, M, nchunk * 8))
                prev = e.top
            elif not e.max_rows and not e.exact:
                prev = e.top
    return out


CASES = _cases()


def test_every_sub_band_reached():
    subs = sum(1 for entries in TABLES.values() for e in entries if e.sub)
    assert subs >= 1 and len(CASES) == 3 * subs


@pytest.mark.parametrize("op,M,N", CASES)
def test_sub_band_entry(op, M, N):
    print(f"[sub band {op}] M={M} N={N}", flush=True)
    rng = np.random.default_rng(M * 3 + N)
    x = random_bf16_bits(rng, (M, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    y = mbn.rmsnorm_fwd(to_gpu_bf16(x), to_gpu_bf16(w), eps=1e-6)
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), o_rms(x, w, 1e-6), f"{op} M={M} N={N}")
