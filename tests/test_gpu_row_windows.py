"""GPU parity of the row-window entries of the one-shot launch tables: small
launches (a few hundred to a few thousand rows) use configurations of their
own, one per window. Every windowed entry of the four tables is reached here
at the lowest row count that selects it (the window's lower edge), at the
band's top width (the fixed-width kernel) and at a ragged width inside the band
(the general kernel), and at the top row count of its window where that launch
stays within 16M elements; against the fp64 oracle, every output compared."""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import add_rmsnorm_fwd as o_add, l2norm_fwd as o_l2, layernorm_fwd as o_ln, rmsnorm_fwd as o_rms
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from tables import TABLES, persistent_windows
from workloads import random_bf16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

OPS = {"kRmsTable": "rms", "kAddRmsTable": "add", "kLayerTable": "layer", "kL2Table": "l2"}


def _cases():
    out = []
    for tname, op in OPS.items():
        prev = 0
        pending = []
        for e in TABLES[tname]:
            top = e.top
            if e.max_rows:
                pending.append((e.max_rows, top))
                continue
            if not e.exact and not e.sub:
                below = 0  # the previous window's top row count
                for max_rows_w, top_w in pending:
                    assert top_w == top
                    lo = below + 1 if below else min(max_rows_w, 100)
                    for nchunk in (top, (prev + 1 + top) // 2):
                        out.append((op, lo, nchunk * 8))
                    if max_rows_w != lo and max_rows_w * top * 8 <= 16 << 20:
                        out.append((op, max_rows_w, top * 8))
                    below = max_rows_w
                pending = []
                prev = top
    return out


CASES = _cases()


def test_every_window_reached():
    assert len(CASES) >= 2 * 30


def _persistent_here(op, M, N):
    if op == "add":
        return False
    return any(lo <= M <= hi for _, lo, hi in persistent_windows(op, N // 8))


@pytest.mark.parametrize("op,M,N", CASES)
def test_row_window_entry(op, M, N):
    if _persistent_here(op, M, N):
        pytest.skip("the persistent kernel serves this launch")  # covered by test_gpu_persistent
    print(f"[row window {op}] M={M} N={N}", flush=True)
    rng = np.random.default_rng(M * 7 + N)
    x = random_bf16_bits(rng, (M, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    if op == "rms":
        y = mbn.rmsnorm_fwd(to_gpu_bf16(x), to_gpu_bf16(w), eps=1e-6)
        ref = o_rms(x, w, 1e-6)
    elif op == "layer":
        b = random_bf16_bits(rng, (N,), lo=-0.5, hi=0.5)
        y = mbn.layernorm_fwd(to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(b), eps=1e-5)
        ref = o_ln(x, w, b, 1e-5)
    elif op == "l2":
        y = mbn.l2norm_fwd(to_gpu_bf16(x), eps=1e-12)
        ref = o_l2(x, 1e-12)
    else:
        r = random_bf16_bits(rng, (M, N))
        h, y = mbn.add_rmsnorm_fwd(to_gpu_bf16(x), to_gpu_bf16(r), to_gpu_bf16(w), eps=1e-6)
        rh, ref = o_add(x, r, w, 1e-6)
        torch.cuda.synchronize()
        assert np.array_equal(from_gpu_bf16(h), rh), f"add M={M} N={N}: h = bf16(x + r) not bit-exact"
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), ref, f"{op} M={M} N={N}")
