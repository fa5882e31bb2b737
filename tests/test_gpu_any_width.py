"""GPU parity of the any-width row norms (rows that are not whole 16-byte
chunks, N % 8 != 0, or pointers that are only element-aligned) against the
fp64 oracle, every output compared.

Two kernel families serve these launches. When x, y (and r, h) sit at the
same address modulo 16, from N = 1024 (except for N % 4 == 0 with 8-byte
aligned pointers, which stay on 4-element groups) and from N = 256 on pointers
that are not 8-byte aligned, the 16-byte staged kernels copy the
aligned chunks that cover each row into LDS (the edge chunks hold elements of
the neighbouring rows, masked out), compute in that chunk grid and store
interior chunks whole and edge chunks element by element; the weight chunks
are shifted windows. Otherwise the element-group kernels access groups of 4,
2 or 1 elements: 4 whenever every pointer is 8-byte aligned (for N % 4 != 0
with a 0-3 element head and tail per row and shifted weight groups), 2 or 1
for pointers aligned to less. The widths cover every band of both families'
launch tables on both sides of the band edges, and every head length (rows
start at different offsets); views at an element offset reach the small
groups (narrow rows, or y at another offset than x modulo 16) and the staged
kernels' non-zero block offsets. Row counts include a single row and counts
that are not a multiple of anything. Outputs are written into views of larger
buffers whose guard elements must stay untouched: no kernel writes outside
its rows, including the neighbouring rows' elements that share a 16-byte
chunk.
"""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import add_rmsnorm_fwd as o_add, l2norm_fwd as o_l2, layernorm_fwd as o_ln, rmsnorm_fwd as o_rms
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from workloads import f32_to_bf16_bits, random_bf16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

WIDTHS = [
    1, 3, 7, 9, 511, 513, 2047, 2049, 8191, 8193, 12345, 32767, 32769, 40001, 65535,  # odd: 1 element
    2, 6, 1002, 1026, 4094, 4098, 8190, 8194, 32766, 32770, 65534,  # N % 4 == 2: 2 elements
    12, 100, 1004, 1028, 4092, 4100, 8188, 8196, 32764, 32772, 40000, 65532,  # N % 8 == 4: 4 elements
    1522, 1523, 3058, 3059, 4082, 4083, 8178, 8179, 16370, 16371, 24562, 24563, 32754, 32755,  # staged-kernel
    65522, 65523,  # band edges
]
GUARD = 8  # guard elements around an output view (16 bytes: keeps the view's alignment)
FILL = 0x4B00  # bf16 / fp16 bit pattern the guards hold


def _rows(N):
    return 3 if N > 32768 else (5 if N > 8192 else 37)


def _inputs(M, N, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    if dtype == "f16":
        f = lambda a: a.astype(np.float16).view(np.uint16)  # noqa: E731
        return (f(rng.standard_normal((M, N))), f(rng.standard_normal((M, N))),
                f(rng.uniform(0.5, 1.5, N)), f(rng.uniform(-0.5, 0.5, N)))
    return (random_bf16_bits(rng, (M, N)), random_bf16_bits(rng, (M, N)),
            random_bf16_bits(rng, (N,), lo=0.5, hi=1.5), random_bf16_bits(rng, (N,), lo=-0.5, hi=0.5))


def _guarded(M, N, dtype, guard=GUARD):
    """An output buffer with `guard` fill elements before and GUARD after an [M, N] view."""
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    buf = torch.full((M * N + guard + GUARD,), 0, dtype=torch.int16, device="cuda")
    buf.fill_(FILL)
    buf = buf.view(tdt)
    return buf, buf[guard : guard + M * N].view(M, N)


def _guards_intact_at(buf, M, N, guard):
    g = torch.cat([buf[:guard], buf[guard + M * N :]]).view(torch.int16).cpu().numpy().view(np.uint16)
    return bool(np.all(g == FILL))


def _vec_view(bits, off, dtype):
    """A GPU copy of the vector `bits` starting `off` elements into a fresh
    allocation (off % 8 != 0: inside a 16-byte block)."""
    g = to_gpu_bf16(bits, dtype=dtype)
    if not off:
        return g
    buf = torch.zeros(g.numel() + off, dtype=g.dtype, device="cuda")
    buf[off:] = g
    return buf[off:]


def _check(op, M, N, seed, dtype="bf16", eps=1e-6, offset=0, out_offset=None, w_off=0, b_off=0):
    """`offset` (elements) places x and r at that offset from an aligned
    address, `out_offset` (default: the same) the outputs: element-aligned
    pointers (2- or 1-element groups, or staged chunks at a block offset);
    `w_off` and `b_off` the weight and the bias."""
    out_offset = offset if out_offset is None else out_offset
    print(f"[any-width {op} {dtype}] M={M} N={N} offset={offset} out_offset={out_offset} w_off={w_off} "
          f"b_off={b_off}", flush=True)
    x, r, w, b = _inputs(M, N, seed, dtype)
    xg, rg = to_gpu_bf16(x, dtype=dtype), to_gpu_bf16(r, dtype=dtype)
    wg, bg = _vec_view(w, w_off, dtype), _vec_view(b, b_off, dtype)
    if offset:
        xb = torch.zeros(M * N + offset, dtype=xg.dtype, device="cuda")
        xb[offset:] = xg.view(-1)
        xg = xb[offset:].view(M, N)
        rb = torch.zeros(M * N + offset, dtype=rg.dtype, device="cuda")
        rb[offset:] = rg.view(-1)
        rg = rb[offset:].view(M, N)
    ybuf, y = _guarded(M, N, dtype, GUARD + out_offset)
    if op == "rms":
        mbn.rmsnorm_fwd(xg, wg, y, eps=eps)
        ref = o_rms(x, w, eps, dtype=dtype)
    elif op == "layer":
        mbn.layernorm_fwd(xg, wg, bg, y, eps=eps)
        ref = o_ln(x, w, b, eps, dtype=dtype)
    elif op == "l2":
        mbn.l2norm_fwd(xg, y, eps=eps)
        ref = o_l2(x, eps, dtype=dtype)
    else:
        hbuf, h = _guarded(M, N, dtype, GUARD + out_offset)
        mbn.add_rmsnorm_fwd(xg, rg, wg, h=h, y=y, eps=eps)
        rh, ref = o_add(x, r, w, eps, dtype=dtype)
        torch.cuda.synchronize()
        assert np.array_equal(from_gpu_bf16(h), rh), f"h = round(x + r) not bit-exact, {op} M={M} N={N}"
        assert _guards_intact_at(hbuf, M, N, GUARD + out_offset), "wrote outside h"
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), ref, f"{op} M={M} N={N} {dtype}", dtype=dtype)
    assert _guards_intact_at(ybuf, M, N, GUARD + out_offset), "wrote outside y"


@pytest.mark.parametrize("N", WIDTHS)
@pytest.mark.parametrize("op", ["rms", "add", "layer", "l2"])
def test_any_width(op, N):
    _check(op, _rows(N), N, seed=N)


# views at an element offset: 1 element -> 2-byte accesses, 2 -> 4-byte (even N)
SMALL_GROUP_WIDTHS = [1, 7, 255, 256, 300, 498, 499, 513, 1010, 1011, 2034, 2035, 2049, 8193, 32769, 65535,
                      2, 1026, 4098, 8194, 32770, 65534]


@pytest.mark.parametrize("N", SMALL_GROUP_WIDTHS)
@pytest.mark.parametrize("op", ["rms", "add", "layer", "l2"])
def test_any_width_small_groups(op, N):
    _check(op, _rows(N), N, seed=N + 7, offset=1 if N % 2 else 2)
    if N % 2 == 0:
        _check(op, _rows(N), N, seed=N + 8, offset=1)


# x (and r) at one offset, the outputs at another modulo 16 bytes: the
# element-group kernels at every width (1-, 2- and 4-element groups)
MIXED_WIDTHS = [2049, 8193, 32769, 65535, 1026, 8194, 32770, 4100, 40000, 4096]


@pytest.mark.parametrize("N", MIXED_WIDTHS)
@pytest.mark.parametrize("op", ["rms", "add", "layer", "l2"])
def test_any_width_mixed_offsets(op, N):
    _check(op, _rows(N), N, seed=N + 9, offset=1, out_offset=0)
    _check(op, _rows(N), N, seed=N + 10, offset=0, out_offset=4 if N % 4 == 0 else 2)


@pytest.mark.parametrize("N", [3, 1001, 8191, 40001, 4098, 4100, 40000])
@pytest.mark.parametrize("op", ["rms", "add", "layer", "l2"])
def test_any_width_f16(op, N):
    _check(op, _rows(N), N, seed=N + 1, dtype="f16", eps=1e-5)


# Weight and bias views that start inside a 16-byte block: the staged kernels
# read each weight (bias) chunk as a shifted window of the two aligned blocks
# under it, clamped to the blocks that hold the vector's elements.
@pytest.mark.parametrize("N,w_off,b_off", [(1011, 3, 3), (1523, 7, 3), (2049, 1, 6), (3059, 4, 1), (8193, 2, 0),
                                           (16383, 5, 2), (24563, 2, 7), (40001, 3, 3), (65535, 6, 5)])
@pytest.mark.parametrize("op", ["rms", "add", "layer"])
def test_staged_weight_offsets(op, N, w_off, b_off):
    _check(op, _rows(N), N, seed=N + 11, offset=1 if N < 1024 else 0, w_off=w_off, b_off=b_off)


@pytest.mark.parametrize("M", [1, 2, 65, 20000])
def test_any_width_row_counts(M):
    _check("rms", M, 1001, seed=M)
    _check("layer", M, 1001, seed=M + 1)
    _check("add", M, 1004, seed=M + 2)
    _check("l2", M, 1002, seed=M + 3)


@pytest.mark.parametrize("offset", [1, 2, 4])
def test_aligned_width_with_misaligned_pointers(offset):
    """N % 8 == 0 but x at an offset of 1, 2 or 4 elements (2, 4 or 8 bytes):
    the any-width kernels serve it with 1-, 2- or 4-element groups."""
    M, N = 9, 4096
    x, r, w, b = _inputs(M, N, 11 + offset)
    for op in ("rms", "layer", "l2"):
        print(f"[any-width misaligned {op}] M={M} N={N} offset={offset}", flush=True)
        xb = torch.zeros(M * N + offset, dtype=torch.bfloat16, device="cuda")
        xb[offset:] = to_gpu_bf16(x).view(-1)
        xv = xb[offset:].view(M, N)
        if op == "rms":
            y, ref = mbn.rmsnorm_fwd(xv, to_gpu_bf16(w)), o_rms(x, w, 1e-6)
        elif op == "layer":
            y, ref = mbn.layernorm_fwd(xv, to_gpu_bf16(w), to_gpu_bf16(b), eps=1e-6), o_ln(x, w, b, 1e-6)
        else:
            y, ref = mbn.l2norm_fwd(xv, eps=1e-6), o_l2(x, 1e-6)
        torch.cuda.synchronize()
        assert_parity(from_gpu_bf16(y), ref, f"misaligned {op} offset {offset}")


def test_in_place_and_special_rows():
    M, N = 6, 4099
    rng = np.random.default_rng(12)
    x = random_bf16_bits(rng, (M, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    x[1, 17] = 0x7FC0  # NaN
    x[2, :] = 0  # zero row
    x[3, 4098] = 0x7F80  # +inf in the last element
    x[4, :] = f32_to_bf16_bits(np.full(N, 1e15, dtype=np.float32))
    ref = o_rms(x, w, 1e-6)
    xg = to_gpu_bf16(x)
    mbn.rmsnorm_fwd(xg, to_gpu_bf16(w), xg, eps=1e-6)  # in place
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(xg), ref, "in place, special rows")
    # eps = 0: the zero row becomes NaN
    xg = to_gpu_bf16(x)
    y = mbn.rmsnorm_fwd(xg, to_gpu_bf16(w), eps=0.0)
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), o_rms(x, w, 0.0), "eps = 0")
