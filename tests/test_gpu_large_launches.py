"""GPU parity of launches too large for one dispatch. A dispatch covers at most
2^32 - 1 work-items (32-bit grid size fields), so the launchers split larger
launches into consecutive row (token) ranges: the staged-row kernel at N = 8
(256 lanes per 4 rows: 67,108,860 rows per dispatch), the any-width kernels
(4,194,296 rows per dispatch) and the QK kernel with one head per token (64
lanes: 67,108,863 tokens per dispatch). Each case runs just past one split; the
input is a seeded block of rows tiled over the launch, so every row's expected
value is the oracle's for its block row. The first block and the rows on both
sides of the split and at the end are compared with the fp64 oracle, and every
other row must equal, bit for bit, the output of its block row in the first
block (so every output is covered)."""

import numpy as np
import pytest

from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from workloads import random_bf16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import memory_bound_normalization_amd as mbn  # noqa: E402
from oracle import qk_norm_rope_fwd as o_qk, rmsnorm_fwd as o_rms  # noqa: E402

BLOCK = 4096


def _assert_tiled(out, what):
    """Every row of `out` [M, W] equals row i % BLOCK of its first BLOCK rows."""
    M = out.shape[0]
    head = out[:BLOCK].view(torch.int16)
    full = M // BLOCK
    body = out[: full * BLOCK].view(torch.int16).view(full, BLOCK, -1)
    for s in range(0, full, 256):
        assert torch.equal(body[s : s + 256], head.expand(min(256, full - s), -1, -1)), f"{what}: tiled rows differ"
    rest = M - full * BLOCK
    if rest:
        assert torch.equal(out[full * BLOCK :].view(torch.int16), head[:rest]), f"{what}: tail rows differ"


def _checked_rows(M, split):
    rows = np.concatenate([np.arange(64), np.arange(split - 64, split + 64), np.arange(M - 64, M)])
    return np.unique(rows[(rows >= 0) & (rows < M)])


def _rms_split(M, N, split, label):
    print(f"[large launch {label}] M={M} N={N} split at row {split}", flush=True)
    rng = np.random.default_rng(N)
    block = random_bf16_bits(rng, (BLOCK, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    x = to_gpu_bf16(block).repeat(-(-M // BLOCK), 1)[:M]
    assert x.is_contiguous() and x.shape == (M, N)
    y = mbn.rmsnorm_fwd(x, to_gpu_bf16(w), eps=1e-6)
    torch.cuda.synchronize()
    _assert_tiled(y, f"{label} M={M} N={N}")
    rows = np.union1d(_checked_rows(M, split), np.arange(BLOCK))
    got = from_gpu_bf16(y[torch.from_numpy(rows).cuda()])
    del x, y
    torch.cuda.empty_cache()
    ref = o_rms(block[rows % BLOCK], w, 1e-6)
    assert_parity(got, ref, f"{label} M={M} N={N}")


def test_staged_row_kernel_split():
    split = (0xFFFFFFFF // 256) * 4  # N = 8: 4 rows per 256-lane workgroup
    _rms_split(split + 100, 8, split, "staged rows")


def test_any_width_kernel_split():
    split = (0xFFFFFFFF // 1024) & ~7
    _rms_split(split + 100, 7, split, "any width")


def test_qk_kernel_split():
    split = 0xFFFFFFFF // 64  # one q head, no kv heads: one wave per token
    T = split + 50
    print(f"[large launch qk] T={T} split at token {split}", flush=True)
    rng = np.random.default_rng(5)
    block = random_bf16_bits(rng, (BLOCK, 128))
    q_w = random_bf16_bits(rng, (128,), lo=0.5, hi=1.5)
    k_w = random_bf16_bits(rng, (128,), lo=0.5, hi=1.5)
    qkv = to_gpu_bf16(block).repeat(-(-T // BLOCK), 1)[:T]
    pos = torch.arange(T, device="cuda", dtype=torch.int64) % 8192
    mbn.qk_norm_rope_fwd(qkv, to_gpu_bf16(q_w), to_gpu_bf16(k_w), pos, 1, 0, 128, eps=1e-6, theta=1e6)
    torch.cuda.synchronize()
    # positions repeat every 8192 tokens and the block every 4096 tokens, so
    # the output repeats every 8192 tokens
    _assert_tiled(qkv[: T - T % 2].reshape(-1, 2 * 128), f"qk T={T} (token pairs)")
    toks = np.union1d(_checked_rows(T, split), np.arange(8192))
    got = from_gpu_bf16(qkv[torch.from_numpy(toks).cuda()])
    del qkv, pos
    torch.cuda.empty_cache()
    ref = o_qk(block[toks % BLOCK], q_w, k_w, (toks % 8192).astype(np.int64), 1, 0, 128, 1e-6, 1e6)
    assert_parity(got, ref, f"qk T={T}")
