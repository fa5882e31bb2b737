"""Seeded synthetic inputs for the normalization workloads.

This module is the one thing the CPU oracle and the HIP path have in common:
it draws the input bit patterns that both sides consume. It holds none of the
method's arithmetic (no sum of squares, no normalization, no rotation); it only
draws random numbers and quantizes them to bf16 (or, for the fp16 tests,
binary16) input bits.

Recipe (every workload): a fresh ``numpy.random.default_rng(seed)`` (PCG64),
values drawn as float32 in the order x -> w -> extras, scaled in float32, then
rounded to bf16 with round-to-nearest-even on the float32 bit pattern. Returned
arrays hold raw bf16 bits as ``uint16``.

Workloads (shapes and distributions of the normalization pages' RMSNorm
benchmark grid, "[Inductor] Codegen Gluon", section 3.1, and of the packed-QKV
operator of "[pretuned] Optimize fused_qk_norm_rope on B200", Summary):

* ``rms_1024x4096``   x[1024, 4096] ~ N(0, 1), w ~ U(0.5, 1.5), eps 1e-6
* ``rms_8192x8192``   x[8192, 8192] ~ N(0, 1) with 1% of rows (81) scaled by
  100 in float32 before rounding, w ~ U(0.5, 1.5), eps 1e-6
* ``rms_16384x16384`` x[16384, 16384] ~ N(0, 1), w ~ U(0.5, 1.5), eps 1e-6
* ``rms_4096x32768``  x[4096, 32768] ~ 0.5 * N(0, 1), w ~ U(0.5, 1.5), eps 1e-5
* residual add + RMSNorm, LayerNorm, L2Norm: x and w of an RMSNorm workload,
  then (same generator, drawn after w) r ~ N(0, 1) [M, N] for the residual
  add, or b ~ U(-0.5, 0.5) [N] for the LayerNorm bias
* ``qk_256``          qkv[256, (32 + 8 + 8) * 128] ~ N(0, 1) (v heads too),
  q_w then k_w [128] ~ U(0.5, 1.5), positions 0..255 (int64), eps 1e-6,
  theta 1e6
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "RMS_WORKLOADS",
    "QK_WORKLOADS",
    "RmsWorkload",
    "QkWorkload",
    "f32_to_bf16_bits",
    "make_rms_inputs",
    "make_norm_family_inputs",
    "make_qk_inputs",
    "random_bf16_bits",
    "random_f16_bits",
]


@dataclasses.dataclass(frozen=True)
class RmsWorkload:
    name: str
    M: int
    N: int
    eps: float
    x_scale: float = 1.0
    outlier_frac: float = 0.0
    outlier_scale: float = 100.0
    seed: int = 0

    @property
    def algorithmic_bytes(self) -> int:
        # every x element read once, every y element written once, w read once
        return 2 * self.M * self.N * 2 + 2 * self.N


@dataclasses.dataclass(frozen=True)
class QkWorkload:
    name: str
    T: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    eps: float
    theta: float
    seed: int = 0

    @property
    def row_width(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def algorithmic_bytes(self) -> int:
        qk = self.T * (self.n_q_heads + self.n_kv_heads) * self.head_dim * 2
        return 2 * qk + 2 * 2 * self.head_dim + 8 * self.T


RMS_WORKLOADS = {
    w.name: w
    for w in (
        RmsWorkload("rms_1024x4096", 1024, 4096, 1e-6),
        RmsWorkload("rms_8192x8192", 8192, 8192, 1e-6, outlier_frac=0.01),
        RmsWorkload("rms_16384x16384", 16384, 16384, 1e-6),
        RmsWorkload("rms_4096x32768", 4096, 32768, 1e-5, x_scale=0.5),
    )
}

QK_WORKLOADS = {
    w.name: w
    for w in (QkWorkload("qk_256", 256, 32, 8, 128, 1e-6, 1e6),)
}


def f32_to_bf16_bits(a: np.ndarray, block: int = 1 << 24) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Works on the float32 bit pattern: add 0x7FFF plus the lowest kept bit, then
    drop the low 16 bits. Processed in blocks to bound temporaries.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for s in range(0, flat.size, block):
        u = flat[s : s + block].view(np.uint32)
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        out[s : s + block] = r.astype(np.uint16)
    return out.reshape(a.shape)


def _uniform_f32(rng: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    return np.float32(lo) + np.float32(hi - lo) * rng.random(n, dtype=np.float32)


def make_rms_inputs(wl: RmsWorkload, rows: int | None = None):
    """Return (x_bits [M, N] uint16, w_bits [N] uint16, eps) for an RMSNorm workload.

    ``rows`` keeps only the first ``rows`` rows (the full matrix is still drawn,
    so the kept rows are identical to those of the full workload).
    """
    rng = np.random.default_rng(wl.seed)
    x = rng.standard_normal((wl.M, wl.N), dtype=np.float32)
    if wl.x_scale != 1.0:
        x *= np.float32(wl.x_scale)
    w = _uniform_f32(rng, wl.N, 0.5, 1.5)
    if wl.outlier_frac > 0.0:
        k = int(wl.M * wl.outlier_frac)
        idx = rng.choice(wl.M, size=k, replace=False)
        x[idx] *= np.float32(wl.outlier_scale)
    if rows is not None:
        x = x[:rows]
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w), wl.eps


def make_norm_family_inputs(wl: RmsWorkload, rows: int | None = None):
    """Inputs for the other row norms on an RMSNorm workload's shape.

    Returns (x_bits, w_bits, r_bits, b_bits, eps): x and w exactly as
    make_rms_inputs (outlier rows included), then r ~ N(0, 1) [M, N] and
    b ~ U(-0.5, 0.5) [N] from the same generator.
    """
    rng = np.random.default_rng(wl.seed)
    x = rng.standard_normal((wl.M, wl.N), dtype=np.float32)
    if wl.x_scale != 1.0:
        x *= np.float32(wl.x_scale)
    w = _uniform_f32(rng, wl.N, 0.5, 1.5)
    if wl.outlier_frac > 0.0:
        k = int(wl.M * wl.outlier_frac)
        idx = rng.choice(wl.M, size=k, replace=False)
        x[idx] *= np.float32(wl.outlier_scale)
    r = rng.standard_normal((wl.M, wl.N), dtype=np.float32)
    b = _uniform_f32(rng, wl.N, -0.5, 0.5)
    if rows is not None:
        x, r = x[:rows], r[:rows]
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w), f32_to_bf16_bits(r), f32_to_bf16_bits(b), wl.eps


def outlier_rows(wl: RmsWorkload) -> np.ndarray:
    """Indices of the rows scaled by ``outlier_scale`` (same draw as make_rms_inputs)."""
    if wl.outlier_frac <= 0.0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(wl.seed)
    rng.standard_normal((wl.M, wl.N), dtype=np.float32)
    rng.random(wl.N, dtype=np.float32)
    return np.sort(rng.choice(wl.M, size=int(wl.M * wl.outlier_frac), replace=False))


def make_qk_inputs(wl: QkWorkload):
    """Return (qkv_bits [T, W] uint16, q_w_bits, k_w_bits, positions int64, eps, theta)."""
    rng = np.random.default_rng(wl.seed)
    qkv = rng.standard_normal((wl.T, wl.row_width), dtype=np.float32)
    q_w = _uniform_f32(rng, wl.head_dim, 0.5, 1.5)
    k_w = _uniform_f32(rng, wl.head_dim, 0.5, 1.5)
    pos = np.arange(wl.T, dtype=np.int64)
    return (
        f32_to_bf16_bits(qkv),
        f32_to_bf16_bits(q_w),
        f32_to_bf16_bits(k_w),
        pos,
        wl.eps,
        wl.theta,
    )


def random_bf16_bits(rng: np.random.Generator, shape, scale: float = 1.0, lo=None, hi=None):
    """Small helper for edge-case tests: N(0, scale) or U(lo, hi) values as bf16 bits."""
    if lo is not None:
        n = int(np.prod(shape))
        v = _uniform_f32(rng, n, lo, hi).reshape(shape)
    else:
        v = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return f32_to_bf16_bits(v)


def random_f16_bits(rng: np.random.Generator, shape, scale: float = 1.0, lo=None, hi=None):
    """As random_bf16_bits, for IEEE binary16 storage (numpy's float16 cast,
    round to nearest even)."""
    if lo is not None:
        n = int(np.prod(shape))
        v = _uniform_f32(rng, n, lo, hi).reshape(shape)
    else:
        v = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return v.astype(np.float16).view(np.uint16)
