"""RMSNorm forward, plain definition in float64 (test infrastructure only).

Source: "[Inductor] Codegen Gluon", section 3.1 ("MVP: RMSNorm with
TMA-Cached Reused Input"). The reference workload needs x twice: for the sum
of its squares, and again when it is scaled by rstd and the weight. Written
out per row i:

    ms_i   = (1/N) * sum_j x_ij^2          mean over the N columns
    rstd_i = 1 / sqrt(ms_i + eps)          eps inside the square root
    y_ij   = x_ij * rstd_i * w_j           weight applied after normalizing

Readings where the page is silent (each listed in the design notes):
* eps is taken as the float32 value the C interface receives, widened exactly.
* No bias and no residual term.
* IEEE semantics for special rows: a zero row gives 0 when eps > 0 and NaN when
  eps == 0; a NaN anywhere in a row makes the whole row NaN; an infinite element
  makes ms infinite, so rstd = 0, finite elements become 0 and infinite ones NaN.

Staging the row on chip (the method) changes where x is read from, not what is
computed, so the oracle is this definition and nothing else.
"""

from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits


def rmsnorm_fwd_f64(x_bits, w_bits, eps: float) -> np.ndarray:
    """Unrounded float64 RMSNorm output for bf16 inputs x [M, N] and w [N]."""
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    if x.ndim != 2 or w.ndim != 1 or x.shape[1] != w.shape[0]:
        raise ValueError(f"expected x [M, N] and w [N], got {x.shape} and {w.shape}")
    n = x.shape[1]
    eps64 = float(np.float32(eps))
    if x.shape[0] == 0 or n == 0:
        return np.zeros(x.shape, dtype=np.float64)
    with np.errstate(all="ignore"):
        ms = np.sum(x * x, axis=1) / n
        rstd = 1.0 / np.sqrt(ms + eps64)
        return (x * rstd[:, None]) * w[None, :]


def rmsnorm_fwd(x_bits, w_bits, eps: float) -> np.ndarray:
    """RMSNorm of bf16 x [M, N] with bf16 weight w [N]; returns y [M, N] as bf16 bits.

    Float64 throughout, one rounding to bf16 at the end.
    """
    return f64_to_bf16_bits(rmsnorm_fwd_f64(x_bits, w_bits, eps))
