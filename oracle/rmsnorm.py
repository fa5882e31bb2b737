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

from .bf16 import narrow, widen


def rmsnorm_fwd_f64(x_bits, w_bits, eps: float, dtype: str = "bf16") -> np.ndarray:
    """Unrounded float64 RMSNorm output for 16-bit inputs x [M, N] and w [N]."""
    x = widen(x_bits, dtype)
    w = widen(w_bits, dtype)
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


def rmsnorm_fwd(x_bits, w_bits, eps: float, dtype: str = "bf16") -> np.ndarray:
    """RMSNorm of x [M, N] with weight w [N]; returns y [M, N] as 16-bit patterns.

    ``dtype`` is the storage type of inputs and output ("bf16" or "f16").
    Float64 throughout, one rounding to the storage type at the end.
    """
    return narrow(rmsnorm_fwd_f64(x_bits, w_bits, eps, dtype), dtype)
