"""Further row norms of the same reused-input family, plain float64 definitions.

TEST INFRASTRUCTURE ONLY.

* ``add_rmsnorm_fwd`` -- residual add fused with RMSNorm. "TorchInductor: from
  ATen IR to Triton kernel", sections 14.25 and 14.27, names the residual add
  fused with the following norm as one of the standard LLM fusions. Reading
  (the page does not fix the precision): the residual stream is a bf16 tensor,
  so h = bf16(x + r) is what is stored, and the norm is taken of that stored h:
      h_ij = RNE_bf16(x_ij + r_ij)
      y_ij = RNE_bf16(h_ij / sqrt(mean_j h_ij^2 + eps) * w_j)
* ``layernorm_fwd`` -- the decomposition printed in section 14.12.2 of the same
  page (var_mean, add eps, rsqrt, subtract the mean, multiply, multiply by the
  weight, add the bias), with the biased (divide-by-N) variance:
      mu = mean_j x_ij,  var = mean_j (x_ij - mu)^2
      y_ij = RNE_bf16((x_ij - mu) / sqrt(var + eps) * w_j + b_j)
  (also "[Inductor] Codegen Gluon", section 3.2: reuses the input in the
  mean/variance reduction and again in the normalize + affine pass).
* ``l2norm_fwd`` -- "[Inductor] Codegen Gluon", section 3.2: one reduction, then
  a scale by the inverse norm. Reading: the eps guard of the usual
  normalize-by-L2 operator, y_ij = RNE_bf16(x_ij / max(sqrt(sum_j x_ij^2), eps)).

All arithmetic in float64 from the exact 16-bit inputs (bf16, or fp16 for the
fp16 variants); eps is the float32 value the C interface receives; one rounding
to the storage type per output.
"""

from __future__ import annotations

import numpy as np

from .bf16 import narrow, widen
from .rmsnorm import rmsnorm_fwd


def add_rmsnorm_fwd(x_bits, r_bits, w_bits, eps: float, dtype: str = "bf16"):
    """Return (h_bits, y_bits): h = round(x + r), y = RMSNorm(h) * w, both rounded
    to the storage type ``dtype``."""
    x = widen(x_bits, dtype)
    r = widen(r_bits, dtype)
    if x.shape != r.shape:
        raise ValueError("x and r must have the same shape")
    with np.errstate(all="ignore"):
        h_bits = narrow(x + r, dtype)
    return h_bits, rmsnorm_fwd(h_bits, w_bits, eps, dtype)


def layernorm_fwd_f64(x_bits, w_bits, b_bits, eps: float, dtype: str = "bf16") -> np.ndarray:
    x = widen(x_bits, dtype)
    w = widen(w_bits, dtype)
    b = widen(b_bits, dtype)
    if x.ndim != 2 or w.shape != (x.shape[1],) or b.shape != (x.shape[1],):
        raise ValueError("expected x [M, N], w [N], b [N]")
    n = x.shape[1]
    if x.shape[0] == 0 or n == 0:
        return np.zeros(x.shape)
    eps64 = float(np.float32(eps))
    with np.errstate(all="ignore"):
        mu = np.sum(x, axis=1) / n
        d = x - mu[:, None]
        var = np.sum(d * d, axis=1) / n
        rstd = 1.0 / np.sqrt(var + eps64)
        return d * rstd[:, None] * w[None, :] + b[None, :]


def layernorm_fwd(x_bits, w_bits, b_bits, eps: float, dtype: str = "bf16") -> np.ndarray:
    """LayerNorm of x [M, N] with weight and bias [N]; 16-bit patterns of ``dtype`` out."""
    return narrow(layernorm_fwd_f64(x_bits, w_bits, b_bits, eps, dtype), dtype)


def l2norm_fwd_f64(x_bits, eps: float, dtype: str = "bf16") -> np.ndarray:
    x = widen(x_bits, dtype)
    if x.ndim != 2:
        raise ValueError("expected x [M, N]")
    if x.size == 0:
        return np.zeros(x.shape)
    eps64 = float(np.float32(eps))
    with np.errstate(all="ignore"):
        nrm = np.sqrt(np.sum(x * x, axis=1))
        return x / np.maximum(nrm, eps64)[:, None]


def l2norm_fwd(x_bits, eps: float, dtype: str = "bf16") -> np.ndarray:
    """Row-wise x / max(||x||_2, eps) of x [M, N]; 16-bit patterns of ``dtype`` out."""
    return narrow(l2norm_fwd_f64(x_bits, eps, dtype), dtype)
