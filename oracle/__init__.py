"""CPU oracle for the normalization hot path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct reference that the HIP
kernels are checked against. It is not part of the product: only the test
suite, the smoke check of the package entry point and the CPU-baseline leg of
the benchmark may import it. The product library never calls it and has no CPU
fallback.

Everything is computed in float64 from the exact bf16 input values and rounded
once to bf16 (round to nearest, ties to even) at the end:

* ``rmsnorm_fwd``       -- row-wise RMSNorm, y = x / sqrt(mean(x^2) + eps) * w
  ("[Inductor] Codegen Gluon", section 3.1, the RMSNorm reference workload:
  a sum of x squared, then x scaled by rstd and the weight).
* ``add_rmsnorm_fwd``, ``layernorm_fwd``, ``l2norm_fwd`` -- the rest of the
  reused-input norm family (see ``oracle/norms.py`` for sources and readings).
* ``qk_norm_rope_fwd``  -- per-head RMSNorm with q/k weights followed by
  rotate-half (NeoX) rotary embedding on the q and k heads of a packed QKV
  tensor, in place, v heads untouched ("[pretuned] Optimize fused_qk_norm_rope
  on B200", Summary).

The oracle shares no code with the HIP path. It takes raw 16-bit patterns
(numpy ``uint16``; bf16 by default, fp16 with ``dtype="f16"``) and returns raw
16-bit patterns of the same type.
"""

from .bf16 import bf16_bits_to_f64, f16_bits_to_f64, f64_to_bf16_bits, f64_to_f16_bits, narrow, widen
from .rmsnorm import rmsnorm_fwd, rmsnorm_fwd_f64
from .norms import add_rmsnorm_fwd, l2norm_fwd, l2norm_fwd_f64, layernorm_fwd, layernorm_fwd_f64
from .qk_norm_rope import (
    qk_norm_rope_fwd,
    qk_norm_rope_fwd_f64,
    rope_inv_freq,
    rope_rotate_neox,
)

__all__ = [
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
    "f16_bits_to_f64",
    "f64_to_f16_bits",
    "narrow",
    "widen",
    "rmsnorm_fwd",
    "rmsnorm_fwd_f64",
    "add_rmsnorm_fwd",
    "layernorm_fwd",
    "layernorm_fwd_f64",
    "l2norm_fwd",
    "l2norm_fwd_f64",
    "qk_norm_rope_fwd",
    "qk_norm_rope_fwd_f64",
    "rope_inv_freq",
    "rope_rotate_neox",
]
