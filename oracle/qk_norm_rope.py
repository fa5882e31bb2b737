"""Fused per-head QK RMSNorm + rotary embedding, plain definition in float64.

TEST INFRASTRUCTURE ONLY.

Source: "[pretuned] Optimize fused_qk_norm_rope on B200", Summary. For the
full-rotary case the operator takes the two rotary halves of each q/k head from
the packed QKV tensor, computes the RMS over the whole head, applies the Q or K
weight and then the rotary embedding, and writes each half back once, with no
intermediate round trip through memory.

Per token t with position p_t, and per head h among the n_q q heads (weight
q_w) and n_kv k heads (weight k_w), with D = head_dim and x = that head's D
values:

    rstd = 1 / sqrt(mean_d(x_d^2) + eps)
    u_d  = x_d * rstd * w_d                    (float64, not rounded)
    phi_i = p_t * theta^(-2i/D),  i in [0, D/2)
    o_i       = u_i       * cos(phi_i) - u_{i+D/2} * sin(phi_i)
    o_{i+D/2} = u_{i+D/2} * cos(phi_i) + u_i       * sin(phi_i)
    store bf16(o) in place of x (one rounding)

Readings where the page is silent (each listed in the design notes):
* The rotary formula is not written on the page; loading each head as its two
  rotary halves, with a NeoX-style rotary embedding, is read as the rotate-half pairing (i, i + D/2)
  with inverse frequencies theta^(-2i/D).
* One weight vector of length D per kind (q or k), shared by every head of that
  kind.
* Order: normalize, multiply by the weight, rotate; no bf16 rounding between
  the steps.
* Layout per token: [q_0 .. q_{n_q-1} | k_0 .. k_{n_kv-1} | v_0 .. v_{n_kv-1}],
  each head D contiguous values; the v heads are neither read nor written.
* eps and theta are taken as the float32 values the C interface receives.
* Partial rotary (rotary_dim R < D; the page keeps the full-head norm for it
  because the tail past the rotary part must still be normalized): the RMS and
  the weight cover all D values; the rotation acts on u[0:R] alone, pairing
  (i, i + R/2) with angles p_t * theta^(-2i/R); u[R:D] is stored unrotated.
"""

from __future__ import annotations

import numpy as np

from .bf16 import narrow, widen


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Inverse frequencies theta^(-2i/D) for i in [0, D/2), float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(theta) ** (-(2.0 * i) / head_dim)


def rope_rotate_neox(u: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of u [..., D] at positions ``pos`` (float64).

    ``pos`` broadcasts against u[..., 0]. Element i and element i + D/2 form one
    pair, rotated by the angle pos * theta^(-2i/D).
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    if d % 2:
        raise ValueError("head_dim must be even")
    half = d // 2
    phi = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(d, theta)
    c = np.cos(phi)
    s = np.sin(phi)
    a = u[..., :half]
    b = u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def qk_norm_rope_fwd_f64(
    qkv_bits, q_w_bits, k_w_bits, positions, n_q_heads: int, n_kv_heads: int,
    head_dim: int, eps: float, theta: float, rotary_dim: int | None = None, dtype: str = "bf16",
) -> np.ndarray:
    """Unrounded float64 outputs of the q and k heads, shape [T, n_q + n_kv, D]."""
    rot = head_dim if rotary_dim is None else rotary_dim
    if rot % 2 or not 0 < rot <= head_dim:
        raise ValueError("rotary_dim must be even and in (0, head_dim]")
    qkv_bits = np.asarray(qkv_bits, dtype=np.uint16)
    t = qkv_bits.shape[0]
    h = n_q_heads + n_kv_heads
    d = head_dim
    if qkv_bits.shape[1] != (n_q_heads + 2 * n_kv_heads) * d:
        raise ValueError("qkv row width does not match the head counts")
    x = widen(qkv_bits[:, : h * d], dtype).reshape(t, h, d)
    q_w = widen(q_w_bits, dtype)
    k_w = widen(k_w_bits, dtype)
    w = np.concatenate([np.tile(q_w, (n_q_heads, 1)), np.tile(k_w, (n_kv_heads, 1))], axis=0)
    eps64 = float(np.float32(eps))
    theta64 = float(np.float32(theta))
    pos = np.asarray(positions, dtype=np.int64).astype(np.float64)
    with np.errstate(all="ignore"):
        ms = np.mean(x * x, axis=-1)
        rstd = 1.0 / np.sqrt(ms + eps64)
        u = x * rstd[..., None] * w[None, :, :]
        rotated = rope_rotate_neox(u[..., :rot], pos[:, None], theta64)
        return np.concatenate([rotated, u[..., rot:]], axis=-1)


def qk_norm_rope_fwd(
    qkv_bits, q_w_bits, k_w_bits, positions, n_q_heads: int, n_kv_heads: int,
    head_dim: int, eps: float, theta: float, rotary_dim: int | None = None, dtype: str = "bf16",
) -> np.ndarray:
    """Return a copy of qkv (16-bit patterns) with q and k heads normalized and rotated.

    ``rotary_dim`` (default: head_dim) rotates only the first rotary_dim values
    of each head; the rest are normalized and weighted only.
    """
    qkv_bits = np.asarray(qkv_bits, dtype=np.uint16)
    t = qkv_bits.shape[0]
    h = n_q_heads + n_kv_heads
    o = qk_norm_rope_fwd_f64(
        qkv_bits, q_w_bits, k_w_bits, positions, n_q_heads, n_kv_heads, head_dim, eps, theta,
        rotary_dim, dtype,
    )
    out = qkv_bits.copy()
    out[:, : h * head_dim] = narrow(o, dtype).reshape(t, h * head_dim)
    return out
