"""bf16 <-> float64 conversions of the oracle (test infrastructure only).

bf16 keeps the float32 sign and 8-bit exponent and 7 stored fraction bits, so a
bf16 bit pattern b is the float32 whose bits are b << 16. Widening is therefore
exact. Narrowing rounds a float64 value once, to nearest with ties to even,
which is the rounding the pages' kernels apply when they store the bf16 output
("[Inductor] Codegen Gluon", section 3.1: values are kept as bf16 and converted
to fp32 only where they are computed on).
"""

from __future__ import annotations

import numpy as np

_BF16_NAN = np.uint16(0x7FC0)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of each bf16 bit pattern, as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(y) -> np.ndarray:
    """Round float64 values once to bf16 (nearest, ties to even); return uint16 bits.

    A normal bf16 has 8 significant bits, so for |y| = m * 2**e with m in
    [0.5, 1) the spacing of bf16 values is 2**(e - 8). Below the smallest normal
    (2**-126) the spacing stays at 2**-133 (subnormals). Scaling by a power of
    two is exact in float64, so ``rint`` (ties to even) of the scaled value is
    the one rounding step. Results of magnitude 2**128 or more overflow to
    infinity; NaN maps to the quiet NaN 0x7FC0; the sign of zero is kept.
    """
    y = np.asarray(y, dtype=np.float64)
    with np.errstate(all="ignore"):
        _, e = np.frexp(y)
        qexp = np.maximum(e - 8, -133)
        r = np.ldexp(np.rint(np.ldexp(y, -qexp)), qexp)
        r = np.where(np.abs(r) >= 2.0**128, np.copysign(np.inf, y), r)
        r = np.where(np.isinf(y), y, r)
        # r is now exactly representable in bf16, hence in float32
        bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(y), _BF16_NAN, bits)


# ---------------------------------------------------------------------------
# IEEE binary16 (fp16): 1 sign, 5 exponent, 10 fraction bits. Used for the fp16
# variants of the operators (bf16 is the primary storage format).

_F16_NAN = np.uint16(0x7E00)


def f16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of each fp16 bit pattern, as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return b.view(np.float16).astype(np.float64)


def f64_to_f16_bits(y) -> np.ndarray:
    """Round float64 values once to fp16 (nearest, ties to even); return uint16 bits.

    A normal fp16 has 11 significant bits, so for |y| = m * 2**e (m in
    [0.5, 1)) the spacing is 2**(e - 11); below the smallest normal (2**-14) it
    stays 2**-24. Results of magnitude 2**16 or more after rounding overflow to
    infinity (the largest finite value is 65504).
    """
    y = np.asarray(y, dtype=np.float64)
    with np.errstate(all="ignore"):
        _, e = np.frexp(y)
        qexp = np.maximum(e - 11, -24)
        r = np.ldexp(np.rint(np.ldexp(y, -qexp)), qexp)
        r = np.where(np.abs(r) >= 2.0**16, np.copysign(np.inf, y), r)
        r = np.where(np.isinf(y), y, r)
        bits = r.astype(np.float16).view(np.uint16)  # exact: r is representable
    return np.where(np.isnan(y), _F16_NAN, bits)


def widen(bits, dtype: str = "bf16") -> np.ndarray:
    """Exact float64 values of 16-bit patterns of the given storage type."""
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def narrow(y, dtype: str = "bf16") -> np.ndarray:
    """One round-to-nearest-even of float64 values to the given storage type."""
    if dtype == "bf16":
        return f64_to_bf16_bits(y)
    if dtype == "f16":
        return f64_to_f16_bits(y)
    raise ValueError(f"unknown dtype {dtype!r}")
