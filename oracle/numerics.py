"""Storage rounding of the oracle (float64 -> bf16 / fp32), test infrastructure only.

bf16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits and
7 fraction bits, so a normal bf16 number carries 8 significant bits.  A value in
[2^(e-1), 2^e) is therefore a multiple of 2^(e-8); below the smallest normal
(2^-126) the spacing stays 2^-133.  Rounding is to nearest, ties to even.
The drafter stores its weights in BF16 ([FN] §3.1).
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each float64 (ties to even), as float64.

    Direct rounding from float64 (no intermediate fp32 step).  Finite inputs
    within the bf16 range only.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = m * 2**e with 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # subnormal range keeps spacing 2**-133
    q = np.ldexp(np.ones_like(x), e - 8)    # spacing of bf16 values around x
    return np.round(x / q) * q              # x / q is exact; np.round is half-to-even


def round_f32(x) -> np.ndarray:
    """Nearest fp32 value of each float64 (ties to even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_storage(x, dtype: str) -> np.ndarray:
    """Round to the storage type: "bf16", "f32", or "f64" (no rounding; used by
    the oracle's brute-force self-checks)."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage type {dtype!r}")


def bf16_bits(x) -> np.ndarray:
    """Bit patterns (uint16) of the bf16 values nearest to ``x``."""
    r = round_bf16(x).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def from_storage(a) -> np.ndarray:
    """Decode a stored tensor to float64: uint16 arrays are bf16 bit patterns,
    float arrays are taken as they are."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64, copy=False)
