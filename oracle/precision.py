"""Exact conversions between bfloat16 bit patterns and float64 for the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

bfloat16 is the upper half of an IEEE-754 binary32 word: 1 sign bit, 8 exponent
bits and 7 fraction bits.  Decoding is exact: place the 16 bits in the top half
of a 32-bit word, read it as binary32 and widen to float64.

Encoding is needed only for the merged value vectors, which the SelKV page
(section 2, "Selective merging") produces as cache entries and which this
project stores in bf16.  It rounds the float64 value to the nearest bf16,
ties to even, in one step (no intermediate float32 rounding).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns (any shape) -> float64 values, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits) -> np.ndarray:
    """uint32 binary32 bit patterns -> float64 values, exactly."""
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> uint16 bf16 bit patterns, round to nearest, ties to even.

    A finite nonzero x is m * 2**e with 0.5 <= |m| < 1 (``np.frexp``).  bf16 keeps
    8 significant bits, so the spacing of bf16 numbers near x is 2**(e - 8); below
    the smallest normal (2**-126, i.e. e = -125) the spacing stays 2**-133.
    Dividing by the spacing gives a number whose nearest integer (ties to even,
    ``np.rint``) times the spacing is the rounded value.  That value has at most
    8 significant bits and an exponent inside binary32 range, so it is exactly a
    binary32 whose low 16 bits are zero; its top 16 bits are the answer.
    Magnitudes that round above the largest finite bf16 become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[finite])
    e = np.maximum(e, -125)
    spacing = np.ldexp(1.0, e - 8)
    out[finite] = np.rint(x[finite] / spacing) * spacing
    out[~finite] = x[~finite]
    max_bf16 = float(np.uint32(0x7F7F0000).view(np.float32))
    big = np.abs(out) > max_bf16
    out[big] = np.copysign(np.inf, out[big])
    f32 = out.astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
