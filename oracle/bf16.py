"""Exact conversions between float64 and bf16 (round to nearest, ties to even).

bf16 keeps float32's 8-bit exponent and 7 of its 23 mantissa bits.  Rounding a
float64 straight to bf16 must not pass through a round-to-nearest float32
(double rounding), so the float32 intermediate is rounded to odd: truncated
toward zero, with the lowest mantissa bit set when anything was discarded.
Rounding-to-odd into a format with at least two more bits than the target,
then rounding to nearest even, equals a single correct rounding.
"""
from __future__ import annotations

import numpy as np


def to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def from_f64(x) -> np.ndarray:
    """float64 values -> bf16 bit patterns, one correct rounding to nearest-even."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        f = x.astype(np.float32)
        back = f.astype(np.float64)
        away = np.abs(back) > np.abs(x)
        t = np.where(away, np.nextafter(f, np.float32(0.0)), f).astype(np.float32)
        inexact = t.astype(np.float64) != x
    u = np.ascontiguousarray(t).view(np.uint32).astype(np.uint64)
    u = u | inexact.astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    inf = np.isinf(x)
    if inf.any():
        r = np.where(inf, np.where(x > 0, np.uint16(0x7F80), np.uint16(0xFF80)), r)
    return r
