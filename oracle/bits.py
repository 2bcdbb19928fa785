"""Exact conversions between stored element bits and float64 (oracle, test infrastructure).

bf16 is the upper half of an IEEE binary32 word, so widening a bf16 value to
float64 is exact: place the 16 bits in the high half of a 32-bit word and read
it as float32.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, to nearest with ties to even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored elements of ``dtype`` ("bf16" bits as uint16 / "f32") to float64."""
    a = np.asarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be given as uint16 bit patterns")
        return bf16_bits_to_f64(a)
    if dtype == "f32":
        if a.dtype == np.uint32:
            return a.view(np.float32).astype(np.float64)
        return a.astype(np.float64)
    raise ValueError(dtype)
