"""Exact conversions from the storage types to float64 (oracle side).

* float32 and float16 widen to float64 exactly.
* bfloat16 arrives as uint16 bit patterns; its value is the float32 whose top
  16 bits are those bits, so shifting left by 16 and reinterpreting is exact.
"""
from __future__ import annotations

import numpy as np


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        assert x.dtype == np.float32
        return x.astype(np.float64)
    if dtype == "f16":
        assert x.dtype == np.float16
        return x.astype(np.float64)
    if dtype == "bf16":
        assert x.dtype == np.uint16
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to binary16 once (nearest, ties to even); return bits.

    NumPy converts double to half directly from the double's bits, so there is
    a single rounding.
    """
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)
