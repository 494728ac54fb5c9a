"""Exact widening of stored inputs to float64 (oracle side).

bfloat16 values arrive as their uint16 bit patterns.  A bfloat16 is the top
half of a float32, so shifting the bits up by 16 gives the float32 of the same
value, and float32 -> float64 is exact.  The oracle never sees the float32
draws that preceded rounding: it computes on exactly the stored values.
"""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen an input tensor stored as ``dtype`` ("bf16" bits or "f32") to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
