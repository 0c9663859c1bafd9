"""Decode the exact input bits handed to both sides into float64.

bf16 bits are the upper half of a float32: widening (u16 << 16) to float32 and
then to float64 is exact. float32 inputs widen exactly to float64.
Pinned by tests/test_oracle_pins.py::test_decode_bf16_exact (hand-checked bit
patterns).
"""

import numpy as np


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
