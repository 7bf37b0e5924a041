"""bfloat16 bit patterns -> float64.  TEST INFRASTRUCTURE ONLY.

bf16 tensors travel through numpy as uint16 bit patterns (numpy has no bf16
type).  A bf16 value is the upper half of an IEEE binary32, so widening is a
16-bit shift; every bf16 value is exactly representable in float64.
"""
from __future__ import annotations

import numpy as np


def to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
