"""Widening of stored fp16 / bf16 values to float64 (oracle side).

fp16 values are numpy float16 arrays.  bf16 values are uint16 bit patterns: a
bfloat16 is the upper half of a float32, so shifting the bits left by 16 and
reinterpreting as float32 is exact.

Test infrastructure only.  Pinned in tests/test_oracle_numerics.py against
torch's own float16/bfloat16 conversions on all 65,536 bit patterns and
against closed forms of the two formats (a shift by 15 instead of 16 fails).
"""

import numpy as np


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        assert x.dtype == np.float16, x.dtype
        return x.astype(np.float64)
    if dtype == "bf16":
        assert x.dtype == np.uint16, x.dtype
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)
