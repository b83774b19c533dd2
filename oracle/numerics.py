"""Exact widening of stored element bits to float64.

bfloat16 is the upper half of an IEEE-754 binary32: its 16 bits, shifted left
by 16, are the bits of a float32 of the same value.  Every float32 (hence
every bfloat16) is exactly representable in float64, so the widening is exact.
"""
import numpy as np

BITS_DTYPE = {"bf16": np.uint16, "f32": np.uint32}
ELT_BYTES = {"bf16": 2, "f32": 4}


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Values of stored elements, given as their raw bits, in float64."""
    if dtype == "bf16":
        assert bits.dtype == np.uint16
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        assert bits.dtype == np.uint32
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)
