"""Exact bf16 -> float64 decoding (test infrastructure only).

A bf16 value is the upper 16 bits of an IEEE-754 binary32 word, so widening
the bit pattern by 16 zero bits gives the float32 value exactly, and float32
widens to float64 exactly.
"""
import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """Inputs as float64: uint16 arrays are bf16 bit patterns, floats widen."""
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return np.asarray(x, dtype=np.float64)
