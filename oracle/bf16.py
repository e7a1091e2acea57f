"""Exact widening of bfloat16 bit patterns to float64 (oracle; test infrastructure only).

A bfloat16 value is the upper 16 bits of an IEEE-754 binary32 value, so placing the 16
bits in the high half of a 32-bit word and reinterpreting it as float32 gives the value
exactly; float32 -> float64 is exact too.
"""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 values (exact)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"expected uint16 bfloat16 bits, got {bits.dtype}")
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
