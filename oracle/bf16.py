"""bfloat16 <-> float64 for the oracle (test infrastructure only).

bfloat16 is the upper half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  Widening is therefore exact: put the 16 bits in the high
half of a 32-bit word, read it as binary32, and convert to binary64 (also exact).
"""

import numpy as np


def widen(bits):
    """Exact float64 value of an array of bf16 bit patterns (``numpy.uint16``)."""
    u16 = np.asarray(bits)
    if u16.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as numpy.uint16 bit patterns")
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16_bits(x):
    """Round float values to bf16 (round to nearest, ties to even); return uint16 bits.

    Used only to build exact bf16 test inputs in pure-NumPy tests.  The value is
    first rounded to binary32, then the low 16 bits are rounded away: add
    0x7FFF plus the lowest kept bit, then truncate.  NaN stays a quiet NaN.
    """
    f32 = np.asarray(x, dtype=np.float32)
    u32 = f32.view(np.uint32).astype(np.uint64)
    lsb = (u32 >> np.uint64(16)) & np.uint64(1)
    rounded = ((u32 + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f32)
    if np.any(nan):
        rounded = np.where(nan, ((u32 >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16), rounded)
    return rounded
