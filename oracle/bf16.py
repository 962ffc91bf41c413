"""bfloat16 <-> float32 conversions of the oracle (test infrastructure only).

bf16 values are carried as ``numpy.uint16`` bit patterns.  A bf16 number is
the upper half of an IEEE-754 binary32 number: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  The hidden states and expert outputs of
[DeepEP-TMA] section "High-Level DeepEP API Usage" are bf16 rows; combine
accumulates in fp32 and rounds once to bf16.

* ``bf16_to_f32`` is exact: shift the 16 bits into the high half of a
  binary32 word.
* ``f32_to_bf16_rne`` rounds to nearest, ties to even, on the 16 bits that
  are dropped.  NaN stays NaN (quiet bit forced on so that rounding can never
  turn a NaN payload into infinity); overflow of the largest finite values
  rounds to +-inf as IEEE round-to-nearest does.
"""

import numpy as np


def bf16_to_f32(h):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(f):
    """float32 values -> uint16 bf16 bit patterns, round to nearest even."""
    f = np.asarray(f, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)  # room for the carry out of bit 31
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1  # parity of the bit that survives
    rounded = (u + 0x7FFF + lsb) >> 16
    quiet_nan = (u >> 16) | 0x0040
    out = np.where(is_nan, quiet_nan, rounded)
    return out.astype(np.uint16)
