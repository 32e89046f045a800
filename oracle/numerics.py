"""Bit-level number helpers for the CPU oracle.

TEST INFRASTRUCTURE ONLY: nothing on the product path may import this module.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use the oracle.

bfloat16 values are carried as ``numpy.uint16`` arrays holding the bit
pattern, because NumPy has no bfloat16 type.  The conversions are written from
the format's definition: bfloat16 is the upper 16 bits of an IEEE-754 binary32
(1 sign, 8 exponent, 7 fraction bits), so widening is a 16-bit left shift and
narrowing rounds the dropped 16 bits to nearest, ties to even.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32.  Exact for every input."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even, as bit patterns.

    Finite values and infinities: add 0x7FFF plus the lowest kept bit to the
    binary32 pattern and keep the top 16 bits.  A carry out of the fraction
    moves into the exponent, which is the correct rounding up to the next
    binade and to infinity on overflow.  NaN keeps its sign and top fraction
    bits with the quiet bit set, so it stays a NaN after truncation.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    # For every non-NaN pattern (at most 0xFF800000) the sum below stays
    # under 2^32; NaN patterns, where it may wrap, take the other branch.
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    quiet_nan = (u >> np.uint32(16)) | np.uint32(0x0040)
    return np.where(is_nan, quiet_nan, rounded).astype(np.uint16)
