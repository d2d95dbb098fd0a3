"""Exact widening of stored element types to float64 (oracle side).

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

BF16 is the top half of an IEEE-754 binary32: the 16 stored bits are the sign,
the 8 exponent bits and the 7 leading mantissa bits. Shifting them into the
high half of a 32-bit word gives the binary32 with the same value, and
binary32 -> binary64 is exact, so the widening below loses nothing. The pages
name BF16 as the cache precision ("b is the precision in bytes, e.g. 2 bytes
for BF16": High-Throughput LLM Inference & Training, KV-footprint paragraph).

Arrays holding BF16 are carried as ``numpy.uint16`` bit patterns so that the
oracle and the device agree bit for bit on what was stored.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Widen an array of BF16 bit patterns (uint16) to float64, exactly."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"expected uint16 BF16 bit patterns, got {bits.dtype}")
    as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return as_f32.astype(np.float64)


def to_f64(x):
    """Widen a stored tensor (uint16 BF16 bits, float32 or float64) to float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported element type {x.dtype}")
