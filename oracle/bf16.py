"""Exact bf16 bit-pattern conversions for the oracle (test infrastructure only).

A bf16 value is the upper 16 bits of an IEEE-754 binary32 value, so widening is
exact: shift the pattern into the high half of a 32-bit word and read it as a
float32, which float64 then represents exactly.  The narrowing direction rounds
to nearest, ties to even, and is used only to build test inputs and to express
expected outputs in bf16 units.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 array of bf16 patterns -> float64 array (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 array -> uint16 bf16 patterns, round to nearest even via float32.

    Values are first rounded to float32 (exact for the small integers and
    dyadic fractions the tests use), then the low 16 bits are rounded away.
    NaN inputs are not expected and not handled specially.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)
