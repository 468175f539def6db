"""Rounding primitives the codec definitions are written in.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

RN16 and RN32 are IEEE-754 round-to-nearest, ties-to-even, to binary16 and
binary32, applied to the exact value of their (fp64) argument.  ``rne`` is the
nearest integer with ties to even.  The pages fix no tie rule; the IEEE
default is the reading taken.
"""

import numpy as np


def rn16(x):
    """Round fp64 values to binary16 (RNE), returned as ``np.float16``.

    NumPy converts float64 to float16 in one correctly rounded step (no
    intermediate binary32), which the CPU tests check against exact rational
    rounding.
    """
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def rn32(x):
    """Round fp64 values to binary32 (RNE), returned as ``np.float32``."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def rne(x):
    """Nearest integer, ties to even, as float64."""
    return np.rint(np.asarray(x, dtype=np.float64))


def f16_bits(x):
    """The 16-bit pattern of binary16 values, as uint16."""
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def f16_from_bits(bits):
    """binary16 values from their 16-bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16)
