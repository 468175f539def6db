"""Rounding primitives the codec definitions are written in.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

RN16 and RN32 are IEEE-754 round-to-nearest, ties-to-even, to binary16 and
binary32, applied to the exact value of their (fp64) argument; RBF16 is the
same rounding to bfloat16 (8 significant bits, binary32's exponent range),
the other precision-tail format the BeeLlama.cpp v0.4.0 release notes name.  ``rne`` is the
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


def rbf16(x):
    """Round fp64 values to bfloat16 (RNE) from their exact value; returns
    the rounded values as float64.  With x = m 2^e, 1/2 <= |m| < 1, the
    quantum is 2^(e - 8) (8 significant bits), never below 2^-133 (the
    subnormal quantum of the binary32 exponent range)."""
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(x)
    quantum = np.ldexp(1.0, np.maximum(ex - 8, -133))
    return rne(x / quantum) * quantum


def bf16_bits(values):
    """16-bit patterns of bfloat16 values (as returned by ``rbf16``): the high
    half of their binary32 encoding, exact since they have <= 8 significant
    bits."""
    v = np.asarray(values, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)
