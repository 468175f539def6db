"""b-bit code packing inside one block's code field.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Reading (the pages print no bit layout): the code field of a block of ``L``
elements at ``b`` bits is ``L*b/8`` bytes read as one little-endian integer;
element ``i`` occupies bits ``[i*b, i*b + b)``.  ``_0`` codes are stored as
b-bit two's complement, ``_1`` codes as unsigned integers.
"""

import numpy as np


def pack_codes(codes, b, signed):
    """Pack int codes [..., L] into uint8 [..., L*b/8] (LSB-first bits)."""
    codes = np.asarray(codes, dtype=np.int64)
    L = codes.shape[-1]
    if (L * b) % 8:
        raise ValueError("block code field must be a whole number of bytes")
    if signed:
        lo, hi = -(2 ** (b - 1)), 2 ** (b - 1) - 1
    else:
        lo, hi = 0, 2 ** b - 1
    if codes.size and (codes.min() < lo or codes.max() > hi):
        raise ValueError("code out of range for %d bits" % b)
    u = codes & ((1 << b) - 1)                       # two's complement field
    bit = (u[..., None] >> np.arange(b)) & 1         # [..., L, b], bit k of element i
    flat = bit.reshape(codes.shape[:-1] + (L * b,)).astype(np.uint8)
    return np.packbits(flat, axis=-1, bitorder="little")


def unpack_codes(packed, b, L, signed):
    """Inverse of ``pack_codes``: uint8 [..., L*b/8] -> int64 [..., L]."""
    packed = np.asarray(packed, dtype=np.uint8)
    flat = np.unpackbits(packed, axis=-1, bitorder="little")[..., : L * b]
    bit = flat.reshape(packed.shape[:-1] + (L, b)).astype(np.int64)
    u = np.sum(bit << np.arange(b), axis=-1)
    if signed:
        u = np.where(u >= 2 ** (b - 1), u - 2 ** b, u)
    return u
