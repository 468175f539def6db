"""Byte layout of a cache plane in device memory.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

This is the storage format the library defines (the pages leave it open):

* A *row* holds one token of one (batch, kv-head): its blocks' code fields
  back to back (``n*b/8`` bytes for ``n`` channels), or ``n`` binary16 values
  (``2n`` bytes) for F16.
* A *plane* holds ``capacity`` rows (capacity a multiple of 64).  Rows are
  grouped in tiles of 64 tokens; a row is cut into ``c``-byte chunks, ``c``
  the largest of 16, 8, 4, 2, 1 dividing the row size, and a tile stores
  chunk ``k`` of its 64 tokens next to each other.  The chunk ``k`` of token
  ``t`` sits at byte ``(t // 64) * 64 * R + (k * 64 + t % 64) * c`` for row
  size ``R``.
* Scales and mins are binary16, token-major: ``[capacity][n_blocks]``.
"""

import numpy as np

from .bitpack import pack_codes, unpack_codes
from .codecs import CODECS

TILE = 64


def row_bytes(codec, n):
    fam, b = CODECS[codec]
    if fam == "f16":
        return 2 * n
    if (n * b) % 8:
        raise ValueError("row is not a whole number of bytes")
    return n * b // 8


def chunk_bytes(rbytes):
    for c in (16, 8, 4, 2, 1):
        if rbytes % c == 0:
            return c
    raise AssertionError


def pack_rows(enc, codec, block_len=32):
    """Rows of bytes [..., R] for what ``codecs.encode_rows`` returned."""
    fam, b = CODECS[codec]
    if fam == "f16":
        v = np.ascontiguousarray(np.asarray(enc["values"], dtype=np.float16))
        return v.view(np.uint8).reshape(v.shape[:-1] + (2 * v.shape[-1],))
    q = np.asarray(enc["codes"])
    n = q.shape[-1]
    qb = q.reshape(q.shape[:-1] + (n // block_len, block_len))
    packed = pack_codes(qb, b, signed=(fam == "0"))        # [..., nblk, L*b/8]
    return packed.reshape(q.shape[:-1] + (n * b // 8,))


def unpack_rows(rows, codec, n, block_len=32):
    """Inverse of ``pack_rows``: codes int64 [..., n] (or float16 values)."""
    fam, b = CODECS[codec]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.uint8))
    if fam == "f16":
        return rows.view(np.float16).reshape(rows.shape[:-1] + (n,))
    fb = block_len * b // 8
    blocks = rows.reshape(rows.shape[:-1] + (n // block_len, fb))
    q = unpack_codes(blocks, b, block_len, signed=(fam == "0"))
    return q.reshape(rows.shape[:-1] + (n,))


def tile_plane(rows):
    """rows uint8 [capacity, R] -> the plane's bytes, uint8 [capacity * R]."""
    rows = np.asarray(rows, dtype=np.uint8)
    cap, R = rows.shape
    if cap % TILE:
        raise ValueError("capacity must be a multiple of 64")
    c = chunk_bytes(R)
    out = np.empty(cap * R, dtype=np.uint8)
    t = np.arange(cap)
    for k in range(R // c):
        for j in range(c):
            off = (t // TILE) * TILE * R + (k * TILE + t % TILE) * c + j
            out[off] = rows[:, k * c + j]
    return out


def untile_plane(plane, R):
    """Inverse of ``tile_plane``: uint8 [capacity * R] -> rows [capacity, R]."""
    plane = np.asarray(plane, dtype=np.uint8)
    cap = plane.size // R
    c = chunk_bytes(R)
    rows = np.empty((cap, R), dtype=np.uint8)
    t = np.arange(cap)
    for k in range(R // c):
        for j in range(c):
            off = (t // TILE) * TILE * R + (k * TILE + t % TILE) * c + j
            rows[:, k * c + j] = plane[off]
    return rows
