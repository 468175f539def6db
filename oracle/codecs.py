"""Block codecs of the packed KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources.  The BeeLlama.cpp v0.4.0 release notes (section on the new standard
KV cache types) name the codec family this library stores: the ``_0`` and
``_1`` types at 2, 3, 4, 5, 6 and 8 bits, with q6_0/q6_1 filling the gap
between the existing 5- and 8-bit types and q2/q3 serving as the extreme
low-bit options.  The KV-COBRA explainer (Jargon, "scalar quantization")
describes scalar quantization as rounding every stored number to one of 2^b
levels.  Neither page prints the block format, so the readings below are
taken (and listed with the design notes):

* A block is 32 consecutive channels of one token of one (batch, kv-head);
  the low-rank basis uses blocks of ``min(32, rank)``.
* ``_0`` (absmax, signed): ``d = RN16(amax / qmax)`` with
  ``qmax = 2^(b-1) - 1``; codes ``q = clamp(rne(x / d), -qmax, qmax)``
  (the code -2^(b-1) is never produced, so every element obeys
  ``|x - q d| <= d / 2``); ``d == 0`` gives all-zero codes; decode ``q d``.
* ``_1`` (min-offset, unsigned): ``m = RN16(min x)``;
  ``y = RN32(x - m)``; ``R = RN32(max x - m)``; ``d = RN16(R / (2^b - 1))``;
  ``u = clamp(rne(y / d), 0, 2^b - 1)``; ``d == 0`` gives all-zero codes;
  decode ``RN32(u d + m)`` (single rounding).  The RN32 steps are part of the
  definition so that a binary32 device can reproduce the codes exactly.
* F16: ``RN16(x)``.

All quotients are exact (fp64 division of binary32/binary16 operands cannot
land on a rounding tie it does not exactly equal, see the test pins).
"""

import numpy as np

from .rounding import rn16, rn32, rne

# name -> (family, bits).  family: "f16", "0" (absmax, signed) or "1"
# (min-offset, unsigned).
CODECS = {
    "f16": ("f16", 16),
    "q8_0": ("0", 8),
    "q6_0": ("0", 6),
    "q5_0": ("0", 5),
    "q4_0": ("0", 4),
    "q3_0": ("0", 3),
    "q2_0": ("0", 2),
    "q8_1": ("1", 8),
    "q6_1": ("1", 6),
    "q5_1": ("1", 5),
    "q4_1": ("1", 4),
    "q3_1": ("1", 3),
    "q2_1": ("1", 2),
    "q1_1": ("1", 1),
}


def family(codec):
    return CODECS[codec][0]


def bits(codec):
    return CODECS[codec][1]


def qmax_0(b):
    """Largest magnitude of a signed ``_0`` code (symmetric levels)."""
    if b < 2:
        raise ValueError("a _0 codec needs at least 2 bits")
    return 2 ** (b - 1) - 1


def levels_1(b):
    """Largest unsigned ``_1`` code, 2^b - 1."""
    return 2 ** b - 1


def encode_0(x, b):
    """Absmax block quantiser.  ``x``: [..., L] (one block on the last axis).

    Returns ``(d, q)``: binary16 scales [...] and int64 codes [..., L].
    """
    x = np.asarray(x, dtype=np.float64)
    qm = qmax_0(b)
    amax = np.max(np.abs(x), axis=-1)
    d = rn16(amax / qm)
    dd = d.astype(np.float64)[..., None]
    safe = np.where(dd == 0.0, 1.0, dd)
    q = np.clip(rne(x / safe), -qm, qm)
    q = np.where(dd == 0.0, 0.0, q)
    return d, q.astype(np.int64)


def decode_0(d, q):
    """``q * d`` (exact in fp64 and in binary32)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(d, dtype=np.float64)[..., None]


def encode_1(x, b):
    """Min-offset block quantiser.  Returns ``(d, m, u)``."""
    x = np.asarray(x, dtype=np.float64)
    L = levels_1(b)
    m = rn16(np.min(x, axis=-1))
    mm = m.astype(np.float64)
    y = rn32(x - mm[..., None]).astype(np.float64)
    R = rn32(np.max(x, axis=-1) - mm).astype(np.float64)
    d = rn16(R / L)
    dd = d.astype(np.float64)[..., None]
    safe = np.where(dd == 0.0, 1.0, dd)
    u = np.clip(rne(y / safe), 0, L)
    u = np.where(dd == 0.0, 0.0, u)
    return d, m, u.astype(np.int64)


def decode_1(d, m, u, rounded=True):
    """``u d + m``; ``rounded`` applies the single RN32 of the definition."""
    exact = (np.asarray(u, dtype=np.float64) * np.asarray(d, dtype=np.float64)[..., None]
             + np.asarray(m, dtype=np.float64)[..., None])
    return rn32(exact).astype(np.float64) if rounded else exact


def encode_rows(x, codec, block_len=32):
    """Encode rows ``x``: [..., n] block by block.

    Returns a dict with ``codes`` (int64 [..., n]), ``scales`` and ``mins``
    (float16 [..., n // block_len]; ``mins`` is None for ``_0``), or
    ``values`` (float16 [..., n]) for F16.
    """
    fam, b = CODECS[codec]
    x = np.asarray(x, dtype=np.float64)
    if fam == "f16":
        return {"values": rn16(x)}
    n = x.shape[-1]
    if n % block_len:
        raise ValueError("row length must be a multiple of the block length")
    xb = x.reshape(x.shape[:-1] + (n // block_len, block_len))
    if fam == "0":
        d, q = encode_0(xb, b)
        return {"codes": q.reshape(x.shape), "scales": d, "mins": None}
    d, m, u = encode_1(xb, b)
    return {"codes": u.reshape(x.shape), "scales": d, "mins": m}


def decode_rows(enc, codec, block_len=32, rounded=True):
    """Dequantise what ``encode_rows`` returned, as fp64 [..., n].

    ``rounded`` selects the binary32 value of a ``_1`` element (what a
    binary32 consumer reads); False gives the exact ``u d + m``.
    """
    fam, _ = CODECS[codec]
    if fam == "f16":
        return np.asarray(enc["values"], dtype=np.float64)
    q = np.asarray(enc["codes"])
    n = q.shape[-1]
    qb = q.reshape(q.shape[:-1] + (n // block_len, block_len))
    if fam == "0":
        out = decode_0(enc["scales"], qb)
    else:
        out = decode_1(enc["scales"], enc["mins"], qb, rounded=rounded)
    return out.reshape(q.shape)
