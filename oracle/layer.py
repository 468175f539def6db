"""One layer's packed cache: append, precision tail, dequantisation, decode,
transcode.  Built only from the other oracle modules.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources and readings:

* Precision tail (BeeLlama v0.4.0 release notes, section on the KV cache
  precision tail): the newest ``N`` tokens are kept at 16-bit precision and
  older ones quantised.  Reading: the tail is F16 in the raw basis, a ring
  where token ``t`` lives in slot ``t mod N``; body codes are written for
  every appended token from its binary32 input (quantise at append), so codes
  never depend on ``N``.  Decode reads token ``t`` from the tail when
  ``t >= T - N`` and from the body otherwise.
* Per-layer codecs and degrade steps (VBR announcement thread, opening
  posts): a layer's cache can be re-encoded to a lower-precision codec as the
  session grows.  Reading: transcode decodes every body row with the source
  codec (binary32 value for ``_1``, the binary16 value for F16) and encodes it
  with the destination codec in the same basis; the tail is untouched.
* Separate K and V codecs (VBR thread, asymmetric ``-ctk``/``-ctv``): each of
  K and V has its own plane description.
"""

from dataclasses import dataclass, field

import numpy as np

from . import attention, cobra, kvarn
from .codecs import CODECS, decode_rows, encode_rows
from .layout import pack_rows, row_bytes, tile_plane, unpack_rows, untile_plane
from .rounding import bf16_bits, f16_bits, f16_from_bits, rbf16, rn16

D = 128


@dataclass
class PlaneSpec:
    """How one of K or V is stored in one layer."""
    codec: str = "q8_0"                  # plain / hadamard bases
    basis: str = "plain"                 # "plain" | "hadamard" | "lowrank"
    w: np.ndarray = None                 # hadamard: [Hkv, 128] binary32, 1/sigma
    P: list = field(default=None)        # lowrank: per head binary16 [128, r_h]
    head_codec: list = field(default=None)  # lowrank: per head codec name

    def codec_of(self, h):
        return self.head_codec[h] if self.basis == "lowrank" else self.codec

    def width(self, h):
        return self.P[h].shape[1] if self.basis == "lowrank" else D

    def block_len(self, h):
        return cobra.block_len(self.width(h)) if self.basis == "lowrank" else 32


def stored_coords(x, spec, h):
    """The coordinates a plane stores for raw vectors ``x``: [..., 128]."""
    if spec.basis == "plain":
        return np.asarray(x, dtype=np.float64)
    if spec.basis == "hadamard":
        return kvarn.rotate(x, spec.w[h])
    if spec.basis == "lowrank":
        return cobra.project(x, spec.P[h])
    raise ValueError(spec.basis)


def to_raw(coords, spec, h):
    """Raw-basis vectors for stored coordinates (exact fp64)."""
    if spec.basis == "plain":
        return np.asarray(coords, dtype=np.float64)
    if spec.basis == "hadamard":
        return kvarn.unrotate(coords, spec.w[h])
    if spec.basis == "lowrank":
        return cobra.reconstruct(coords, spec.P[h])
    raise ValueError(spec.basis)


def encode_head(x, spec, h):
    """Encode raw vectors x: [T, 128] of kv head ``h``."""
    return encode_rows(stored_coords(x, spec, h), spec.codec_of(h), spec.block_len(h))


def encode_plane(x, spec):
    """x: [B, T, Hkv, 128] binary32 -> per (b, h) encodings, list[B][Hkv]."""
    x = np.asarray(x)
    B, _, Hkv, _ = x.shape
    return [[encode_head(x[b, :, h, :], spec, h) for h in range(Hkv)] for b in range(B)]


def dequant_head(enc, spec, h, exact=True):
    """Raw-basis fp64 reconstructions [T, 128] of one head's rows.

    ``exact`` uses ``u d + m`` without the binary32 rounding of ``_1``.
    """
    vals = decode_rows(enc, spec.codec_of(h), spec.block_len(h), rounded=not exact)
    return to_raw(vals, spec, h)


def tail_ring(x, N, fmt="f16"):
    """The tail ring after appending tokens 0..T-1 of x: [B, T, Hkv, 128].

    Returns [B, Hkv, N, 128]: binary16 values (fmt "f16"), or bfloat16 values
    held as float32 (fmt "bf16"); slots never written hold zeros.
    """
    x = np.asarray(x)
    B, T, Hkv, _ = x.shape
    rnd = {"f16": rn16, "bf16": lambda y: rbf16(y).astype(np.float32)}[fmt]
    ring = np.zeros((B, Hkv, N, D), dtype=np.float16 if fmt == "f16" else np.float32)
    for t in range(T):
        ring[:, :, t % N, :] = rnd(x[:, t, :, :])
    return ring


def attention_kv(enc_planes, tail, spec, T, N):
    """fp64 raw-basis cache [B, T, Hkv, 128] that decode attends over."""
    B, Hkv = len(enc_planes), len(enc_planes[0])
    out = np.empty((B, T, Hkv, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hkv):
            out[b, :, h, :] = dequant_head(enc_planes[b][h], spec, h)[:T]
    if N > 0:
        for t in range(max(0, T - N), T):
            out[:, t, :, :] = tail[:, :, t % N, :].astype(np.float64)
    return out


def decode(q, kenc, venc, ktail, vtail, kspec, vspec, T, N, sm_scale):
    """Decode attention of q: [B, Hq, 128] over the first T tokens."""
    K = attention_kv(kenc, ktail, kspec, T, N)
    V = attention_kv(venc, vtail, vspec, T, N)
    return attention.attend_batch(q, K, V, sm_scale)


def transcode_head(enc, src, dst, h):
    """Re-encode one head's rows with ``dst``'s codec, same basis."""
    vals = decode_rows(enc, src.codec_of(h), src.block_len(h), rounded=True)
    return encode_rows(vals, dst.codec_of(h), dst.block_len(h))


def transcode_plane(enc_planes, src, dst):
    return [[transcode_head(e, src, dst, h) for h, e in enumerate(row)] for row in enc_planes]


# ----------------------------------------------------------------- bytes --

def head_row_bytes(spec, h):
    return row_bytes(spec.codec_of(h), spec.width(h))


def head_nblk(spec, h):
    return spec.width(h) // spec.block_len(h)


def pack_plane(enc_planes, spec, capacity):
    """Device bytes of a plane: dict with ``codes`` (uint8), ``scales`` and
    ``mins`` (uint16 binary16 patterns, or None).

    Planes follow (batch, kv head) order, each ``capacity`` rows long; rows
    beyond the encoded ones are zero.
    """
    codes, scales, mins = [], [], []
    fam1 = False
    for row in enc_planes:
        for h, enc in enumerate(row):
            codec = spec.codec_of(h)
            R = head_row_bytes(spec, h)
            rows = np.zeros((capacity, R), dtype=np.uint8)
            packed = pack_rows(enc, codec, spec.block_len(h))
            rows[: packed.shape[0]] = packed
            codes.append(tile_plane(rows))
            if CODECS[codec][0] == "f16":
                continue
            nb = head_nblk(spec, h)
            s = np.zeros((capacity, nb), dtype=np.uint16)
            s[: enc["scales"].shape[0]] = f16_bits(enc["scales"])
            scales.append(s.reshape(-1))
            if enc["mins"] is not None:
                fam1 = True
                m = np.zeros((capacity, nb), dtype=np.uint16)
                m[: enc["mins"].shape[0]] = f16_bits(enc["mins"])
                mins.append(m.reshape(-1))
    return {
        "codes": np.concatenate(codes),
        "scales": np.concatenate(scales) if scales else None,
        "mins": np.concatenate(mins) if fam1 else None,
    }


def unpack_plane(buf, spec, B, Hkv, capacity, T):
    """Inverse of ``pack_plane`` for the first T rows of every (b, h)."""
    out = []
    co = so = 0
    for b in range(B):
        row = []
        for h in range(Hkv):
            codec = spec.codec_of(h)
            R = head_row_bytes(spec, h)
            rows = untile_plane(buf["codes"][co: co + capacity * R], R)[:T]
            co += capacity * R
            vals = unpack_rows(rows, codec, spec.width(h), spec.block_len(h))
            if CODECS[codec][0] == "f16":
                row.append({"values": vals})
                continue
            nb = head_nblk(spec, h)
            s = f16_from_bits(buf["scales"][so: so + capacity * nb].reshape(capacity, nb)[:T])
            m = None
            if buf.get("mins") is not None and CODECS[codec][0] == "1":
                m = f16_from_bits(buf["mins"][so: so + capacity * nb].reshape(capacity, nb)[:T])
            so += capacity * nb
            row.append({"codes": vals, "scales": s, "mins": m})
        out.append(row)
    return out


def pack_tail(ring, fmt="f16"):
    """Device bytes of a tail ring [B, Hkv, N, 128] (``tail_ring``'s output):
    256-byte rows of 16-bit values in the tiled layout."""
    B, Hkv, N, _ = ring.shape
    planes = []
    for b in range(B):
        for h in range(Hkv):
            if fmt == "f16":
                rows = pack_rows({"values": ring[b, h]}, "f16")
            else:
                bits = np.ascontiguousarray(bf16_bits(ring[b, h]))
                rows = bits.view(np.uint8).reshape(N, 2 * D)
            planes.append(tile_plane(rows))
    return np.concatenate(planes) if planes else np.zeros(0, np.uint8)


def unpack_tail(buf, B, Hkv, N):
    out = np.empty((B, Hkv, N, D), dtype=np.float16)
    per = N * 2 * D
    for b in range(B):
        for h in range(Hkv):
            i = b * Hkv + h
            rows = untile_plane(buf[i * per: (i + 1) * per], 2 * D)
            out[b, h] = unpack_rows(rows, "f16", D)
    return out
