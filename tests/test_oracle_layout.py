"""Pins of oracle.bitpack / oracle.layout / oracle.budget: round trips,
hand-worked bit patterns and offsets, and the closed-form byte sizes."""

import numpy as np
import pytest

from oracle import budget
from oracle.bitpack import pack_codes, unpack_codes
from oracle.codecs import CODECS, encode_rows
from oracle.layout import (chunk_bytes, pack_rows, row_bytes, tile_plane, unpack_rows,
                           untile_plane)


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("signed", [False, True])
def test_pack_roundtrip(b, signed):
    if signed and b < 2:
        return
    rng = np.random.default_rng(b)
    lo, hi = (-(2 ** (b - 1)), 2 ** (b - 1) - 1) if signed else (0, 2 ** b - 1)
    for L in (16, 32):
        q = rng.integers(lo, hi + 1, (50, L))
        p = pack_codes(q, b, signed)
        assert p.shape == (50, L * b // 8)
        assert np.array_equal(unpack_codes(p, b, L, signed), q)


def test_hand_worked_bit_patterns():
    # 3-bit unsigned: element i at bits [3i, 3i+3), little-endian bytes
    q = np.array([[1, 2, 3, 4, 5, 6, 7, 0] + [0] * 24])
    p = pack_codes(q, 3, False)
    # bits: 001 010 011 100 101 110 111 000 (LSB first per element)
    # integer = 1 | 2<<3 | 3<<6 | 4<<9 | 5<<12 | 6<<15 | 7<<18 | 0<<21
    v = 1 | 2 << 3 | 3 << 6 | 4 << 9 | 5 << 12 | 6 << 15 | 7 << 18
    assert list(p[0, :3]) == [v & 0xFF, (v >> 8) & 0xFF, (v >> 16) & 0xFF]
    # 4-bit signed two's complement: -1 -> 0xF, 7 -> 0x7, -7 -> 0x9
    q = np.array([[-1, 7, -7, 0] + [0] * 28])
    p = pack_codes(q, 4, True)
    assert list(p[0, :2]) == [0x7F, 0x09]
    # 8-bit signed: bytes are the two's complement values
    q = np.array([[-128 + 1, -1, 0, 127] + [0] * 28])
    p = pack_codes(q, 8, True)
    assert list(p[0, :4]) == [0x81, 0xFF, 0x00, 0x7F]


def test_closed_form_block_sizes():
    # bytes per 32 elements: 4b code bytes + 2 (scale) [+ 2 (min)]
    want0 = {"q8_0": 34, "q6_0": 26, "q5_0": 22, "q4_0": 18, "q3_0": 14, "q2_0": 10}
    for c, n in want0.items():
        assert budget.row_total_bytes(c, 32, 32) == n
        assert budget.row_total_bytes(c.replace("_0", "_1"), 32, 32) == n + 2
    assert budget.row_total_bytes("q1_1", 32, 32) == 8
    assert budget.row_total_bytes("f16", 128) == 256
    # the per-token-head sizes the decode workload reads
    assert budget.row_total_bytes("q8_0") == 136 and budget.row_total_bytes("q4_0") == 72
    assert budget.row_total_bytes("q3_0") == 56
    assert budget.bits_per_value("q4_0") == 4.5 and budget.bits_per_value("q8_0") == 8.5


def test_row_layout_roundtrip_all_codecs():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((70, 128)).astype(np.float32)
    for c in CODECS:
        enc = encode_rows(x, c)
        rows = pack_rows(enc, c)
        assert rows.shape == (70, row_bytes(c, 128))
        back = unpack_rows(rows, c, 128)
        if c == "f16":
            assert np.array_equal(back, enc["values"])
        else:
            assert np.array_equal(back, enc["codes"])


def test_tile_offsets_hand_worked():
    # R = 128 -> 16-byte chunks; token 65, chunk 2, byte 0 sits at
    # (65 // 64) * 64 * 128 + (2 * 64 + 65 % 64) * 16 = 8192 + 2064 = 10256
    R, cap = 128, 128
    rows = np.zeros((cap, R), np.uint8)
    rows[65, 32] = 0xAB
    plane = tile_plane(rows)
    assert plane[10256] == 0xAB and plane.sum() == 0xAB
    # R = 24 -> 8-byte chunks; token 3 chunk 2 byte 5: (2 * 64 + 3) * 8 + 5 = 1053
    rows = np.zeros((64, 24), np.uint8)
    rows[3, 21] = 7
    assert tile_plane(rows)[1053] == 7
    assert [chunk_bytes(r) for r in (128, 64, 48, 24, 12, 6, 2)] == [16, 16, 16, 8, 4, 2, 2]


def test_tile_roundtrip():
    rng = np.random.default_rng(4)
    for R in (16, 24, 48, 128, 256, 6):
        rows = rng.integers(0, 256, (192, R)).astype(np.uint8)
        assert np.array_equal(untile_plane(tile_plane(rows), R), rows)
