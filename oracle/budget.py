"""Bit and byte accounting of the stored formats.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources: the KV-COBRA explainer's jargon list defines bits per dimension
(bpd) as the mean storage cost, in bits, of one stored coordinate (F16 is
16), and
its worked example ("Where the bits actually go") prices a head at
``rank * bits`` code bits per token against a budget of ``128 * bpd``.  The
bandwidth thread's arithmetic (bytes read per generated token bound the
token rate) is why these byte counts are the numerator of the throughput
metric.
"""

from .codecs import CODECS


def code_bits(codec, n=128):
    fam, b = CODECS[codec]
    return 16 * n if fam == "f16" else b * n


def side_bits(codec, n=128, block_len=32):
    """Scale (and min) bits of a row: one binary16 each per block."""
    fam, _ = CODECS[codec]
    if fam == "f16":
        return 0
    per_block = 16 if fam == "0" else 32
    return per_block * (n // block_len)


def bits_per_value(codec, n=128, block_len=32):
    return (code_bits(codec, n) + side_bits(codec, n, block_len)) / n


def row_total_bytes(codec, n=128, block_len=32):
    """Bytes one token of one head occupies (codes + scales + mins)."""
    return (code_bits(codec, n) + side_bits(codec, n, block_len)) // 8


def head_code_bits(rank, b):
    """Code bits per token of a low-rank head: rank coordinates at b bits."""
    return rank * b


def budget_bits(bpd, n=128):
    return bpd * n
