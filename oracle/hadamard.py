"""Sylvester Hadamard matrix (dense definition).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The KV-COBRA explainer (Jargon, "Hadamard rotation") describes the rotation
as a fixed orthogonal transform with +-1 entries that mixes channels so their
variances even out; the BeeLlama v0.4.0 notes name the variance-normalised
KVarN cache the rotation serves.  Reading: the Sylvester construction
``H_1 = [1]``, ``H_2n = [[H_n, H_n], [H_n, -H_n]]`` in natural order, entries
+-1, unnormalised, no random signs; ``H_n H_n^T = n I``.
"""

import numpy as np


def sylvester(n):
    """The n x n Sylvester Hadamard matrix (n a power of two), int64."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def transform(x, n=None):
    """``H x`` along the last axis, by dense matrix product in fp64."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1] if n is None else n
    return x @ sylvester(n).T.astype(np.float64)
