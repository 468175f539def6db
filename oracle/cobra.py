"""KV-COBRA-style per-head low-rank basis.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources: the KV-COBRA explainer.  Each head keeps its top ``r_h`` directions
(found by a per-head SVD) and stores each kept coordinate with ``b_h`` bits;
a Hadamard rotation is fused into the same projection matrix so that the kept
coordinates have even variances; at inference every key is projected,
rotated and quantised with the frozen per-head settings (section on the two
supporting pieces), and the worked example in "Where the bits actually go"
prices a head at ``r_h * b_h`` code bits per token.  Readings taken:

* The per-head basis ``U_h`` is an input (orthonormal 128 x 128; the SVD of
  real calibration data is replaced by a seeded random orthonormal basis).
* ``P_h = RN16(U_h[:, :r] H_r / sqrt(r))`` (128 x r, binary16): the fused
  rotation.
* Stored coordinates ``u = P_h^T x`` (fp64 from the binary16 entries of P),
  coded with ``q{b_h}_1`` on blocks of ``min(32, r)``.
* Attention in rank space: ``<P^T q, u^>`` and output ``P (sum_t p_t u^_t)``,
  i.e. the raw-basis reconstructions ``x~ = P u^``.  K and V share ``P_h``.
"""

import numpy as np

from . import hadamard
from .rounding import rn16


def projection(U, r):
    """``RN16(U[:, :r] H_r / sqrt(r))``: binary16 [128, r]."""
    U = np.asarray(U, dtype=np.float64)
    H = hadamard.sylvester(r).astype(np.float64)
    return rn16(U[:, :r] @ H / np.sqrt(r))


def project(x, P):
    """Coordinates ``P^T x`` in fp64.  x: [..., 128], P: [128, r]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(P, dtype=np.float64)


def reconstruct(u, P):
    """Raw-basis vectors ``P u``.  u: [..., r] -> [..., 128]."""
    return np.asarray(u, dtype=np.float64) @ np.asarray(P, dtype=np.float64).T


def block_len(r):
    return min(32, r)
