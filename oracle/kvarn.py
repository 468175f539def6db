"""KVarN basis: per-channel variance normalisation, then Hadamard rotation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources.  The BeeLlama.cpp v0.4.0 release notes (section on KVarN) describe
variance-normalised KV-cache quantisation that gains accuracy at a given bit
width; the KV-COBRA explainer lists KVarN as the Hadamard-rotated low-bit
cache whose rotation spreads outliers so one quantiser setting fits every
channel.  Readings taken:

* The caller supplies ``w = 1/sigma`` per (kv head, channel) in binary32;
  the library does not estimate sigma.
* Stored basis: ``y = H (x * w)`` with the unnormalised Sylvester ``H`` of
  order 128, then any ``_0``/``_1`` block codec on blocks of 32.
* Raw-basis reconstruction: ``x~ = (H y^) / 128 / w`` (``H^-1 = H / 128``).
* Both K and V are rotated.
"""

import numpy as np

from . import hadamard


def rotate(x, w):
    """``y = H (x * w)`` in fp64.  x: [..., 128], w: [128] (or broadcastable)."""
    z = np.asarray(x, dtype=np.float64) * np.asarray(w, dtype=np.float64)
    return hadamard.transform(z)


def unrotate(y, w):
    """``(H y) / 128 / w`` in fp64: the raw-basis vector of a stored one."""
    n = np.asarray(y).shape[-1]
    return hadamard.transform(y) / n / np.asarray(w, dtype=np.float64)
