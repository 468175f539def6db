"""Packed low-bit KV cache and decode attention for AMD Instinct MI355X.

The computation lives in ``libkvq.so`` (hand-written HIP for gfx950, C ABI in
``include/kvq.h``); this package is its binding:

* ``lib``   - ctypes declarations of the C ABI (same names as the header);
* ``cache`` - ``LayerCache``: one layer's device buffers and token count;
* ``calib`` - host helpers for the frozen per-head settings (KVarN
  normalisers, low-rank projections);
* ``build`` - compiles the library in-tree.
"""

from . import lib  # noqa: F401

__all__ = ["lib"]
