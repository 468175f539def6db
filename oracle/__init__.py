"""Reference oracle for the packed low-bit KV cache and decode attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU implementation (NumPy, fp64 unless a step's definition fixes a narrower
rounding) of everything the GPU library computes.  It exists to check the
library.  Only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark import it; the library itself never does, and the library shares no
code, headers, tables or helpers with it.

Module map (each function cites the passage of the source pages it follows):

* ``rounding``  - RN16 / RN32 / round-half-even primitives.
* ``codecs``    - the ``_0`` (absmax, signed) and ``_1`` (min-offset,
                  unsigned) block codecs and the F16 codec.
* ``bitpack``   - b-bit code packing inside a block's code field.
* ``layout``    - the byte layout of a plane in device memory.
* ``hadamard``  - the Sylvester Hadamard matrix (dense definition).
* ``kvarn``     - variance normalisation + Hadamard rotation basis.
* ``cobra``     - per-head low-rank projection basis.
* ``attention`` - single-query softmax attention (fp64).
* ``layer``     - one layer's cache: append semantics, precision tail,
                  dequantisation, decode and transcode, built from the above.
* ``budget``    - bit accounting of the stored formats.
* ``vbr``       - the VBR budget controller (degrade plan over a codec
                  ladder under a byte budget).
* ``allocator`` - per-head rank/bit allocation: the error model, the exact
                  optimum (dynamic programming) and the C1/C2
                  water-filling steps.

Parity status: every function here is pinned by a CPU test in
``tests/test_oracle_*.py`` against something other than itself (closed forms,
library routines, brute force over exact rationals, printed figures of the
pages).  Exceptions are listed in the function's docstring as
"parity unpinned".
"""
