"""CPU oracle for group-wise INT4 (W4A16), AWQ calibration and the FP4 decode path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
restatement of what the hot path computes, written from the pages'
formulas.  It is imported by ``tests/``, by ``__graft_entry__.smoke()`` and by
the ``cpu_baseline`` leg of ``bench.py`` and by nothing else; the product
library never calls it and shares no code, table or constant with it.

Precision: fp32 wherever the method fixes fp32 (the group scale, zero point
and code computations, all true IEEE operations in a fixed order), fp64 for
every sum and matrix product (the forward reference, the MSE of the search).

Modules
  int4   group min/max -> scale, zero, codes, nibble packing, dequantization,
         the fp64 W4A16 forward reference
  stats  per-input-channel mean |x| (exact sum, rounded once)
  awq    candidate channel scales and the exhaustive alpha-grid MSE search
  fp4    E2M1 / E4M3 decoding, the FP4 forward reference, and an encoder used
         only to build realistic FP4 inputs

Parity pins: every function is pinned in ``tests/test_oracle_*.py`` against
closed forms, exhaustive or brute-force enumeration and the pages' own
worked numbers.  One function is *parity unpinned* beyond a round-trip
bound: ``fp4.encode`` (the pages name the FP4 format but not an encoder).
"""
