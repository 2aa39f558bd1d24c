"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library and must never be
used as a fallback for it.

* ``recurrence``: the token-by-token recurrence (Systolic Linear Attention,
  section 2.1, Eq. (2)) in C (threaded) and in numpy; this is *the* oracle for
  the exact chunkwise mode, which reaches the same result up to rounding.
* ``chunk``: the chunkwise WY form (same paper, Table 2 and the proof of the
  tile-grouped packed WY equivalence in section 2.4.2) in fp64 numpy, with the
  in-chunk inverse taken exactly, by recursive block doubling (section 2.4.3),
  or by the truncated Neumann series with residual correction (the
  paper "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
  Approximation for Quantized Gated DeltaNet").  It is the
  parity oracle for the Neumann mode and for per-stage checks.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, invariants and brute force; none is "parity unpinned".
"""
