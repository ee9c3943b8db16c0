"""Plain float64 CPU oracle for paged FP8 (E4M3) flash-decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
anything in this package: only the test-suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP library (no kernels, headers, tables or helpers) and never
consumes a value produced by it.

What it computes, and the page each part follows:

* ``fp8``       -- the E4M3 and E8M0 value tables built from the bit-field
                  definitions, the round-to-nearest-even E4M3 encoder and the
                  block-scale rules (page "fp8 paged attention for MoE serving",
                  sections "Supported scope" and "Smallest correct example";
                  page "Attention MXFP8 TKG Kernel API Reference" for MXFP8).
* ``pool``      -- the packed-row pool format (payload then scale footer), the
                  addressing of a code/scale through the block table, and the
                  reference KV append (same page, "Supported scope").
* ``attention`` -- decode attention written as its plain definition: window,
                  sink logit in the denominator, custom sm_scale, GQA head map;
                  the split partials and their log-sum-exp merge (same page,
                  "Why it happens", "Expected result").

Every function is pinned by tests under ``tests/test_oracle_*.py`` to library
routines, closed forms, invariants or brute force; none is "parity unpinned".
"""
from . import fp8, pool, attention  # noqa: F401
