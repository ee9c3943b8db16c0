"""Paged FP8 (E4M3) flash-decode attention for MI355X (gfx950).

The compute path is the HIP library ``libfp8pa.so`` built from ``csrc/``; the
Python layer in ``ops`` only marshals arguments through its C ABI.  Importing
this package loads nothing; the library is opened on first use and a missing
library is an error (there is no fallback).
"""
