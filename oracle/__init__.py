"""Reference oracle for the shared-matrix sparse-MoE expert layer (TEST INFRASTRUCTURE).

A plain, slow, float64 CPU implementation of what the layer computes, written
from the pages and the stated readings, sharing no code with the HIP library.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the product path never does.

Modules
-------
codecs : exact decoders of the storage formats (bf16, fp16, packed int4) and the
         round-to-nearest-even helpers used at the layer's rounding points.
layer  : route() and moe_forward() in "contract" and "exact" modes.
mx     : the microscaling variant: MXFP4 (E2M1 + E8M0) weights, MXFP8 (E4M3)
         product inputs, moe_forward_mx().

Every function cites the passage it follows.  Parity status of each function is
listed in its docstring; the only unpinned quantity is the absolute value of a
whole layer's output against the pages, which print no worked example
("parity unpinned" for that comparison; every internal step is pinned by the
tests under tests/test_oracle_*.py).
"""
from . import codecs, layer, mx  # noqa: F401
from .layer import route, moe_forward  # noqa: F401
