"""int4 weight-only decode step for MI355X (gfx950): hand-written HIP kernels behind
a C ABI (``include/kmr.h``), with a thin ctypes binding in ``kmr.py``.

Importing the package is cheap; ``from int4_weight_only_gemv_amd import kmr`` loads
the built HIP library and fails loudly if it is missing.
"""
