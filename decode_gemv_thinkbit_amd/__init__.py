"""ThinkBit low-bit GEMV/GEMM for MI355X (gfx950).

The compute path is the HIP library ``libqlinear.so`` behind the C ABI in
``include/qlinear.h``; ``qlinear`` is its thin Python binding (argument
marshalling only).  ``synth`` and ``configs`` hold the seeded synthetic
workloads.
"""
