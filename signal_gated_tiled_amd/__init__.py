"""Signal-gated tiled AllGather+GEMM / GEMM+ReduceScatter for MI355X (gfx950).

The compute path lives in ``libsgt.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/sgt.h``); this package holds the thin ctypes binding
and the seeded input generators.
"""
