"""Signal-gated tiled AllGather+GEMM / GEMM+ReduceScatter for MI355X (gfx950).

The compute path lives in ``libsgt.so`` (hand-written HIP kernels behind the C
ABI declared in ``include/sgt.h``).  ``_sgt`` is the thin ctypes binding with
the same names; ``inputs`` holds the seeded synthetic workload generators.
"""
from ._sgt import (Context, Opts, SgtError, a2a_flag_count, ag_flag_count, ag_panel_rows, lib, make_opts, panel_order,  # noqa: F401
                   gemm_rs_static, gemm_rs_static_scratch_bytes,
                   ll_buffer_bytes, moe_trace_words, ring_flag_count, rs_flag_count, rs_trace_words, trace_words, version, LIB_PATH, SGT_BF16,
                   SGT_F32, SGT_ETIMEDOUT, SGT_EINVAL, SGT_EUNSUPPORTED)
