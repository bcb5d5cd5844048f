"""sgt_gemm_rs_static (GEMM + ReduceScatter with no allocation: flags, claim counter and status in the library's
static per-device scratch) against sgt_gemm_rs (the context entry point with the same kernels), through the C ABI:
two calls in a row, the second with a smaller input, each bit-identical to the context call and within the bf16
tolerance of the oracle (Triton-distributed semantics page, "GEMM + ReduceScatter overlap")."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import TOL_BF16, assert_close, dev, host, poison_like  # noqa: E402


def _run_static(A, B, parts, rank, b_layout, **kw):
    W = len(parts)
    M = A.shape[0]
    N = B.shape[1] if b_layout == "kn" else B.shape[0]
    P = poison_like(torch.empty((M, N), dtype=torch.float32, device="cuda:0"))
    Cs = poison_like(torch.empty((M // W, N), dtype=torch.float32, device="cuda:0"))
    dparts = [dev(p) if q != rank else None for q, p in enumerate(parts)]
    sgt.gemm_rs_static(dev(A), dev(B), dparts, P, Cs, rank=rank, b_layout=b_layout, blocking=True, **kw)
    torch.cuda.synchronize()
    return host(P), host(Cs)


def _run_ctx(ctx, A, B, parts, rank, b_layout):
    W = len(parts)
    M = A.shape[0]
    N = B.shape[1] if b_layout == "kn" else B.shape[0]
    ng, npf = sgt.rs_flag_count(W, M, N)
    P = poison_like(torch.empty((M, N), dtype=torch.float32, device="cuda:0"))
    Cs = poison_like(torch.empty((M // W, N), dtype=torch.float32, device="cuda:0"))
    dparts = [dev(p) if q != rank else None for q, p in enumerate(parts)]
    ctx.gemm_rs(dev(A), dev(B), dparts, P, Cs, torch.zeros(ng, dtype=torch.int32, device="cuda:0"),
                torch.zeros(npf, dtype=torch.int32, device="cuda:0"), rank=rank, b_layout=b_layout, blocking=True)
    torch.cuda.synchronize()
    return host(P), host(Cs)


def test_static_scratch_matches_context_call_twice(orc):
    assert torch.cuda.is_available()
    assert sgt.gemm_rs_static_scratch_bytes() == 64 * 1024
    cases = [
        # the larger call first, then a smaller one (fewer flags, fewer items) on the same scratch
        (I.RSWorkload("t", W=8, M=8 * 512, K=1000, N=1288, seed_index=61), 5, "nk"),
        (I.RSWorkload("t", W=4, M=4 * 256, K=200, N=328, seed_index=62), 1, "kn"),
    ]
    with sgt.Context(0) as ctx:
        for w, rank, lay in cases:
            A, B, parts = I.make_rs(w, B_layout=lay)
            P_s, C_s = _run_static(A, B, parts, rank, lay)
            P_c, C_c = _run_ctx(ctx, A, B, parts, rank, lay)
            assert np.array_equal(P_s.view(np.uint32), P_c.view(np.uint32)), "partial_out bits"
            assert np.array_equal(C_s.view(np.uint32), C_c.view(np.uint32)), "C_shard bits"
            assert_close(P_s, orc.gemm(A, B, b_layout=lay), what="partial_out", **TOL_BF16)
            assert_close(C_s, orc.gemm_rs(A, B, parts, rank, b_layout=lay), what="C_shard", **TOL_BF16)


def test_static_scratch_rejects_too_many_flags():
    # 16384 x 8192 with W = 8: 8192 GEMM flags + 8192 peer flags > 16320 words; rejected before any launch
    w = I.RSWorkload("t", W=8, M=16384, K=64, N=8192, seed_index=63)
    A = torch.zeros((w.M, w.K), dtype=torch.bfloat16, device="cuda:0")
    B = torch.zeros((w.K, w.N), dtype=torch.bfloat16, device="cuda:0")
    parts = [torch.zeros((w.M // w.W, w.N), dtype=torch.float32, device="cuda:0") for _ in range(w.W)]
    P = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
    Cs = torch.empty((w.M // w.W, w.N), dtype=torch.float32, device="cuda:0")
    with pytest.raises(sgt.SgtError) as ei:
        sgt.gemm_rs_static(A, B, parts, P, Cs, rank=0, blocking=True)
    assert ei.value.status == sgt.SGT_EINVAL and "static scratch" in str(ei.value)
