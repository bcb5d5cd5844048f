"""GPU parity of the GEMM + ReduceScatter path against the CPU oracle (through the C ABI)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import TOL_BF16, assert_close, dev, host, poison_like, sample_rows  # noqa: E402


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = sgt.Context(0)
    yield c
    c.close()


def run_rs(ctx, A, B, parts, rank, b_layout="kn", rs_tile=0, **kw):
    W = len(parts)
    M, K = A.shape
    N = B.shape[1] if b_layout == "kn" else B.shape[0]
    ng, npf = sgt.rs_flag_count(W, M, N, rs_tile=rs_tile)
    P = poison_like(torch.empty((M, N), dtype=torch.float32, device="cuda:0"))
    Cs = poison_like(torch.empty((M // W, N), dtype=torch.float32, device="cuda:0"))
    gf = torch.zeros(max(ng, 4), dtype=torch.int32, device="cuda:0")
    pf = torch.zeros(max(npf, 4), dtype=torch.int32, device="cuda:0")
    dparts = [dev(p) if q != rank else None for q, p in enumerate(parts)]
    ctx.gemm_rs(dev(A), dev(B), dparts, P, Cs, gf, pf, rank=rank, b_layout=b_layout, rs_tile=rs_tile,
                blocking=True, **kw)
    torch.cuda.synchronize()
    return host(P), host(Cs), host(gf)[:ng], host(pf)[:npf]


SHAPES = [
    # W, block rows, K, N, rs_tile
    (4, 256, 200, 328, 128),    # K tail, N tail of 72 in the last signal tile
    (2, 512, 1024, 512, 128),   # exact tiles
    (8, 128, 136, 264, 64),     # blocks smaller than a GEMM tile
    (4, 256, 320, 520, 256),    # one signal tile per GEMM tile
]


@pytest.mark.parametrize("b_layout", ["kn", "nk"])
@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_rs_parity(ctx, orc, shape, b_layout):
    W, br, K, N, rt = shape
    w = I.RSWorkload("t", W=W, M=W * br, K=K, N=N, seed_index=21)
    A, B, parts = I.make_rs(w, B_layout=b_layout)
    P_ref = orc.gemm(A, B, b_layout=b_layout)
    for rank in sorted({0, W - 1}):
        P, Cs, gf, pf = run_rs(ctx, A, B, parts, rank, b_layout=b_layout, rs_tile=rt)
        assert_close(P, P_ref, what="partial_out", **TOL_BF16)
        C_ref = orc.gemm_rs(A, B, parts, rank, b_layout=b_layout)
        assert_close(Cs, C_ref, what="C_shard rank %d" % rank, **TOL_BF16)
        assert (gf == gf[0]).all() and (pf == gf[0]).all()


def test_gemm_rs_zero_A_is_exact_peer_sum(ctx, orc):
    w = I.RSWorkload("t", W=4, M=1024, K=64, N=256, dist="int", peer_dist="int", seed_index=22)
    A, B, parts = I.make_rs(w)
    A = np.zeros_like(A)
    for rank in range(4):
        _, Cs, _, _ = run_rs(ctx, A, B, parts, rank)
        assert np.array_equal(Cs.astype(np.float64), orc.gemm_rs(A, B, parts, rank))


def test_gemm_rs_zero_peers_is_exact_block(ctx, orc):
    w = I.RSWorkload("t", W=4, M=1024, K=520, N=264, dist="int", peer_dist="zero", seed_index=23)
    A, B, parts = I.make_rs(w)
    full = orc.gemm(A, B)
    for rank in [1, 2]:
        P, Cs, _, _ = run_rs(ctx, A, B, parts, rank)
        assert np.array_equal(P.astype(np.float64), full)
        assert np.array_equal(Cs.astype(np.float64), full[rank * 256:(rank + 1) * 256])


def test_gemm_rs_bits_repeat(ctx):
    w = I.RSWorkload("t", W=8, M=2048, K=512, N=512, seed_index=24)
    A, B, parts = I.make_rs(w)
    a = run_rs(ctx, A, B, parts, 5)
    b = run_rs(ctx, A, B, parts, 5, consumer_cus=37)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_gemm_rs_rejects_bad_tile(ctx):
    w = I.RSWorkload("t", W=4, M=1024, K=64, N=256, seed_index=25)
    A, B, parts = I.make_rs(w)
    with pytest.raises(sgt.SgtError):
        run_rs(ctx, A, B, parts, 0, rs_tile=96)


@pytest.mark.slow
def test_full_gemm_rs_shape(ctx, orc):
    w = I.GEMM_RS
    A, B, parts = I.make_rs(w)
    rank = 3
    P, Cs, gf, pf = run_rs(ctx, A, B, parts, rank)
    rows = sample_rows(w.M // w.W, 1, per_shard=12, seed=1)
    C_ref = orc.gemm_rs(A, B, parts, rank, rows=rows)
    assert_close(Cs[rows], C_ref, what="C_shard", **TOL_BF16)
    prow = sample_rows(w.M, w.W, per_shard=3, seed=2)
    assert_close(P[prow], orc.gemm(A, B, rows=prow), what="partial_out", **TOL_BF16)
    assert (gf == gf[0]).all() and (pf == gf[0]).all()
