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


def test_gemm_rs_grid_request_above_cu_count(ctx, orc):
    """A consumer_cus of twice the CU count is capped at one workgroup per CU (a reduction item waits on GEMM
    tiles other workgroups own, so every workgroup must be resident): the call succeeds with the bits of the
    default grid.  320 GEMM tiles and 2560 reduction items, more than 2 x 256 work items."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    w = I.RSWorkload("t", W=8, M=8192, K=128, N=2560, seed_index=31)
    A, B, parts = I.make_rs(w, B_layout="nk")
    a = run_rs(ctx, A, B, parts, 6, b_layout="nk")
    b = run_rs(ctx, A, B, parts, 6, b_layout="nk", consumer_cus=2 * n_cu)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert_close(b[1], orc.gemm_rs(A, B, parts, 6, b_layout="nk"), what="C_shard", **TOL_BF16)


@pytest.mark.parametrize("rs_tile", [128, 64])
def test_gemm_rs_trace_fills_exactly_its_words(ctx, rs_tile):
    """A traced call writes every one of sgt_rs_trace_words' words (one record per GEMM tile and reduction
    item) and nothing past them; results are the untraced call's bits."""
    w = I.RSWorkload("t", W=4, M=1024, K=256, N=392, seed_index=26)
    A, B, parts = I.make_rs(w)
    nw = sgt.rs_trace_words(w.W, w.M, w.N, rs_tile=rs_tile)
    canary = 0x5A5A5A5A5A5A5A5A
    tr = torch.full((nw + 64,), canary, dtype=torch.int64, device="cuda:0")
    a = run_rs(ctx, A, B, parts, 1, rs_tile=rs_tile, trace=tr.data_ptr())
    b = run_rs(ctx, A, B, parts, 1, rs_tile=rs_tile)
    t = tr.cpu().numpy()
    assert (t[nw:] == canary).all(), "trace written past sgt_rs_trace_words"
    rec = t[:nw].reshape(-1, 3)
    assert (rec[:, 0] != canary).all() and (rec[:, 1] >= rec[:, 0]).all(), "a work item left no record"
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


def run_rs_paced(ctx, A, B, parts, rank, b_layout="kn", rs_tile=0, **kw):
    """sgt_gemm_rs_paced: the peers' blocks start outside the inbox and arrive through the producer."""
    W = len(parts)
    M, K = A.shape
    N = B.shape[1] if b_layout == "kn" else B.shape[0]
    ng, npf = sgt.rs_flag_count(W, M, N, rs_tile=rs_tile)
    P = poison_like(torch.empty((M, N), dtype=torch.float32, device="cuda:0"))
    Cs = poison_like(torch.empty((M // W, N), dtype=torch.float32, device="cuda:0"))
    gf = torch.zeros(max(ng, 4), dtype=torch.int32, device="cuda:0")
    pf = torch.zeros(max(npf, 4), dtype=torch.int32, device="cuda:0")
    src = [dev(p) if q != rank else None for q, p in enumerate(parts)]
    inbox = [poison_like(torch.empty_like(s)) if s is not None else None for s in src]
    ctx.gemm_rs_paced(dev(A), dev(B), src, inbox, P, Cs, gf, pf, rank=rank, b_layout=b_layout, rs_tile=rs_tile,
                      blocking=True, **kw)
    torch.cuda.synchronize()
    return host(P), host(Cs), host(gf)[:ng], host(pf)[:npf], [host(x) if x is not None else None for x in inbox]


PACED = [
    dict(producer="cu"),
    dict(producer="cu", peer_gbps=40.0, jitter_us=3.0, arrival_seed=5),
    dict(producer="cu", peer_gbps=20.0, arrival_order="global", arrival_seed=9),
    dict(producer="serial", peer_gbps=60.0),
]


@pytest.mark.parametrize("opts", PACED, ids=["cu", "cu-40gbps-jitter", "cu-20gbps-shuffled", "serial"])
@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2]])
def test_gemm_rs_paced_parity(ctx, orc, shape, opts):
    W, br, K, N, rt = shape
    w = I.RSWorkload("t", W=W, M=W * br, K=K, N=N, seed_index=26)
    A, B, parts = I.make_rs(w)
    rank = 1
    P, Cs, gf, pf, inbox = run_rs_paced(ctx, A, B, parts, rank, rs_tile=rt, **opts)
    for q in range(W):
        if q != rank:
            assert np.array_equal(inbox[q].view(np.uint32), parts[q].view(np.uint32)), "inbox %d" % q
    assert_close(P, orc.gemm(A, B), what="partial_out", **TOL_BF16)
    assert_close(Cs, orc.gemm_rs(A, B, parts, rank), what="C_shard", **TOL_BF16)
    assert (gf == gf[0]).all() and gf[0] != 0
    nb = len(pf) // W
    for q in range(W):
        if q != rank:
            assert (pf[q * nb:(q + 1) * nb] == gf[0]).all(), "peer %d flags" % q


def test_gemm_rs_paced_matches_resident_bits(ctx):
    w = I.RSWorkload("t", W=4, M=1024, K=256, N=392, seed_index=27)
    A, B, parts = I.make_rs(w, B_layout="nk")
    a = run_rs(ctx, A, B, parts, 2, b_layout="nk")
    b = run_rs_paced(ctx, A, B, parts, 2, b_layout="nk", peer_gbps=30.0)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_gemm_rs_paced_zero_A_is_exact_peer_sum(ctx, orc):
    w = I.RSWorkload("t", W=8, M=1024, K=64, N=256, dist="int", peer_dist="int", seed_index=28)
    A, B, parts = I.make_rs(w)
    A = np.zeros_like(A)
    for rank in [0, 7]:
        _, Cs, _, _, _ = run_rs_paced(ctx, A, B, parts, rank, peer_gbps=50.0, arrival_order="global",
                                      arrival_seed=rank + 1)
        assert np.array_equal(Cs.astype(np.float64), orc.gemm_rs(A, B, parts, rank))


def test_gemm_rs_paced_withheld_peer_times_out(ctx):
    w = I.RSWorkload("t", W=4, M=1024, K=64, N=256, seed_index=29)
    A, B, parts = I.make_rs(w)
    with pytest.raises(sgt.SgtError) as ei:
        run_rs_paced(ctx, A, B, parts, 0, withhold_peer=2, timeout_ms=20.0)
    assert ei.value.status == sgt.SGT_ETIMEDOUT
    # the context stays usable
    _, Cs, _, _, _ = run_rs_paced(ctx, A, B, parts, 0)
    assert np.isfinite(Cs).all()


def test_gemm_rs_paced_rejects_bad_modes(ctx):
    w = I.RSWorkload("t", W=4, M=1024, K=64, N=256, seed_index=30)
    A, B, parts = I.make_rs(w)
    with pytest.raises(sgt.SgtError) as ei:
        run_rs_paced(ctx, A, B, parts, 0, producer="preset")
    assert ei.value.status == sgt.SGT_EINVAL
    with pytest.raises(sgt.SgtError) as ei:
        run_rs(ctx, A, B, parts, 0, peer_gbps=10.0)
    assert ei.value.status == sgt.SGT_EUNSUPPORTED
