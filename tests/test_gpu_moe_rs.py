"""GPU parity of the MoE GEMM + ReduceScatter (combine side) against the CPU oracle.

The routing tables are inputs of this call (the AllGather side computes them); the tests build them with
the oracle's routing from seeded logits, and one test chains the GPU routing of sgt_moe_ag_gemm into it.
Y, P and C are checked to the bf16 tolerance of the workload definition, or exactly for integer-valued
inputs with power-of-two gates.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import TOL_BF16, assert_close, assert_close_bf16_out, dev, host, poison_like, sample_rows  # noqa: E402


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = sgt.Context(0)
    yield c
    c.close()


def run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, rank, w_layout="kn", paced=False, **kw):
    """Upload, run sgt_moe_gemm_rs (or the paced variant, whose peers' blocks arrive into an inbox);
    return host (Y, P, C, gflags, pflags) and, when paced, the inbox."""
    W = len(parts)
    T, k = ids.shape
    H = W2.shape[2] if w_layout == "kn" else W2.shape[1]
    rows = T * k
    ng, npf = sgt.rs_flag_count(W, T, H, rs_tile=128)
    y_dtype = kw.pop("y_dtype", torch.float32)
    Y = poison_like(torch.empty((rows, H), dtype=y_dtype, device="cuda:0"))
    P = poison_like(torch.empty((T, H), dtype=torch.float32, device="cuda:0"))
    C = poison_like(torch.empty((T // W, H), dtype=torch.float32, device="cuda:0"))
    gf = torch.zeros(max(ng, 4), dtype=torch.int32, device="cuda:0")
    pf = torch.zeros(max(npf, 4), dtype=torch.int32, device="cuda:0")
    dparts = [dev(p) if q != rank else None for q, p in enumerate(parts)]
    inbox = [poison_like(torch.empty_like(p)) if p is not None else None for p in dparts] if paced else None
    ctx.moe_gemm_rs(dev(Hg), dev(W2), dev(gate), dev(ids), dev(off), dev(rt), dparts, Y, P, C, gf, pf, rank=rank,
                    b_layout=w_layout, blocking=True, inbox=inbox, **kw)
    torch.cuda.synchronize()
    out = (host(Y), host(P), host(C), host(gf)[:ng], host(pf)[:npf])
    if paced:
        return out + ([host(x) if x is not None else None for x in inbox],)
    return out


def make(w, w_layout="kn", pow2_gates=False):
    Hg, W2, gate, logits, parts = I.make_moe_rs(w, W_layout=w_layout)
    if pow2_gates:
        gate = (2.0 ** -np.random.default_rng(w.seed_index).integers(0, 3, size=gate.shape)).astype(np.float32)
    return Hg, W2, gate, logits, parts


SHAPES = [
    # T, W, E, k, I, H
    (512, 4, 8, 2, 256, 512),
    (1024, 8, 16, 4, 136, 264),   # K tail; last combine column tile 8 wide
    (256, 2, 4, 1, 64, 128),
]


@pytest.mark.parametrize("w_layout", ["kn", "nk"])
@pytest.mark.parametrize("shape", SHAPES)
def test_moe_rs_parity(ctx, orc, shape, w_layout):
    T, W, E, k, n_in, H = shape
    w = I.scaled(I.MOE_RS, T=T, W=W, E=E, topk=k, I=n_in, H=H, seed_index=31)
    Hg, W2, gate, logits, parts = make(w, w_layout)
    ids, off, rt = orc.moe_route(logits, k)
    for rank in sorted({0, W - 1}):
        Y, P, C, gf, pf = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, rank, w_layout)
        Y_ref = orc.moe_gemm(Hg, W2, off, np.arange(T * k, dtype=np.int32), w_layout)
        assert_close(Y, Y_ref, what="Y", **TOL_BF16)
        P_ref = orc.moe_gemm_rs_p(Hg, W2, gate, ids, off, rt, np.arange(T), w_layout)
        assert_close(P, P_ref, what="P", **TOL_BF16)
        C_ref = orc.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, rank, w_layout)
        assert_close(C, C_ref, what="C rank %d" % rank, **TOL_BF16)
        assert (gf == gf[0]).all() and gf[0] != 0 and (pf == gf[0]).all()


def test_moe_rs_integer_inputs_exact(ctx, orc):
    w = I.scaled(I.MOE_RS, T=512, W=4, E=8, topk=3, I=128, H=256, dist="int", peer_dist="int", seed_index=32)
    Hg, W2, gate, logits, parts = make(w, pow2_gates=True)
    ids, off, rt = orc.moe_route(logits, 3)
    Y, P, C, _, _ = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 2)
    assert np.array_equal(C.astype(np.float64), orc.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, 2))
    assert np.array_equal(P.astype(np.float64), orc.moe_gemm_rs_p(Hg, W2, gate, ids, off, rt, np.arange(512)))


def test_moe_rs_single_expert_top1_matches_dense_gemm_rs_bits(ctx, orc):
    # one expert, one pick, gate 1: the grouped rows are the tokens in order, and the result must be the
    # dense GEMM+ReduceScatter's bit for bit (same tiles, same k order, same reduction)
    w = I.scaled(I.MOE_RS, T=1024, W=4, E=1, topk=1, I=192, H=384, seed_index=33)
    Hg, W2, gate, logits, parts = make(w)
    ids = np.zeros((1024, 1), np.int32)
    off = np.array([0, 1024], np.int32)
    rt = np.arange(1024, dtype=np.int32)
    gate = np.ones((1024, 1), np.float32)
    Y, P, C, _, _ = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 1)
    ng, npf = sgt.rs_flag_count(4, 1024, 384, rs_tile=128)
    P2 = poison_like(torch.empty((1024, 384), dtype=torch.float32, device="cuda:0"))
    C2 = poison_like(torch.empty((256, 384), dtype=torch.float32, device="cuda:0"))
    gf = torch.zeros(ng, dtype=torch.int32, device="cuda:0")
    pf = torch.zeros(npf, dtype=torch.int32, device="cuda:0")
    ctx.gemm_rs(dev(Hg), dev(W2[0]), [dev(p) if q != 1 else None for q, p in enumerate(parts)], P2, C2, gf, pf,
                rank=1, rs_tile=128, tile_waves=8, blocking=True)
    torch.cuda.synchronize()
    assert np.array_equal(P.view(np.uint32), host(P2).view(np.uint32))
    assert np.array_equal(C.view(np.uint32), host(C2).view(np.uint32))


def test_moe_rs_bits_repeat_and_grid(ctx, orc):
    w = I.scaled(I.MOE_RS, T=1024, W=8, E=16, topk=4, I=256, H=512, seed_index=34)
    Hg, W2, gate, logits, parts = make(w, "nk")
    ids, off, rt = orc.moe_route(logits, 4)
    a = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 5, "nk")
    b = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 5, "nk", consumer_cus=37)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_moe_rs_takes_gpu_routing(ctx, orc):
    # the AllGather side's routing tables feed the combine side directly
    m = I.scaled(I.MOE, T=512, W=4, H=128, I=64, E=8, topk=2, seed_index=35)
    shards, We, logits = I.make_moe(m)
    T, k = 512, 2
    Xg = torch.empty((T, 128), dtype=torch.bfloat16, device="cuda:0")
    Yup = torch.empty((T * k, 64), dtype=torch.float32, device="cuda:0")
    off = torch.empty(9, dtype=torch.int32, device="cuda:0")
    rt = torch.empty(T * k, dtype=torch.int32, device="cuda:0")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda:0")
    fl = torch.zeros(sgt.ag_flag_count(4, T, 128), dtype=torch.int32, device="cuda:0")
    ctx.moe_ag_gemm([dev(s) for s in shards], dev(We), dev(logits), Xg, Yup, off, rt, ids, fl, topk=k,
                    producer="preset", blocking=True)
    torch.cuda.synchronize()
    w = I.scaled(I.MOE_RS, T=T, W=4, E=8, topk=k, I=128, H=256, seed_index=36)
    Hg, W2, gate, _, parts = make(w)
    ids_h, off_h, rt_h = host(ids), host(off), host(rt)
    ids_o, off_o, rt_o = orc.moe_route(logits, k)
    assert np.array_equal(ids_h, ids_o) and np.array_equal(off_h, off_o) and np.array_equal(rt_h, rt_o)
    Y, P, C, _, _ = run_moe_rs(ctx, Hg, W2, gate, ids_h, off_h, rt_h, parts, 3)
    assert_close(C, orc.moe_gemm_rs(Hg, W2, gate, ids_o, off_o, rt_o, parts, 3), what="C", **TOL_BF16)


@pytest.mark.parametrize("opts", [dict(producer="cu", peer_gbps=40.0, jitter_us=3.0, arrival_seed=2),
                                  dict(producer="cu", peer_gbps=0.0, arrival_order="global", arrival_seed=5),
                                  dict(producer="serial", peer_gbps=60.0)], ids=["cu-40gbps", "cu-unthrottled",
                                                                                 "serial"])
def test_moe_rs_paced_matches_resident_bits(ctx, orc, opts):
    w = I.scaled(I.MOE_RS, T=1024, W=4, E=8, topk=2, I=128, H=264, seed_index=38)
    Hg, W2, gate, logits, parts = make(w, "nk")
    ids, off, rt = orc.moe_route(logits, 2)
    a = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 2, "nk")
    b = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 2, "nk", paced=True, **opts)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    for q in range(4):
        if q != 2:
            assert np.array_equal(b[5][q].view(np.uint32), parts[q].view(np.uint32)), "inbox %d" % q
    nb = len(b[4]) // 4   # peer flags, one block per rank; this rank's own block is never sent
    for q in range(4):
        if q != 2:
            assert (b[4][q * nb:(q + 1) * nb] == b[3][0]).all(), "peer %d flags" % q


def test_moe_rs_paced_withheld_peer_times_out(ctx, orc):
    w = I.scaled(I.MOE_RS, T=512, W=4, E=8, topk=2, I=64, H=128, seed_index=39)
    Hg, W2, gate, logits, parts = make(w)
    ids, off, rt = orc.moe_route(logits, 2)
    with pytest.raises(sgt.SgtError) as ei:
        run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 0, paced=True, withhold_peer=1, timeout_ms=20.0)
    assert ei.value.status == sgt.SGT_ETIMEDOUT
    # the context stays usable
    _, _, C, _, _ = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 0)
    assert_close(C, orc.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, 0), what="C", **TOL_BF16)


def test_moe_rs_bad_args(ctx, orc):
    w = I.scaled(I.MOE_RS, T=512, W=4, E=8, topk=2, I=64, H=128, seed_index=37)
    Hg, W2, gate, logits, parts = make(w)
    ids, off, rt = orc.moe_route(logits, 2)
    with pytest.raises(sgt.SgtError) as ei:      # T/W not a multiple of 128
        run_moe_rs(ctx, Hg[:2 * 384], W2, gate[:384], ids[:384], off, rt[:768], parts, 0)
    assert ei.value.status == sgt.SGT_EINVAL
    with pytest.raises(sgt.SgtError) as ei:      # paced peers go through the paced entry point
        run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 0, peer_gbps=10.0)
    assert ei.value.status == sgt.SGT_EUNSUPPORTED
    with pytest.raises(sgt.SgtError) as ei:      # the paced entry point needs a producer mode
        run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, 0, paced=True, producer="preset")
    assert ei.value.status == sgt.SGT_EINVAL


@pytest.mark.slow
def test_full_moe_rs_shape_paced_back_to_back(ctx, orc):
    """The full shape with the peers at 50 GB/s from rank 0: 7 peers x 4 bands = 28 producer workgroups
    beside the persistent consumer, twelve calls queued back to back; each call's P and C keep the bits of
    the resident-peer call (no flag wait may expire)."""
    w = I.MOE_RS
    Hg, W2, gate, logits, parts = make(w, "nk")
    ids, off, rt = orc.moe_route(logits, w.topk)
    rank = 0
    _, P0, C0, _, _ = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, rank, "nk")
    ng, npf = sgt.rs_flag_count(w.W, w.T, w.H, rs_tile=128)
    Y = torch.empty((w.T * w.topk, w.H), dtype=torch.float32, device="cuda:0")
    P = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda:0")
    C = torch.empty((w.T // w.W, w.H), dtype=torch.float32, device="cuda:0")
    gf = torch.zeros(ng, dtype=torch.int32, device="cuda:0")
    pf = torch.zeros(npf, dtype=torch.int32, device="cuda:0")
    dparts = [dev(p) if q != rank else None for q, p in enumerate(parts)]
    inbox = [torch.empty_like(p) if p is not None else None for p in dparts]
    args = (dev(Hg), dev(W2), dev(gate), dev(ids), dev(off), dev(rt), dparts, Y, P, C, gf, pf)
    for i in range(12):
        ctx.moe_gemm_rs(*args, rank=rank, b_layout="nk", inbox=inbox, peer_gbps=50.0, arrival_seed=i + 1)
    torch.cuda.synchronize()
    ctx.sync()
    assert np.array_equal(host(C).view(np.uint32), C0.view(np.uint32))
    assert np.array_equal(host(P).view(np.uint32), P0.view(np.uint32))
    e = host(gf)[0]
    assert (host(gf) == e).all()
    nb = npf // w.W   # peer flags, one block per rank; this rank's own block is never sent
    pfl = host(pf)
    for q in range(1, w.W):
        assert (pfl[q * nb:(q + 1) * nb] == e).all(), "peer %d flags" % q


@pytest.mark.slow
def test_full_moe_rs_shape(ctx, orc):
    w = I.MOE_RS
    Hg, W2, gate, logits, parts = make(w, "nk")
    ids, off, rt = orc.moe_route(logits, w.topk)
    rank = 3
    Y, P, C, gf, pf = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, rank, "nk")
    blk = w.T // w.W
    toks = sample_rows(blk, 1, per_shard=10, seed=4)
    C_ref = orc.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, rank, "nk", tokens=rank * blk + toks)
    assert_close(C[toks], C_ref, what="C", **TOL_BF16)
    other = sample_rows(w.T, w.W, per_shard=2, seed=5)
    assert_close(P[other], orc.moe_gemm_rs_p(Hg, W2, gate, ids, off, rt, other, "nk"), what="P", **TOL_BF16)
    assert (gf == gf[0]).all() and (pf == gf[0]).all()


@pytest.mark.parametrize("w_layout", ["kn", "nk"])
@pytest.mark.parametrize("shape", [(512, 4, 8, 2, 256, 512), (1024, 8, 16, 4, 136, 264)])
def test_moe_rs_bf16_y_parity(ctx, orc, shape, w_layout):
    """Y stored in bf16: Y within its rounding of the fp64 product, P and C within the bf16 tolerance (the
    combine sums the rounded rows), the same gathered flags as the fp32 call."""
    T, W, E, k, n_in, H = shape
    w = I.scaled(I.MOE_RS, T=T, W=W, E=E, topk=k, I=n_in, H=H, seed_index=33)
    Hg, W2, gate, logits, parts = make(w, w_layout)
    ids, off, rt = orc.moe_route(logits, k)
    rank = W - 1
    Y, P, C, gf, pf = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, rank, w_layout, y_dtype=torch.bfloat16)
    Y_ref = orc.moe_gemm(Hg, W2, off, np.arange(T * k, dtype=np.int32), w_layout)
    assert_close_bf16_out(Y, Y_ref, what="Y bf16")
    P_ref = orc.moe_gemm_rs_p(Hg, W2, gate, ids, off, rt, np.arange(T), w_layout)
    assert_close(P, P_ref, what="P (bf16 Y)", **TOL_BF16)
    C_ref = orc.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, rank, w_layout)
    assert_close(C, C_ref, what="C (bf16 Y)", **TOL_BF16)
    _, _, _, gf32, pf32 = run_moe_rs(ctx, Hg, W2, gate, ids, off, rt, parts, rank, w_layout)
    assert (gf == gf[0]).all() and (gf32 == gf32[0]).all()
