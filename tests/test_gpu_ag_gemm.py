"""GPU parity of the AllGather + GEMM path against the CPU oracle (through the C ABI)."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import (TOL_BF16, TOL_F32, assert_close, assert_close_bf16_out, dev, host, poison_like,  # noqa: E402
                      sample_rows, values)


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = sgt.Context(0)
    yield c
    c.close()


def run_ag(ctx, shards, B, *, out="f32", b_layout="kn", poison=True, **kw):
    """Upload, run sgt_ag_gemm (blocking), return (A_gathered, C, flags) on the host."""
    W = len(shards)
    R, K = shards[0].shape
    M = R * W
    N = B.shape[1] if b_layout == "kn" else B.shape[0]
    dA = [dev(s) for s in shards]
    dB = dev(B)
    in_dtype = sgt.SGT_BF16 if shards[0].dtype == np.uint16 else sgt.SGT_F32
    dt = torch.bfloat16 if in_dtype == sgt.SGT_BF16 else torch.float32
    Ag = torch.empty((M, K), dtype=dt, device="cuda:0")
    if poison:
        poison_like(Ag)
    C = torch.empty((M, N), dtype=torch.bfloat16 if out == "bf16" else torch.float32, device="cuda:0")
    poison_like(C)
    nf = sgt.ag_flag_count(W, M, K, in_dtype=in_dtype, flag_rows=kw.get("flag_rows", 0))
    flags = kw.pop("flags", None)
    if flags is None:
        flags = torch.zeros(max(nf, 4), dtype=torch.int32, device="cuda:0")
    ctx.ag_gemm(dA, dB, Ag, C, flags, b_layout=b_layout, blocking=True, **kw)
    torch.cuda.synchronize()
    return host(Ag), host(C), host(flags)[:nf]


# ---------------------------------------------------------------- fp32 tiny workload
@pytest.mark.parametrize("rank", [0, 2])
def test_tiny_f32_random_arrival(ctx, orc, rank):
    w = I.TINY
    shards, B = I.make_ag(w)
    A_ref, C_ref = orc.ag_gemm(shards, B)
    outs = []
    for seed in [0, 1, 2, 3, 4, 5]:
        Ag, C, fl = run_ag(ctx, shards, B, rank=rank, flag_rows=w.flag_rows, arrival_seed=seed,
                           arrival_order="global" if seed else "inorder", jitter_us=w.jitter_us,
                           peer_gbps=1.0 if seed % 2 else 0.0)
        assert np.array_equal(Ag, A_ref)
        assert len(fl) == w.M // w.flag_rows and (fl == fl[0]).all() and fl[0] > 0
        assert_close(C, C_ref, what="tiny f32 C", **TOL_F32)
        outs.append(C)
    for C in outs[1:]:
        assert np.array_equal(C.view(np.uint32), outs[0].view(np.uint32))


def test_tiny_f32_nk_and_bf16_out(ctx, orc):
    shards, B = I.make_ag(I.TINY)
    _, C_ref = orc.ag_gemm(shards, B)
    _, C, _ = run_ag(ctx, shards, np.ascontiguousarray(B.T), b_layout="nk", flag_rows=16)
    assert_close(C, C_ref, what="nk", **TOL_F32)
    _, Cb, _ = run_ag(ctx, shards, B, out="bf16", flag_rows=16)
    assert_close_bf16_out(Cb, C_ref, what="f32 in, bf16 out")


# ---------------------------------------------------------------- bf16 MFMA path
RAGGED = [
    # W, rows per shard, K, N, flag_rows
    (4, 200, 328, 392, 40),     # panels straddle shards, K tail of 8, N tail of 136
    (2, 256, 512, 256, 64),     # exact tiles
    (8, 96, 136, 72, 32),       # everything smaller than one tile
    (3, 300, 1032, 520, 100),   # odd W, 17 K steps (odd count), N tail of 8
]


@pytest.mark.parametrize("b_layout", ["kn", "nk"])
@pytest.mark.parametrize("shape", RAGGED)
def test_bf16_ragged_parity(ctx, orc, shape, b_layout):
    W, R, K, N, fr = shape
    w = I.AGWorkload("t", W=W, M=W * R, K=K, N=N, seed_index=11)
    shards, B = I.make_ag(w, B_layout=b_layout)
    A_ref, C_ref = orc.ag_gemm(shards, B, b_layout=b_layout)
    for rank in sorted({0, W - 1}):
        Ag, C, fl = run_ag(ctx, shards, B, b_layout=b_layout, rank=rank, flag_rows=fr, arrival_seed=rank + 3,
                           arrival_order="per_peer", jitter_us=20.0)
        assert np.array_equal(Ag, A_ref)
        assert (fl == fl[0]).all()
        assert_close(C, C_ref, what="bf16 %s %s rank %d" % (shape, b_layout, rank), **TOL_BF16)


def test_bf16_output_rounding(ctx, orc):
    w = I.AGWorkload("t", W=4, M=512, K=256, N=264, seed_index=12)
    shards, B = I.make_ag(w)
    _, C_ref = orc.ag_gemm(shards, B)
    _, C, _ = run_ag(ctx, shards, B, out="bf16", flag_rows=32)
    assert_close_bf16_out(C, C_ref, what="bf16 out")


@pytest.mark.parametrize("b_layout", ["kn", "nk"])
def test_identity_B_is_bit_exact(ctx, b_layout):
    """B = I: each output is one exact product, so C must equal the gathered rows exactly."""
    W, R, K = 8, 160, 520
    w = I.AGWorkload("t", W=W, M=W * R, K=K, N=K, seed_index=13)
    shards, _ = I.make_ag(w)
    eye = I.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    Ag, C, _ = run_ag(ctx, shards, eye, b_layout=b_layout, rank=5, flag_rows=32, arrival_seed=9,
                      arrival_order="global")
    assert np.array_equal(C, values(np.concatenate(shards)).astype(np.float32))


def test_integer_inputs_are_bit_exact(ctx, orc):
    """Integer inputs in [-3, 3]: every partial sum is an exact fp32 integer."""
    w = I.AGWorkload("t", W=4, M=4 * 264, K=1000, N=584, dist="int", seed_index=14)
    shards, B = I.make_ag(w)
    _, C_ref = orc.ag_gemm(shards, B)
    for order in ["mesh", "shard"]:
        _, C, _ = run_ag(ctx, shards, B, rank=1, flag_rows=24, order=order, arrival_seed=2, arrival_order="per_peer")
        assert np.array_equal(C.astype(np.float64), C_ref)


def test_bits_invariant_across_modes(ctx):
    """Arrival order, jitter, pacing, producer mode, consumer order and rank change timing only."""
    w = I.AGWorkload("t", W=8, M=8 * 256, K=768, N=512, seed_index=15)
    shards, B = I.make_ag(w)
    ref = None
    for kw in [dict(producer="serial"), dict(producer="cu"),
               dict(producer="cu", arrival_seed=5, jitter_us=30.0, arrival_order="per_peer"),
               dict(producer="cu", arrival_seed=6, jitter_us=5.0, arrival_order="global", peer_gbps=40.0),
               dict(producer="cu", peer_gbps=20.0, order="shard", rank=3),
               dict(producer="cu", rank=7, producer_cus=3, consumer_cus=17), dict(producer="cu", flag_rows=256)]:
        kw.setdefault("flag_rows", 64)
        Ag, C, _ = run_ag(ctx, shards, B, **kw)
        if ref is None:
            ref = (Ag, C)
        assert np.array_equal(Ag, ref[0])
        assert np.array_equal(C.view(np.uint32), ref[1].view(np.uint32)), kw
    # gathered data already resident, flags preset: the GEMM alone gives the same bits
    dA = [dev(s) for s in shards]
    Ag = dev(np.concatenate(shards))
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
    flags = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    ctx.ag_gemm(dA, dev(B), Ag, C, flags, producer="preset", flag_rows=64, blocking=True)
    assert np.array_equal(host(C).view(np.uint32), ref[1].view(np.uint32))


def test_flags_hold_the_epoch_and_are_reused(ctx):
    """Flags are zeroed once; each call's epoch is one more than the last."""
    w = I.AGWorkload("t", W=4, M=4 * 64, K=64, N=64, seed_index=16)
    shards, B = I.make_ag(w)
    flags = torch.zeros(16, dtype=torch.int32, device="cuda:0")
    seen = []
    for _ in range(3):
        _, _, fl = run_ag(ctx, shards, B, flag_rows=16, flags=flags)
        assert (fl == fl[0]).all()
        seen.append(int(fl[0]))
    assert seen[1] == seen[0] + 1 and seen[2] == seen[1] + 1


def test_withheld_peer_times_out_and_recovers(ctx):
    """A peer whose tiles are never signalled: every wait ends at its bound, the call reports it."""
    w = I.AGWorkload("t", W=4, M=4 * 128, K=128, N=256, seed_index=17)
    shards, B = I.make_ag(w)
    with pytest.raises(sgt.SgtError) as ei:
        run_ag(ctx, shards, B, flag_rows=32, withhold_peer=2, timeout_ms=20.0)
    assert ei.value.status == sgt.SGT_ETIMEDOUT
    # the next call on the same context succeeds
    Ag, C, fl = run_ag(ctx, shards, B, flag_rows=32)
    assert np.isfinite(C).all() and (fl == fl[0]).all()


def test_degenerate_shapes(ctx, orc):
    # a single shard (W = 1): only local data
    w = I.AGWorkload("t", W=1, M=96, K=64, N=40, seed_index=18)
    shards, B = I.make_ag(w)
    _, C_ref = orc.ag_gemm(shards, B)
    _, C, _ = run_ag(ctx, shards, B, flag_rows=32)
    assert_close(C, C_ref, what="W=1", **TOL_BF16)
    # M = 0 is a no-op; N = 0 still gathers
    dA = [torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0") for _ in range(2)]
    ctx.ag_gemm(dA, dev(B), torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0"),
                torch.empty((0, 40), dtype=torch.float32, device="cuda:0"),
                torch.zeros(4, dtype=torch.int32, device="cuda:0"), blocking=True)
    shards2, _ = I.make_ag(I.AGWorkload("t", W=2, M=64, K=64, N=8, seed_index=19))
    B0 = torch.empty((64, 0), dtype=torch.bfloat16, device="cuda:0")
    Ag = torch.empty((64, 64), dtype=torch.bfloat16, device="cuda:0")
    ctx.ag_gemm([dev(s) for s in shards2], B0, Ag, torch.empty((64, 0), dtype=torch.float32, device="cuda:0"),
                torch.zeros(4, dtype=torch.int32, device="cuda:0"), flag_rows=16, blocking=True)
    assert np.array_equal(host(Ag), np.concatenate(shards2))


def test_bad_arguments_are_rejected_before_launch(ctx):
    shards, B = I.make_ag(I.AGWorkload("t", W=4, M=256, K=64, N=64, seed_index=20))
    dA = [dev(s) for s in shards]
    Ag = torch.empty((256, 64), dtype=torch.bfloat16, device="cuda:0")
    C = torch.empty((256, 64), dtype=torch.float32, device="cuda:0")
    flags = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    with pytest.raises(sgt.SgtError) as e:
        ctx.ag_gemm(dA, dev(B), Ag, C, flags, flag_rows=48)        # 64 rows per shard, 48 does not divide
    assert e.value.status == sgt.SGT_EINVAL
    with pytest.raises(sgt.SgtError):
        ctx.ag_gemm(dA, dev(B), Ag, C, flags, rank=4)               # rank outside [0, W)
    with pytest.raises(sgt.SgtError):
        ctx.ag_gemm(dA[:3], dev(B), Ag[:254], C[:254], flags)       # M = 254 is not a multiple of W = 3


# ---------------------------------------------------------------- full-size workloads
def _full_size(ctx, orc, w, b_layout, dist):
    w = I.scaled(w, dist=dist)
    shards, B = I.make_ag(w, B_layout=b_layout)
    rows = sample_rows(w.M, w.W, per_shard=4, seed=w.seed_index)
    A_ref, C_rows = orc.ag_gemm(shards, B, b_layout=b_layout, rows=rows)
    Ag, C, fl = run_ag(ctx, shards, B, b_layout=b_layout, rank=3, peer_gbps=w.peer_gbps, jitter_us=w.jitter_us,
                       arrival_seed=1)
    assert np.array_equal(Ag, A_ref)
    assert (fl == fl[0]).all()
    if dist == "int":
        assert np.array_equal(C[rows].astype(np.float64), C_rows)
    else:
        assert_close(C[rows], C_rows, what=w.name, **TOL_BF16)
    # every row: C @ 1 = A @ (B @ 1), within the worst-case fp32 accumulation bound
    # K * 2^-24 * sum_j sum_k |a_ik| |b_kj| (exact for integer inputs)
    Bv = values(B)
    if b_layout == "nk":
        Bv = Bv.T
    Av = values(A_ref)
    lhs = C.astype(np.float64).sum(axis=1)
    rhs = Av @ Bv.sum(axis=1)
    bound = w.K * 2.0 ** -24 * (np.abs(Av) @ np.abs(Bv).sum(axis=1)) + 1e-9
    if dist == "int":
        assert np.array_equal(lhs, rhs)
    assert (np.abs(lhs - rhs) <= bound).all()


@pytest.mark.slow
@pytest.mark.parametrize("dist", ["normal", "int"])
def test_full_llama_shape(ctx, orc, dist):
    _full_size(ctx, orc, I.LLAMA_AG, "kn", dist)


@pytest.mark.slow
@pytest.mark.parametrize("b_layout", ["kn", "nk"])
def test_full_qwen_shape(ctx, orc, b_layout):
    _full_size(ctx, orc, I.QWEN_AG, b_layout, "normal")


# ---------------------------------------------------------------- K-chunked signal tiles
def _run_kc(ctx, dA, dB, M, K, N, b_layout, **kw):
    W = len(dA)
    Ag = poison_like(torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0"))
    C = poison_like(torch.empty((M, N), dtype=torch.float32, device="cuda:0"))
    nf = sgt.ag_flag_count(W, M, K, k_chunks=kw.get("k_chunks", 0))
    flags = torch.zeros(nf, dtype=torch.int32, device="cuda:0")
    ctx.ag_gemm(dA, dB, Ag, C, flags, b_layout=b_layout, blocking=True, **kw)
    torch.cuda.synchronize()
    return Ag, C, flags


@pytest.mark.parametrize("b_layout", ["nk", "kn"])
@pytest.mark.parametrize("link", [dict(peer_gbps=4.0, jitter_us=30.0, arrival_seed=3), dict(),
                                  dict(peer_gbps=4.0, arrival_seed=9, arrival_order="global")])
def test_k_chunks_are_bit_identical_to_whole_rows(ctx, orc, b_layout, link):
    """Signal tiles of one panel x one K chunk: with slow, jittered links most remote tiles start on a panel
    whose later chunks are still in flight (B stored N x K: chunk by chunk; K x N: after the whole panel).
    Gathered bits, C bits and the flags (all at the call's epoch) match the whole-row signal tiles."""
    w = I.AGWorkload("t", W=4, M=4 * 512, K=1024, N=520, seed_index=34)
    shards, B = I.make_ag(w, B_layout=b_layout)
    dA, dB = [dev(s) for s in shards], dev(B)
    assert sgt.ag_flag_count(w.W, w.M, w.K, k_chunks=8) == (w.M // 256) * 8
    Ag0, C0, _ = _run_kc(ctx, dA, dB, w.M, w.K, w.N, b_layout, rank=2, **link)
    Ag1, C1, fl = _run_kc(ctx, dA, dB, w.M, w.K, w.N, b_layout, rank=2, k_chunks=8, **link)
    assert torch.equal(Ag1.view(torch.int16), torch.cat(dA).view(torch.int16)), "gathered buffer"
    assert torch.equal(C1.view(torch.int32), C0.view(torch.int32)), "C bits differ from whole-row signal tiles"
    f = fl.cpu().numpy()
    assert (f == f[0]).all() and f[0] > 0
    _, C_ref = orc.ag_gemm(shards, B, b_layout=b_layout, rows=sample_rows(w.M, w.W))
    assert_close(host(C1)[sample_rows(w.M, w.W)], C_ref, what="k-chunked C", **TOL_BF16)


@pytest.mark.slow
def test_k_chunks_full_llama_shape(ctx):
    """The Llama-3-70B share with 8 K chunks per panel at 153.6 GB/s per link + jitter: the same C bits as the
    whole-row signal tiles."""
    w = I.LLAMA_AG
    shards, B = I.make_ag(w, B_layout="nk")
    dA, dB = [dev(s) for s in shards], dev(B)
    link = dict(peer_gbps=w.peer_gbps, jitter_us=w.jitter_us, arrival_seed=5)
    _, C0, _ = _run_kc(ctx, dA, dB, w.M, w.K, w.N, "nk", **link)
    Ag1, C1, fl = _run_kc(ctx, dA, dB, w.M, w.K, w.N, "nk", k_chunks=8, **link)
    assert torch.equal(C1.view(torch.int32), C0.view(torch.int32))
    assert torch.equal(Ag1.view(torch.int16), torch.cat(dA).view(torch.int16))
    assert bool((fl == fl[0]).all())


def test_k_chunks_rejections(ctx):
    w = I.AGWorkload("t", W=4, M=4 * 256, K=1024, N=256, seed_index=35)
    shards, B = I.make_ag(w, B_layout="nk")
    dA, dB = [dev(s) for s in shards], dev(B)
    for kw in (dict(k_chunks=3),                      # 1024 is not a multiple of 128 x 3
               dict(k_chunks=65)):                    # above 64
        with pytest.raises(sgt.SgtError):
            _run_kc(ctx, dA, dB, w.M, w.K, w.N, "nk", **kw)
    w2 = I.AGWorkload("t", W=4, M=4 * 200, K=1024, N=256, seed_index=35)   # shards of 200 rows: not whole panels
    s2, B2 = I.make_ag(w2, B_layout="nk")
    with pytest.raises(sgt.SgtError):
        sgt.ag_flag_count(w2.W, w2.M, w2.K, k_chunks=8)
    g = torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(sgt.SgtError):
        ctx.allgather(dA, g, torch.zeros(64, dtype=torch.int32, device="cuda:0"), k_chunks=8, blocking=True)


@pytest.mark.slow
def test_k_chunks_full_qwen_shape(ctx):
    """The Qwen3-32B share (K = 5120: 8 chunks of 640 columns) at 50 GB/s per link: the same C bits as the
    whole-row signal tiles."""
    w = I.QWEN_AG
    shards, B = I.make_ag(w, B_layout="nk")
    dA, dB = [dev(s) for s in shards], dev(B)
    link = dict(peer_gbps=w.peer_gbps, arrival_seed=2)
    _, C0, _ = _run_kc(ctx, dA, dB, w.M, w.K, w.N, "nk", rank=5, **link)
    Ag1, C1, fl = _run_kc(ctx, dA, dB, w.M, w.K, w.N, "nk", rank=5, k_chunks=8, **link)
    assert torch.equal(C1.view(torch.int32), C0.view(torch.int32))
    assert torch.equal(Ag1.view(torch.int16), torch.cat(dA).view(torch.int16))
    assert bool((fl == fl[0]).all())


# ---------------------------------------------------------------- copy-engine producer
@pytest.mark.parametrize("k_chunks", [0, 8])
@pytest.mark.parametrize("sdma", [dict(producer="sdma"), dict(producer="sdma", sdma_peers=1, producer_cus=8)],
                         ids=["engines", "engines+cu"])
def test_sdma_producer_bits_match_cu_producer(ctx, orc, k_chunks, sdma):
    """The copy engines move the shards (or, with sdma_peers, the first peers' shards while CU workgroups move the
    rest); the releaser publishes each signal tile once its copy has landed and its link time has come.  Gathered
    bits, C bits and flags equal those of the CU producer under the same slow, jittered links."""
    w = I.AGWorkload("t", W=4, M=4 * 512, K=1024, N=520, seed_index=36)
    shards, B = I.make_ag(w, B_layout="nk")
    dA, dB = [dev(s) for s in shards], dev(B)
    link = dict(peer_gbps=8.0, jitter_us=20.0, arrival_seed=4, rank=1, k_chunks=k_chunks)
    _, C0, _ = _run_kc(ctx, dA, dB, w.M, w.K, w.N, "nk", **link)
    for rep in range(2):   # the second call reuses the context's copy-engine state
        Ag1, C1, fl = _run_kc(ctx, dA, dB, w.M, w.K, w.N, "nk", **link, **sdma)
        assert torch.equal(Ag1.view(torch.int16), torch.cat(dA).view(torch.int16)), "gathered buffer"
        assert torch.equal(C1.view(torch.int32), C0.view(torch.int32)), "C bits differ from the CU producer"
        f = fl.cpu().numpy()
        assert (f == f[0]).all() and f[0] > 0
    rows = sample_rows(w.M, w.W)
    _, C_ref = orc.ag_gemm(shards, B, b_layout="nk", rows=rows)
    assert_close(host(C1)[rows], C_ref, what="copy-engine C", **TOL_BF16)


def test_sdma_producer_tiny_f32(ctx, orc):
    w = I.TINY
    shards, B = I.make_ag(w)
    A_ref, C_ref = orc.ag_gemm(shards, B)
    Ag, C, fl = run_ag(ctx, shards, B, rank=3, flag_rows=w.flag_rows, producer="sdma", arrival_seed=2,
                       arrival_order="global", jitter_us=w.jitter_us)
    assert np.array_equal(Ag, A_ref)
    assert (fl == fl[0]).all() and fl[0] > 0
    assert_close(C, C_ref, what="tiny f32 C, copy engines", **TOL_F32)


def test_sdma_producer_withheld_peer_times_out(ctx):
    w = I.AGWorkload("t", W=4, M=4 * 256, K=512, N=256, seed_index=37)
    shards, B = I.make_ag(w)
    with pytest.raises(sgt.SgtError) as ei:
        run_ag(ctx, shards, B, producer="sdma", withhold_peer=2, timeout_ms=30.0)
    assert ei.value.status == sgt.SGT_ETIMEDOUT
    Ag, C, _ = run_ag(ctx, shards, B, producer="sdma")   # the context stays usable
    assert np.array_equal(Ag, np.concatenate(shards))


def test_sdma_producer_only_for_ag_gemm(ctx):
    w = I.RSWorkload("t", W=4, M=1024, K=64, N=256, seed_index=38)
    A, B, parts = I.make_rs(w)
    ng, npf = sgt.rs_flag_count(w.W, w.M, w.N)
    with pytest.raises(sgt.SgtError) as ei:
        ctx.gemm_rs(dev(A), dev(B), [dev(p) for p in parts], torch.empty((w.M, w.N), device="cuda:0"),
                    torch.empty((w.M // w.W, w.N), device="cuda:0"), torch.zeros(ng, dtype=torch.int32, device="cuda:0"),
                    torch.zeros(npf, dtype=torch.int32, device="cuda:0"), producer="sdma", blocking=True)
    assert ei.value.status == sgt.SGT_EUNSUPPORTED


# ---------------------------------------------------------------- stream order after an overlapped call
@pytest.mark.parametrize("producer", ["cu", "sdma"])
def test_stream_order_covers_the_whole_allgather(ctx, orc, producer):
    """After a non-blocking overlapped call, work queued on the caller's stream sees the whole gathered buffer,
    the local shard's copy (the producer's last items, which the consumer never waits on) included: the
    bf16 consumer joins the producer on the GPU, the copy-engine path with an event.  The check runs on the
    caller's stream before any synchronization, for several calls back to back."""
    w = I.AGWorkload("t", W=8, M=4096, K=2048, N=256, seed_index=52)
    shards, B = I.make_ag(w, B_layout="nk")
    dA = [dev(s) for s in shards]
    dB = dev(B)
    Ag = torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda:0")
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
    flags = torch.zeros(sgt.ag_flag_count(w.W, w.M, w.K), dtype=torch.int32, device="cuda:0")
    ref = torch.cat(dA).view(torch.int16)
    oks = []
    for i in range(4):
        poison_like(Ag)
        ctx.ag_gemm(dA, dB, Ag, C, flags, rank=3, b_layout="nk", producer=producer, arrival_seed=i + 1)
        oks.append(torch.equal(Ag.view(torch.int16), ref))   # queued on the caller's stream
    torch.cuda.synchronize()
    ctx.sync()
    assert all(oks)
    rows = sample_rows(w.M, w.W, per_shard=2, seed=3)
    _, C_ref = orc.ag_gemm(shards, B, b_layout="nk", rows=rows)
    assert_close(host(C)[rows], C_ref, what="C", **TOL_BF16)
