"""GPU parity of the MoE AllGather + grouped GEMM against the CPU oracle.

Routing tables (top-k ids, expert offsets, grouped row tokens) and the gathered
tokens are integer or byte results: bit-exact.  Y is checked to the bf16
tolerance of the workload definition, or exactly for integer-valued inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import TOL_BF16, assert_close, assert_close_bf16_out, dev, host, poison_like, values  # noqa: E402


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = sgt.Context(0)
    yield c
    c.close()


def run_moe(ctx, shards, We, logits, topk, *, w_layout="kn", out="f32", flags=None, Xg=None, poison=True, **kw):
    """Upload, run sgt_moe_ag_gemm (blocking); return host copies of
    (X_gathered, Y, topk_ids, expert_off, row_token, flags)."""
    W = len(shards)
    R, H = shards[0].shape
    T = R * W
    E = We.shape[0]
    Icols = We.shape[2] if w_layout == "kn" else We.shape[1]
    dX = [dev(s) for s in shards]
    dW = dev(We)
    dL = dev(logits)
    if Xg is None:
        Xg = torch.empty((T, H), dtype=torch.bfloat16, device="cuda:0")
        if poison:
            poison_like(Xg)
    Y = torch.empty((T * topk, Icols), dtype=torch.bfloat16 if out == "bf16" else torch.float32, device="cuda:0")
    poison_like(Y)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda:0")
    rt = torch.full((T * topk,), -7, dtype=torch.int32, device="cuda:0")
    ids = torch.full((T, topk), -7, dtype=torch.int32, device="cuda:0")
    nf = sgt.ag_flag_count(W, T, H, flag_rows=kw.get("flag_rows", 0))
    if flags is None:
        flags = torch.zeros(max(nf, 4), dtype=torch.int32, device="cuda:0")
    ctx.moe_ag_gemm(dX, dW, dL, Xg, Y, off, rt, ids, flags, topk=topk, b_layout=w_layout, blocking=True, **kw)
    torch.cuda.synchronize()
    return host(Xg), host(Y), host(ids), host(off), host(rt), host(flags)[:nf]


def check_moe(orc, shards, We, logits, topk, res, w_layout="kn", out="f32", exact=False, what=""):
    Xg, Y, ids, off, rt, _ = res
    X_ref, ids_ref, off_ref, rt_ref, Y_ref = orc.moe_ag_gemm(shards, We, logits, topk, w_layout=w_layout)
    assert np.array_equal(Xg, X_ref), what + ": gathered tokens differ"
    assert np.array_equal(ids, ids_ref), what + ": top-k ids differ"
    assert np.array_equal(off, off_ref), what + ": expert offsets differ"
    assert np.array_equal(rt, rt_ref), what + ": grouped row tokens differ"
    if exact:
        assert np.array_equal(values(Y), Y_ref), what + ": integer-valued Y not exact"
    elif out == "bf16":
        assert_close_bf16_out(Y, Y_ref, what=what)
    else:
        assert_close(Y, Y_ref, what=what, **TOL_BF16)


SMALL = [
    # W, T, H, I, E, topk, flag_rows
    (4, 256, 256, 192, 16, 4, 16),      # one row tile per expert, I tail of 192
    (8, 1024, 264, 320, 64, 8, 32),     # Zipf groups beyond 256 rows, H tail of 8, I tail of 64
    (2, 600, 128, 256, 5, 2, 100),      # E not a multiple of 64, shards of 300 tokens
    (4, 512, 128, 128, 40, 12, 32),     # top-k above 8 (the wave-per-token selection)
]
TILES = [(128, 8), (256, 8), (128, 4)]   # (tile rows, waves per workgroup)


@pytest.mark.parametrize("tile", TILES, ids=["r%dw%d" % t for t in TILES])
@pytest.mark.parametrize("shape", SMALL)
@pytest.mark.parametrize("w_layout", ["kn", "nk"])
def test_moe_parity_overlapped(ctx, orc, shape, w_layout, tile):
    W, T, H, Ic, E, k, fr = shape
    w = I.scaled(I.MOE, W=W, T=T, H=H, I=Ic, E=E, topk=k)
    shards, We, logits = I.make_moe(w, W_layout=w_layout)
    res = run_moe(ctx, shards, We, logits, k, w_layout=w_layout, flag_rows=fr, peer_gbps=20.0, jitter_us=5.0,
                  arrival_seed=3, rank=W - 1, tile_rows=tile[0], tile_waves=tile[1])
    check_moe(orc, shards, We, logits, k, res, w_layout=w_layout, what="moe %s %s %s" % (shape, w_layout, tile))
    assert (res[5] == res[5][0]).all() and res[5][0] > 0


@pytest.mark.parametrize("mode", ["serial", "preset"])
def test_moe_modes_and_bf16_out(ctx, orc, mode):
    W, T, H, Ic, E, k = 8, 1024, 256, 256, 64, 8
    w = I.scaled(I.MOE, W=W, T=T, H=H, I=Ic, E=E, topk=k)
    shards, We, logits = I.make_moe(w, salt=1)
    Xg = None
    if mode == "preset":  # the gathered buffer must already hold every shard
        Xg = dev(np.concatenate(shards, axis=0))
    res = run_moe(ctx, shards, We, logits, k, producer=mode, out="bf16", Xg=Xg)
    check_moe(orc, shards, We, logits, k, res, out="bf16", what="moe " + mode)


def test_moe_integer_inputs_exact(ctx, orc):
    w = I.scaled(I.MOE, W=4, T=512, H=128, I=256, E=8, topk=3, dist="int")
    shards, We, logits = I.make_moe(w)
    res = run_moe(ctx, shards, We, logits, 3, flag_rows=32, peer_gbps=10.0, arrival_order="global", arrival_seed=7)
    check_moe(orc, shards, We, logits, 3, res, exact=True, what="integer moe")


def test_moe_tied_logits(ctx, orc):
    """Many equal logits: the lower expert id must win every tie."""
    W, T, H, Ic, E, k = 4, 256, 64, 64, 12, 4
    w = I.scaled(I.MOE, W=W, T=T, H=H, I=Ic, E=E, topk=k)
    shards, We, _ = I.make_moe(w)
    rng = np.random.default_rng(5)
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    logits[::7, 0::2] = -0.0   # -0 and +0 compare equal: in these rows the lowest ids win
    logits[::7, 1::2] = 0.0
    res = run_moe(ctx, shards, We, logits, k, flag_rows=16)
    check_moe(orc, shards, We, logits, k, res, what="ties")


def test_moe_single_expert_is_allgather_gemm(ctx, orc):
    """E = 1, k = 1: every token goes to the one expert in token order, so Y = X_gathered * W_0."""
    w = I.scaled(I.MOE, W=4, T=512, H=256, I=192, E=1, topk=1)
    shards, We, logits = I.make_moe(w)
    res = run_moe(ctx, shards, We, logits, 1, flag_rows=32, peer_gbps=20.0)
    Xg, Y, ids, off, rt, _ = res
    assert np.array_equal(off, [0, 512]) and np.array_equal(rt, np.arange(512)) and (ids == 0).all()
    _, C_ref = orc.ag_gemm(shards, We[0])
    assert_close(Y, C_ref, what="E=1 moe vs AG-GEMM", **TOL_BF16)


def test_moe_repeat_reuses_flags(ctx, orc):
    """Flags are never reset between calls: the epoch advances; a new routing each call."""
    w = I.scaled(I.MOE, W=4, T=256, H=128, I=128, E=16, topk=4)
    nf = sgt.ag_flag_count(4, 256, 128, flag_rows=16)
    flags = torch.zeros(nf, dtype=torch.int32, device="cuda:0")
    last = None
    for salt in (0, 1, 2):
        shards, We, logits = I.make_moe(w, salt=salt)
        res = run_moe(ctx, shards, We, logits, 4, flag_rows=16, flags=flags, peer_gbps=5.0, arrival_seed=salt)
        check_moe(orc, shards, We, logits, 4, res, what="repeat %d" % salt)
        fl = res[5]
        assert (fl == fl[0]).all()
        if last is not None:
            assert fl[0] > last
        last = fl[0]


def test_moe_expert_count_changes_between_calls(ctx, orc):
    """One context, successive calls with fewer and more experts: every call's routing tables must be
    exact whatever the previous call routed (the per-expert counts are reused across calls)."""
    for (E, k) in [(5, 2), (200, 12), (3, 3), (64, 8), (256, 1)]:
        w = I.scaled(I.MOE, W=2, T=384, H=64, I=64, E=E, topk=k)
        shards, We, logits = I.make_moe(w, salt=E)
        res = run_moe(ctx, shards, We, logits, k, flag_rows=32, peer_gbps=10.0, arrival_seed=E)
        check_moe(orc, shards, We, logits, k, res, what="E=%d k=%d" % (E, k))


def test_moe_bits_independent_of_arrival(ctx):
    """The order in which tiles land and are claimed changes no bit of the results."""
    w = I.scaled(I.MOE, W=8, T=1024, H=256, I=256, E=64, topk=8)
    shards, We, logits = I.make_moe(w, salt=2)
    outs = []
    for kw in (dict(producer="preset"), dict(producer="serial"),
               dict(peer_gbps=10.0, arrival_order="global", arrival_seed=1, jitter_us=20.0),
               dict(peer_gbps=10.0, arrival_order="per_peer", arrival_seed=2, rank=5)):
        Xg = dev(np.concatenate(shards, axis=0)) if kw.get("producer") == "preset" else None
        outs.append(run_moe(ctx, shards, We, logits, 8, flag_rows=32, Xg=Xg, **kw))
    for o in outs[1:]:
        for a, b in zip(o[:5], outs[0][:5]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_moe_trace_covers_every_item(ctx, orc):
    """A traced overlapped call: one record per work item of the list (row tiles x column tiles), each with
    wait <= flags seen <= end, its workgroup and a plausible engine-clock cycle count; nothing past the list;
    a release time for every signal tile.  The results stay those of the oracle."""
    W, T, H, Ic, E, k = 8, 1024, 256, 768, 64, 8
    w = I.scaled(I.MOE, W=W, T=T, H=H, I=Ic, E=E, topk=k)
    shards, We, logits = I.make_moe(w, salt=3, W_layout="nk")
    nw = sgt.moe_trace_words(W, T, H, Ic, E, k, b_layout="nk")
    tr = torch.zeros(nw, dtype=torch.int64, device="cuda:0")
    res = run_moe(ctx, shards, We, logits, k, w_layout="nk", peer_gbps=10.0, trace=tr.data_ptr())
    check_moe(orc, shards, We, logits, k, res, w_layout="nk", what="traced moe")
    off = res[3]
    groups = np.diff(off.astype(np.int64))
    n_items = int(np.sum((groups + 255) // 256)) * (Ic // 256)
    nf = sgt.ag_flag_count(W, T, H)
    t = host(tr).astype(np.uint64)
    rec = t[: n_items * 4].reshape(-1, 4)
    wait, seen, end = rec[:, 0].astype(np.int64), rec[:, 1].astype(np.int64), rec[:, 2].astype(np.int64)
    assert (wait > 0).all() and (seen >= wait).all() and (end > seen).all(), "an item is missing or out of order"
    wg = (rec[:, 3] & np.uint64(0xFFFF)).astype(np.int64)
    cyc = (rec[:, 3] >> np.uint64(16)).astype(np.float64)
    assert (wg < 1024).all() and (cyc > 0).all()
    mhz = cyc / ((end - wait) / 100.0)   # the 100 MHz clock: (end - wait) / 100 microseconds
    assert (mhz > 300).all() and (mhz < 3000).all(), (mhz.min(), mhz.max())
    assert not t[n_items * 4: nw - nf].any(), "records past the work list"
    assert (t[nw - nf:] > 0).all(), "a signal tile without a release time"


def test_moe_withheld_peer_times_out(ctx):
    w = I.scaled(I.MOE, W=4, T=256, H=64, I=64, E=8, topk=2)
    shards, We, logits = I.make_moe(w)
    with pytest.raises(sgt.SgtError) as ei:
        run_moe(ctx, shards, We, logits, 2, flag_rows=16, withhold_peer=2, timeout_ms=50.0)
    assert ei.value.status == sgt.SGT_ETIMEDOUT
    # the context stays usable
    res = run_moe(ctx, shards, We, logits, 2, flag_rows=16)
    assert (res[5] > 0).all()


def test_moe_degenerate(ctx, orc):
    # I = 0: routing and the gather still happen, Y is empty
    w = I.scaled(I.MOE, W=2, T=128, H=64, I=8, E=4, topk=2)
    shards, We, logits = I.make_moe(w)
    We0 = np.zeros((4, 64, 0), np.uint16)
    Xg, Y, ids, off, rt, _ = run_moe(ctx, shards, We0, logits, 2, flag_rows=16)
    X_ref, ids_ref, off_ref, rt_ref, _ = orc.moe_ag_gemm(shards, We, logits, 2)
    assert Y.shape == (256, 0)
    assert np.array_equal(Xg, X_ref) and np.array_equal(ids, ids_ref) and np.array_equal(off, off_ref)
    assert np.array_equal(rt, rt_ref)
    # topk = E: every token in every group
    res = run_moe(ctx, shards, We, logits, 4, flag_rows=16)
    check_moe(orc, shards, We, logits, 4, res, what="topk = E")


def test_moe_bad_args(ctx):
    w = I.scaled(I.MOE, W=2, T=128, H=64, I=64, E=4, topk=2)
    shards, We, logits = I.make_moe(w)
    with pytest.raises(sgt.SgtError):
        run_moe(ctx, shards, We, logits, 5)          # topk > E
    with pytest.raises(sgt.SgtError):
        run_moe(ctx, shards, We, logits, 2, flag_rows=48)   # does not divide 64 rows per shard
    with pytest.raises(sgt.SgtError):
        run_moe(ctx, shards, We, logits, 2, tile_rows=64)   # 128 or 256 only
    bad = [s[:, :60].copy() for s in shards]         # H % 8 != 0
    with pytest.raises(sgt.SgtError):
        run_moe(ctx, bad, We[:, :60].copy(), logits, 2)


@pytest.mark.slow
@pytest.mark.parametrize("tile_rows", [128, 256])
@pytest.mark.parametrize("w_layout", ["kn", "nk"])
def test_moe_full_shape(ctx, orc, w_layout, tile_rows):
    """The full workload (T 4096, H 2048, I 768, 64 experts, top-8), overlapped at 50 GB/s per peer:
    routing tables and the gathered tokens in full, Y on sampled rows."""
    w = I.MOE
    shards, We, logits = I.make_moe(w, W_layout=w_layout)
    res = run_moe(ctx, shards, We, logits, w.topk, w_layout=w_layout, peer_gbps=w.peer_gbps, arrival_seed=1,
                  tile_rows=tile_rows)
    Xg, Y, ids, off, rt, _ = res
    X_ref = np.concatenate(shards, axis=0)
    ids_ref, off_ref, rt_ref = orc.moe_route(logits, w.topk)
    assert np.array_equal(Xg, X_ref) and np.array_equal(ids, ids_ref)
    assert np.array_equal(off, off_ref) and np.array_equal(rt, rt_ref)
    rng = np.random.default_rng(0)
    rows = set()
    for e in range(w.E):  # first and last row of every group, plus random rows
        if off_ref[e + 1] > off_ref[e]:
            rows |= {int(off_ref[e]), int(off_ref[e + 1]) - 1}
    rows |= set(int(r) for r in rng.integers(0, w.T * w.topk, size=200))
    rows = np.array(sorted(rows), np.int64)
    Y_ref = orc.moe_gemm(X_ref, We, off_ref, rt_ref, w_layout=w_layout, rows=rows)
    assert_close(Y[rows], Y_ref, what="full moe sampled rows", **TOL_BF16)
