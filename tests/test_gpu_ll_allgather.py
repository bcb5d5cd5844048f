"""GPU parity of the stand-alone AllGather calls against the CPU oracle (through the C ABI).

sgt_ll_allgather (low-latency packets) and sgt_allgather (a flag per chunk)
must both leave the gathered buffer equal, bit for bit, to the oracle's row
concatenation; the LL call must leave in its receive buffer exactly the
packets the oracle's packing gives for the call's epoch, and the flag call
every flag at that epoch.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import dev, host, poison_like  # noqa: E402


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = sgt.Context(0)
    yield c
    c.close()


def _in_dtype(shards):
    return sgt.SGT_BF16 if shards[0].dtype == np.uint16 else sgt.SGT_F32


def run_ll(ctx, shards, ll_buf=None, **kw):
    """Upload, run sgt_ll_allgather (blocking); return (gathered, LL buffer as uint64 words, buffer)."""
    W = len(shards)
    R, K = shards[0].shape
    M = R * W
    in_dtype = _in_dtype(shards)
    G = poison_like(torch.empty((M, K), dtype=torch.bfloat16 if in_dtype == sgt.SGT_BF16 else torch.float32,
                                device="cuda:0"))
    if ll_buf is None:
        nb = sgt.ll_buffer_bytes(W, M, K, in_dtype=in_dtype, flag_rows=kw.get("flag_rows", 0))
        ll_buf = torch.zeros(max(nb // 8, 2), dtype=torch.int64, device="cuda:0")
    print("ll_allgather W=%d M=%d K=%d %s" % (W, M, K, kw), flush=True)
    ctx.ll_allgather([dev(s) for s in shards], ll_buf, G, blocking=True, **kw)
    torch.cuda.synchronize()
    return host(G), ll_buf.cpu().numpy().view(np.uint64).copy(), ll_buf


def run_flag(ctx, shards, flags=None, **kw):
    W = len(shards)
    R, K = shards[0].shape
    M = R * W
    in_dtype = _in_dtype(shards)
    G = poison_like(torch.empty((M, K), dtype=torch.bfloat16 if in_dtype == sgt.SGT_BF16 else torch.float32,
                                device="cuda:0"))
    nf = sgt.ag_flag_count(W, M, K, in_dtype=in_dtype, flag_rows=kw.get("flag_rows", 0))
    if flags is None:
        flags = torch.zeros(max(nf, 4), dtype=torch.int32, device="cuda:0")
    print("allgather W=%d M=%d K=%d %s" % (W, M, K, kw), flush=True)
    ctx.allgather([dev(s) for s in shards], G, flags, blocking=True, **kw)
    torch.cuda.synchronize()
    return host(G), host(flags)[:nf]


def _shards(W, R, K, dtype="bf16", seed=40):
    w = I.AGWorkload("t", W=W, M=W * R, K=K, N=0, dtype=dtype, dist="normal" if dtype == "bf16" else "uniform",
                     seed_index=seed)
    return I.make_ag(w)[0]


def _epoch_of(buf, shards, rank):
    """The epoch the call stored: the high half of the first remote packet (None for W = 1)."""
    W = len(shards)
    per = shards[0].size * shards[0].itemsize // 4
    remote = [p for p in range(W) if p != rank]
    return int(buf[remote[0] * per] >> np.uint64(32)) if remote else None


def _check_ll(orc, shards, rank, flag_rows, G, buf, before=None):
    assert np.array_equal(G, orc.allgather(shards)), "gathered rows"
    e = _epoch_of(buf, shards, rank)
    if e is None:
        return None
    fr = flag_rows if flag_rows else shards[0].shape[0]
    assert np.array_equal(buf, orc.ll_buffer(shards, rank, e, fr, before=before)), "LL buffer"
    return e


# (W, rows per shard, K, dtype, flag_rows, rank)
CASES = [
    (8, 16, 8192, "bf16", 2, 0),      # decode-size Llama-3-70B activations, 16 tokens per rank
    (8, 16, 8192, "bf16", 16, 5),     # one chunk per peer
    (4, 6, 40, "f32", 3, 1),          # fp32, chunks far below one pass
    (3, 5, 24, "bf16", 5, 2),         # 240-byte chunks: a ragged pass
    (2, 512, 4096, "bf16", 256, 1),   # 2 MiB chunks: several passes per chunk
    (8, 64, 5120, "bf16", 0, 3),      # library default chunk
    (1, 8, 64, "bf16", 4, 0),         # W = 1: only the local shard
]


@pytest.mark.parametrize("W,R,K,dtype,fr,rank", CASES)
def test_ll_allgather_parity(ctx, orc, W, R, K, dtype, fr, rank):
    shards = _shards(W, R, K, dtype)
    G, buf, _ = run_ll(ctx, shards, rank=rank, flag_rows=fr)
    _check_ll(orc, shards, rank, fr, G, buf)


@pytest.mark.parametrize("W,R,K,dtype,fr,rank", CASES)
def test_flag_allgather_parity(ctx, orc, W, R, K, dtype, fr, rank):
    shards = _shards(W, R, K, dtype)
    G, fl = run_flag(ctx, shards, rank=rank, flag_rows=fr)
    assert np.array_equal(G, orc.allgather(shards))
    assert fl.size and (fl == fl[0]).all() and fl[0] > 0


def test_ll_new_data_each_call(ctx, orc):
    # the same LL buffer over three calls: packets of an older epoch are never taken for new ones
    a = _shards(8, 16, 1024, seed=41)
    b = _shards(8, 16, 1024, seed=42)
    G1, buf1, ll = run_ll(ctx, a, rank=2, flag_rows=4)
    e1 = _check_ll(orc, a, 2, 4, G1, buf1)
    G2, buf2, ll = run_ll(ctx, b, ll_buf=ll, rank=2, flag_rows=4)
    e2 = _check_ll(orc, b, 2, 4, G2, buf2)
    G3, buf3, ll = run_ll(ctx, a, ll_buf=ll, rank=2, flag_rows=4, peer_gbps=20.0)
    e3 = _check_ll(orc, a, 2, 4, G3, buf3)
    assert e2 == e1 + 1 and e3 == e2 + 1


@pytest.mark.parametrize("mode", [dict(peer_gbps=20.0, jitter_us=30.0, arrival_order="per_peer", arrival_seed=3),
                                  dict(peer_gbps=50.0, arrival_order="global", arrival_seed=4),
                                  dict(producer="serial", jitter_us=10.0),
                                  dict(producer_cus=3, consumer_cus=5, peer_gbps=40.0)])
def test_ll_paced_and_shuffled(ctx, orc, mode):
    shards = _shards(8, 32, 2048, seed=43)
    G, buf, _ = run_ll(ctx, shards, rank=6, flag_rows=8, **mode)
    _check_ll(orc, shards, 6, 8, G, buf)
    Gf, fl = run_flag(ctx, shards, rank=6, flag_rows=8, **mode)
    assert np.array_equal(Gf, G)
    assert (fl == fl[0]).all()


def test_ll_trace_stamps(ctx, orc):
    W, R, K, fr = 8, 16, 8192, 2
    shards = _shards(W, R, K)
    n = W * R // fr
    for call in ("ll", "flag"):
        tr = torch.zeros(2 * n, dtype=torch.int64, device="cuda:0")
        if call == "ll":
            G, _, _ = run_ll(ctx, shards, rank=1, flag_rows=fr, trace=tr.data_ptr())
        else:
            G, _ = run_flag(ctx, shards, rank=1, flag_rows=fr, trace=tr.data_ptr())
        assert np.array_equal(G, orc.allgather(shards))
        t = tr.cpu().numpy().reshape(n, 2)
        assert (t > 0).all(), call
        assert (t[:, 1] >= t[:, 0]).all(), call


@pytest.mark.parametrize("call", ["ll", "flag"])
def test_withheld_peer_times_out(ctx, orc, call):
    shards = _shards(4, 32, 512, seed=44)
    with pytest.raises(sgt.SgtError) as ei:
        if call == "ll":
            run_ll(ctx, shards, rank=0, flag_rows=8, withhold_peer=2, timeout_ms=20.0)
        else:
            run_flag(ctx, shards, rank=0, flag_rows=8, withhold_peer=2, timeout_ms=20.0)
    assert ei.value.status == sgt.SGT_ETIMEDOUT
    # the next call on the same context succeeds
    G, buf, _ = run_ll(ctx, shards, rank=0, flag_rows=8)
    _check_ll(orc, shards, 0, 8, G, buf)


def test_bad_arguments(ctx):
    shards = [dev(s) for s in _shards(2, 4, 24)]
    G = torch.empty((8, 24), dtype=torch.bfloat16, device="cuda:0")
    ll = torch.zeros(8 * 24 * 2 * 2 // 8, dtype=torch.int64, device="cuda:0")
    fl = torch.zeros(8, dtype=torch.int32, device="cuda:0")
    s5 = [dev(s) for s in _shards(2, 4, 5, dtype="f32")]
    G5 = torch.empty((8, 5), dtype=torch.float32, device="cuda:0")
    cases = [
        (lambda: ctx.ll_allgather(s5, ll, G5, flag_rows=1), sgt.SGT_EINVAL),     # 20-byte chunks
        (lambda: ctx.allgather(s5, G5, fl, flag_rows=2), sgt.SGT_EINVAL),        # 40-byte chunks
        (lambda: ctx.ll_allgather(shards, ll, G, producer="preset"), sgt.SGT_EINVAL),
        (lambda: ctx.allgather(shards, G, fl, producer="preset"), sgt.SGT_EINVAL),
        (lambda: ctx.ll_allgather(shards, ll, G, flag_rows=3), sgt.SGT_EINVAL),    # rows per shard not a multiple
        (lambda: ctx.ll_allgather(shards, ll, G, rank=2), sgt.SGT_EINVAL),
        (lambda: ctx.ll_allgather(shards, ll[1:], G), sgt.SGT_EINVAL),            # ll_buf misaligned
    ]
    for f, st in cases:
        with pytest.raises(sgt.SgtError) as ei:
            f()
        assert ei.value.status == st
    # M = 0 is a no-op
    e = [torch.empty((0, 24), dtype=torch.bfloat16, device="cuda:0")] * 2
    ctx.ll_allgather(e, ll, torch.empty((0, 24), dtype=torch.bfloat16, device="cuda:0"), blocking=True)
    ctx.allgather(e, torch.empty((0, 24), dtype=torch.bfloat16, device="cuda:0"), fl, blocking=True)
