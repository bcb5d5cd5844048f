"""GPU parity of one rank's signal-gated ring AllReduce against the CPU oracle (through the C ABI).

The left neighbour's messages come from the oracle's emulation of the whole
ring; the rank's result and every message it sends must equal, bit for bit,
what the oracle's ring gives that rank (one fp32 addition per element and
step, the same in both), and its result must be the sum over ranks.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import dev, poison_like  # noqa: E402


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = sgt.Context(0)
    yield c
    c.close()


def run_ring(ctx, x, msgs, W, *, resident=False, flags=None, **kw):
    """Upload and run one rank's ring AllReduce (blocking); return (out, outbox, flags) on the host."""
    N = x.size
    C = N // W
    nf, _ = sgt.ring_flag_count(W, N)
    dx = dev(x)
    out = poison_like(torch.empty(N, dtype=torch.float32, device="cuda:0"))
    nm = max(2 * (W - 1), 1)
    outbox = poison_like(torch.empty(nm * max(C, 1), dtype=torch.float32, device="cuda:0"))
    if resident:
        inbox = dev(np.ascontiguousarray(msgs).reshape(-1)) if W > 1 else None
        left = None
        kw["producer"] = "preset"
    else:
        left = dev(np.ascontiguousarray(msgs).reshape(-1)) if W > 1 else None
        inbox = poison_like(torch.empty(nm * max(C, 1), dtype=torch.float32, device="cuda:0"))
    if flags is None:
        flags = torch.zeros(max(nf, 4), dtype=torch.int32, device="cuda:0")
    print("ring W=%d N=%d rank=%s resident=%s %s" % (W, N, kw.get("rank"), resident, kw), flush=True)
    ctx.ring_allreduce(dx, left, inbox, outbox, out, flags, W, blocking=True, **kw)
    torch.cuda.synchronize()
    ob = outbox.cpu().numpy()[:2 * (W - 1) * C].reshape(2 * (W - 1), C)
    return out.cpu().numpy(), ob, flags.cpu().numpy()[:nf]


def _xs(W, N, dist="normal", seed=7, salt=0):
    return I.make_ring(I.RingWorkload("t", W=W, N=N, dist=dist, seed_index=seed), salt=salt)


def _check(orc, xs, rank, out, outbox, fl):
    outs, inbox, outboxes = orc.ring_allreduce(xs)
    assert np.array_equal(out, outs[rank]), "result"
    assert np.array_equal(outbox, outboxes[rank]), "messages sent"
    ref = orc.allreduce(xs)
    mag = np.sum(np.abs(np.stack(xs).astype(np.float64)), axis=0)
    assert np.all(np.abs(out - ref) <= len(xs) * 2.0**-24 * mag + 1e-30), "sum over ranks"
    if fl.size:
        assert (fl == fl[0]).all() and fl[0] > 0, "flags"


# (W, N, rank): multi-tile chunks with a ragged last pass, one small tile, many 4-element tiles
CASES = [(8, 8 * 20480, 0), (8, 8 * 20480, 5), (4, 4 * 12, 1), (3, 3 * 16396, 2), (2, 2 * 65536, 1)]


@pytest.mark.parametrize("W,N,rank", CASES)
@pytest.mark.parametrize("mode", ["resident", "cu", "serial"])
def test_ring_parity(ctx, orc, W, N, rank, mode):
    xs = _xs(W, N)
    _, inbox, _ = orc.ring_allreduce(xs)
    kw = dict(rank=rank)
    if mode == "serial":
        kw["producer"] = "serial"
    if mode == "cu":
        kw["peer_gbps"] = 40.0
    out, ob, fl = run_ring(ctx, xs[rank], inbox[rank], W, resident=mode == "resident", **kw)
    _check(orc, xs, rank, out, ob, fl)


def test_ring_integer_inputs_sum_exactly(ctx, orc):
    W, N = 8, 8 * 4096
    xs = _xs(W, N, dist="int")
    _, inbox, _ = orc.ring_allreduce(xs)
    out, _, _ = run_ring(ctx, xs[3], inbox[3], W, rank=3, peer_gbps=80.0, jitter_us=5.0)
    assert np.array_equal(out.astype(np.int64), np.sum(np.stack(xs).astype(np.int64), axis=0))


def test_ring_paced_shuffled_grids_bit_identical(ctx, orc):
    W, N = 8, 8 * 20480
    xs = _xs(W, N, seed=8)
    _, inbox, _ = orc.ring_allreduce(xs)
    ref = None
    for kw in (dict(), dict(peer_gbps=30.0, jitter_us=20.0, arrival_seed=5), dict(consumer_cus=3),
               dict(producer_cus=2, consumer_cus=40, peer_gbps=100.0)):
        out, ob, fl = run_ring(ctx, xs[6], inbox[6], W, rank=6, **kw)
        if ref is None:
            ref = (out, ob)
            _check(orc, xs, 6, out, ob, fl)
        assert np.array_equal(out, ref[0]) and np.array_equal(ob, ref[1]), kw


def test_ring_repeated_calls_new_data(ctx, orc):
    W, N = 4, 4 * 8192
    flags = torch.zeros(sgt.ring_flag_count(W, N)[0], dtype=torch.int32, device="cuda:0")
    for salt in (0, 1, 2):
        xs = _xs(W, N, seed=9, salt=salt)
        _, inbox, _ = orc.ring_allreduce(xs)
        out, ob, fl = run_ring(ctx, xs[2], inbox[2], W, rank=2, flags=flags, peer_gbps=60.0)
        _check(orc, xs, 2, out, ob, fl)


def test_ring_of_one(ctx):
    x = _xs(1, 1000 * 4)[0]
    out, _, _ = run_ring(ctx, x, np.zeros((0,), np.float32), 1, rank=0, resident=True)
    assert np.array_equal(out, x)


def test_ring_trace(ctx, orc):
    W, N = 8, 8 * 20480
    xs = _xs(W, N, seed=10)
    _, inbox, _ = orc.ring_allreduce(xs)
    _, tile = sgt.ring_flag_count(W, N)
    n_items = (N // W // tile) * (2 * W - 1)
    tr = torch.zeros(3 * n_items, dtype=torch.int64, device="cuda:0")
    out, ob, fl = run_ring(ctx, xs[1], inbox[1], W, rank=1, peer_gbps=50.0, trace=tr.data_ptr())
    _check(orc, xs, 1, out, ob, fl)
    t = tr.cpu().numpy().reshape(n_items, 3)
    assert (t > 0).all() and (t[:, 1] >= t[:, 0]).all() and (t[:, 2] >= t[:, 1]).all()


def test_ring_withheld_neighbour_times_out(ctx, orc):
    W, N = 4, 4 * 4096
    xs = _xs(W, N, seed=11)
    _, inbox, _ = orc.ring_allreduce(xs)
    with pytest.raises(sgt.SgtError) as ei:
        run_ring(ctx, xs[1], inbox[1], W, rank=1, withhold_peer=0, timeout_ms=20.0)
    assert ei.value.status == sgt.SGT_ETIMEDOUT
    out, ob, fl = run_ring(ctx, xs[1], inbox[1], W, rank=1)
    _check(orc, xs, 1, out, ob, fl)


def test_ring_bad_arguments(ctx):
    x = torch.zeros(4 * 8, dtype=torch.float32, device="cuda:0")
    buf = torch.zeros(6 * 8, dtype=torch.float32, device="cuda:0")
    fl = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    cases = [
        (lambda: ctx.ring_allreduce(x[:30], buf, buf, buf, x, fl, 4), sgt.SGT_EINVAL),        # N % W
        (lambda: ctx.ring_allreduce(x[:24], buf, buf, buf, x, fl, 4), sgt.SGT_EINVAL),        # C = 6
        (lambda: ctx.ring_allreduce(x, None, buf, buf, x, fl, 4), sgt.SGT_EINVAL),            # no messages
        (lambda: ctx.ring_allreduce(x, buf, buf, buf, x, fl, 4, in_dtype=sgt.SGT_BF16), sgt.SGT_EUNSUPPORTED),
        (lambda: ctx.ring_allreduce(x, buf, buf, buf, x, fl, 4, rank=4), sgt.SGT_EINVAL),
    ]
    for f, st in cases:
        with pytest.raises(sgt.SgtError) as ei:
            f()
        assert ei.value.status == st
    # N = 0 is a no-op
    e = torch.empty(0, dtype=torch.float32, device="cuda:0")
    ctx.ring_allreduce(e, None, None, None, e, None, 4, blocking=True)


@pytest.mark.slow
def test_ring_full_shape(ctx, orc):
    w = I.RING
    xs = I.make_ring(w)
    _, inbox, _ = orc.ring_allreduce(xs)
    out, ob, fl = run_ring(ctx, xs[0], inbox[0], w.W, rank=0, peer_gbps=w.peer_gbps)
    _check(orc, xs, 0, out, ob, fl)
