"""GPU parity of the expert-parallel AllToAll (dispatch and combine, one rank's share) against the CPU oracle,
through the C ABI.

Dispatch: the received rows, their token ids and counts are bit-exact, slots past a block's count and flags
past its last chunk are left untouched.  Combine: the receive slots and slot table are bit-exact, the fp32
output is within the fp32 tolerance of the fp64 oracle, and a round trip through identity experts returns
every token's own row exactly.
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import TOL_F32, assert_close, dev, host, poison_like  # noqa: E402


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = sgt.Context(0)
    yield c
    c.close()


def _case(orc, W, T_r, H, E, k, seed=8, salt=0, invalid=False):
    """Seeded tokens, routing (the oracle's top-k of the workload's logits), gates and expert outputs."""
    w = I.A2AWorkload("t", W=W, T=W * T_r, H=H, E=E, topk=k, seed_index=seed)
    X, logits, gate, back = I.make_a2a(w, salt=salt)
    ids, _, _ = orc.moe_route(logits, k)
    topk = [np.ascontiguousarray(ids[p * T_r:(p + 1) * T_r]) for p in range(W)]
    if invalid:
        rng = np.random.default_rng(seed + 100)
        for tk in topk:
            n = max(1, T_r // 8)
            tk[rng.integers(0, T_r, n), rng.integers(0, k, n)] = rng.choice([-1, E, E + 1000], n)
    gates = [np.ascontiguousarray(gate[p * T_r:(p + 1) * T_r]) for p in range(W)]
    return X, topk, gates, back


def run_dispatch(ctx, X, topk, E, **kw):
    W = len(X)
    T_r, H = X[0].shape
    E_l = E // W
    dt = torch.bfloat16 if X[0].dtype == np.uint16 else torch.float32
    recv = poison_like(torch.empty((E_l, W, T_r, H), dtype=dt, device="cuda:0"))
    tok = torch.full((E_l, W, T_r), -7, dtype=torch.int32, device="cuda:0")
    cnt = torch.zeros((E_l, W), dtype=torch.int64, device="cuda:0")
    nf = sgt.a2a_flag_count(W, T_r, E, flag_rows=kw.get("flag_rows", 0))
    flags = torch.zeros(max(nf, 1), dtype=torch.int32, device="cuda:0")
    print("a2a dispatch W=%d T_r=%d H=%d E=%d k=%d %s" % (W, T_r, H, E, topk[0].shape[1], kw), flush=True)
    ctx.a2a_dispatch([dev(x) for x in X], [dev(t) for t in topk], recv, tok, cnt, flags, E, blocking=True, **kw)
    torch.cuda.synchronize()
    return host(recv), tok.cpu().numpy(), cnt.cpu().numpy().view(np.uint64), flags.cpu().numpy()[:nf].view(np.uint32)


def check_dispatch(orc, X, topk, E, rank, chunk, recv, tok, cnt, flags):
    W = len(X)
    T_r = X[0].shape[0]
    E_l = E // W
    ref, ref_tok, ref_cnt = orc.a2a_dispatch(X, topk, E, rank)
    epoch = int(cnt[0, 0] >> np.uint64(32))
    assert epoch > 0
    assert np.array_equal((cnt >> np.uint64(32)).astype(np.int64), np.full((E_l, W), epoch)), "count packet epochs"
    assert np.array_equal((cnt & np.uint64(0xFFFFFFFF)).astype(np.int64), ref_cnt), "counts"
    nch = -(-T_r // chunk)
    poison = np.uint16(0x7FC0) if recv.dtype == np.uint16 else np.float32(np.nan)
    for l in range(E_l):
        for p in range(W):
            n = int(ref_cnt[l, p])
            assert np.array_equal(recv[l, p, :n], ref[l, p, :n]), "rows of block (%d, %d)" % (l, p)
            assert np.array_equal(tok[l, p, :n], ref_tok[l, p, :n]), "tokens of block (%d, %d)" % (l, p)
            assert (tok[l, p, n:] == -7).all(), "token entries past the count written"
            rest = recv[l, p, n:]
            if recv.dtype == np.uint16:
                assert (rest == poison).all(), "slots past the count written"
            else:
                assert np.isnan(rest).all(), "slots past the count written"
            b = l * W + p
            used = -(-n // chunk)
            f = flags[b * nch:(b + 1) * nch]
            assert (f[:used] == epoch).all() and (f[used:] == 0).all(), "chunk flags of block (%d, %d)" % (l, p)


DISPATCH_CASES = [
    # W, T_r, H, E, k, chunk, rank, peer_gbps, invalid
    (8, 64, 256, 64, 8, 16, 0, 0.0, False),
    (8, 50, 128, 64, 8, 16, 5, 20.0, False),       # ragged last chunk, paced links
    (4, 37, 72, 8, 3, 5, 2, 0.0, True),            # 144-byte rows, invalid ids
    (1, 20, 64, 4, 2, 32, 0, 0.0, False),          # one rank
    (2, 300, 8, 6, 6, 1, 1, 0.0, False),           # k = E / W * W (every expert), one-row chunks
    (1, 40, 64, 80, 3, 8, 0, 0.0, False),          # 80 local experts: the scan kernel runs before the senders
    (2, 24, 64, 130, 4, 8, 1, 10.0, False),        # 65 local experts, paced
]


@pytest.mark.parametrize("W,T_r,H,E,k,chunk,rank,gbps,invalid", DISPATCH_CASES)
def test_dispatch_matches_oracle(ctx, orc, W, T_r, H, E, k, chunk, rank, gbps, invalid):
    X, topk, _, _ = _case(orc, W, T_r, H, E, k, invalid=invalid)
    recv, tok, cnt, flags = run_dispatch(ctx, X, topk, E, rank=rank, flag_rows=chunk, peer_gbps=gbps)
    check_dispatch(orc, X, topk, E, rank, chunk, recv, tok, cnt, flags)


def test_dispatch_fp32_rows(ctx, orc):
    W, T_r, H, E, k = 4, 33, 36, 8, 2
    _, topk, _, _ = _case(orc, W, T_r, H, E, k)
    rng = np.random.default_rng(3)
    X = [rng.standard_normal((T_r, H)).astype(np.float32) for _ in range(W)]
    recv, tok, cnt, flags = run_dispatch(ctx, X, topk, E, rank=3, flag_rows=8, in_dtype=sgt.SGT_F32)
    check_dispatch(orc, X, topk, E, 3, 8, recv, tok, cnt, flags)


def test_dispatch_full_shape(ctx, orc):
    """The MoE layer's dispatch: 8 ranks of 512 tokens, hidden 2048 bf16, top-8 of 64 experts (Zipf-skewed),
    links at 50 GB/s per peer, 32-row chunks."""
    w = I.A2A
    X, topk, _, _ = _case(orc, w.W, w.tokens_per_rank, w.H, w.E, w.topk, seed=w.seed_index)
    recv, tok, cnt, flags = run_dispatch(ctx, X, topk, w.E, rank=0, flag_rows=w.chunk_rows, peer_gbps=w.peer_gbps)
    check_dispatch(orc, X, topk, w.E, 0, w.chunk_rows, recv, tok, cnt, flags)


def run_combine(ctx, back, topk, gate, E, *, cbuf_init=None, **kw):
    W = len(back)
    T_r, k = topk.shape
    H = back[0].shape[2]
    if cbuf_init is not None:
        cbuf = dev(cbuf_init)
    else:
        cbuf = poison_like(torch.empty((E, T_r, H), dtype=torch.bfloat16, device="cuda:0"))
    slot = torch.full((T_r, k), -9, dtype=torch.int32, device="cuda:0")
    out = poison_like(torch.empty((T_r, H), dtype=torch.float32, device="cuda:0"))
    nf = sgt.a2a_flag_count(W, T_r, E, flag_rows=kw.get("flag_rows", 0))
    flags = torch.zeros(max(nf, 1), dtype=torch.int32, device="cuda:0")
    print("a2a combine W=%d T_r=%d H=%d E=%d k=%d %s" % (W, T_r, H, E, k, kw), flush=True)
    bk = None if kw.get("producer") == "preset" else [dev(b) for b in back]
    ctx.a2a_combine(bk, dev(topk), dev(gate), cbuf, slot, out, flags, W, blocking=True, **kw)
    torch.cuda.synchronize()
    return host(cbuf), slot.cpu().numpy(), out.cpu().numpy()


def check_combine(orc, back, topk, gate, E, cbuf, slot, out):
    T_r = topk.shape[0]
    assert np.array_equal(slot, orc.a2a_slots(topk, E)), "slot table"
    ref_cbuf = orc.a2a_combine_recv(back, topk, E)
    for e in range(E):
        n = len(orc.a2a_tokens(topk, e))
        assert np.array_equal(cbuf[e, :n], ref_cbuf[e, :n]), "receive slots of expert %d" % e
        assert (cbuf[e, n:] == np.uint16(0x7FC0)).all(), "receive slots past the count of expert %d" % e
    ref = orc.a2a_combine(back, topk, gate, E)
    assert out.shape == (T_r, back[0].shape[2])
    assert_close(out, ref, what="a2a combine", **TOL_F32)


COMBINE_CASES = [
    # W, T_r, H, E, k, chunk, rank, producer, peer_gbps, invalid
    (8, 64, 256, 64, 8, 16, 0, "cu", 0.0, False),
    (8, 50, 128, 64, 8, 16, 6, "cu", 20.0, False),
    (8, 50, 128, 64, 8, 16, 6, "serial", 20.0, False),
    (4, 37, 72, 8, 3, 5, 2, "cu", 0.0, True),
    (1, 20, 1032, 4, 2, 32, 0, "cu", 0.0, False),   # one rank; rows of more than one receiver pass
    (2, 300, 8, 6, 6, 1, 1, "cu", 0.0, False),
]


@pytest.mark.parametrize("W,T_r,H,E,k,chunk,rank,producer,gbps,invalid", COMBINE_CASES)
def test_combine_matches_oracle(ctx, orc, W, T_r, H, E, k, chunk, rank, producer, gbps, invalid):
    _, topk, gates, back = _case(orc, W, T_r, H, E, k, invalid=invalid)
    cbuf, slot, out = run_combine(ctx, back, topk[rank], gates[rank], E, rank=rank, flag_rows=chunk,
                                  producer=producer, peer_gbps=gbps)
    check_combine(orc, back, topk[rank], gates[rank], E, cbuf, slot, out)


def test_combine_preset_matches_oracle(ctx, orc):
    W, T_r, H, E, k = 8, 64, 256, 64, 8
    _, topk, gates, back = _case(orc, W, T_r, H, E, k)
    before = np.full((E, T_r, H), 0x7FC0, np.uint16)
    cb = orc.a2a_combine_recv(back, topk[1], E, before=before)
    cbuf, slot, out = run_combine(ctx, back, topk[1], gates[1], E, cbuf_init=cb, rank=1, flag_rows=16,
                                  producer="preset")
    check_combine(orc, back, topk[1], gates[1], E, cbuf, slot, out)


def test_combine_full_shape(ctx, orc):
    """The MoE layer's combine on rank 0: 512 tokens, top-8 of 64 experts, hidden 2048, links at 50 GB/s."""
    w = I.A2A
    _, topk, gates, back = _case(orc, w.W, w.tokens_per_rank, w.H, w.E, w.topk, seed=w.seed_index)
    cbuf, slot, out = run_combine(ctx, back, topk[0], gates[0], w.E, rank=0, flag_rows=w.chunk_rows,
                                  peer_gbps=w.peer_gbps)
    check_combine(orc, back, topk[0], gates[0], w.E, cbuf, slot, out)


def test_round_trip_through_identity_experts(ctx, orc):
    """Every rank's dispatch on the GPU; each expert returns the rows it received; with gates that are powers
    of two summing to one the combine gives back each token's own row exactly."""
    W, T_r, H, E, k = 4, 40, 64, 16, 4
    X, topk, _, _ = _case(orc, W, T_r, H, E, k)
    recvs = [run_dispatch(ctx, X, topk, E, rank=q, flag_rows=8)[0] for q in range(W)]
    gate = np.tile(np.array([0.5, 0.25, 0.125, 0.125], np.float32), (T_r, 1))
    for r in (0, 3):
        back = [np.ascontiguousarray(recvs[q][:, r]) for q in range(W)]
        _, _, out = run_combine(ctx, back, topk[r], gate, E, rank=r, flag_rows=8)
        assert np.array_equal(out, I.bf16_bits_to_f32(X[r])), "round trip of rank %d" % r


def test_repeated_calls_reuse_flags(ctx, orc):
    """Two dispatches and two combines on the same flag words: each call's epoch sets them anew."""
    W, T_r, H, E, k = 8, 48, 64, 32, 4
    nf = sgt.a2a_flag_count(W, T_r, E, flag_rows=16)
    flags = torch.zeros(nf, dtype=torch.int32, device="cuda:0")
    for salt in (0, 1):
        X, topk, gates, back = _case(orc, W, T_r, H, E, k, salt=salt)
        recv = poison_like(torch.empty((E // W, W, T_r, H), dtype=torch.bfloat16, device="cuda:0"))
        tok = torch.full((E // W, W, T_r), -7, dtype=torch.int32, device="cuda:0")
        cnt = torch.zeros((E // W, W), dtype=torch.int64, device="cuda:0")
        ctx.a2a_dispatch([dev(x) for x in X], [dev(t) for t in topk], recv, tok, cnt, flags, E, rank=2,
                         flag_rows=16, blocking=True)
        ref, _, ref_cnt = orc.a2a_dispatch(X, topk, E, 2)
        rc = host(recv)
        for l in range(E // W):
            for p in range(W):
                n = int(ref_cnt[l, p])
                assert np.array_equal(rc[l, p, :n], ref[l, p, :n])
        cbuf = poison_like(torch.empty((E, T_r, H), dtype=torch.bfloat16, device="cuda:0"))
        slot = torch.empty((T_r, k), dtype=torch.int32, device="cuda:0")
        out = torch.empty((T_r, H), dtype=torch.float32, device="cuda:0")
        ctx.a2a_combine([dev(b) for b in back], dev(topk[2]), dev(gates[2]), cbuf, slot, out, flags, W, rank=2,
                        flag_rows=16, blocking=True)
        assert_close(out.cpu().numpy(), orc.a2a_combine(back, topk[2], gates[2], E), what="combine", **TOL_F32)


def test_withheld_link_times_out(ctx, orc):
    """A link whose chunks are copied but never flagged: the combine's bounded waits expire and the call
    reports SGT_ETIMEDOUT; the context then works normally."""
    W, T_r, H, E, k = 4, 32, 64, 8, 2
    _, topk, gates, back = _case(orc, W, T_r, H, E, k)
    with pytest.raises(sgt.SgtError) as ei:
        run_combine(ctx, back, topk[0], gates[0], E, rank=0, flag_rows=8, withhold_peer=2, timeout_ms=50)
    assert ei.value.status == sgt.SGT_ETIMEDOUT
    cbuf, slot, out = run_combine(ctx, back, topk[0], gates[0], E, rank=0, flag_rows=8)
    check_combine(orc, back, topk[0], gates[0], E, cbuf, slot, out)


def test_invalid_arguments_are_rejected(ctx):
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda:0")
    t = torch.zeros((8, 2), dtype=torch.int32, device="cuda:0")
    recv = torch.zeros((2, 2, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    tok = torch.zeros((2, 2, 8), dtype=torch.int32, device="cuda:0")
    cnt = torch.zeros((2, 2), dtype=torch.int64, device="cuda:0")
    fl = torch.zeros(64, dtype=torch.int32, device="cuda:0")

    def epoch_of_valid_call():
        ctx.a2a_dispatch([x, x], [t, t], recv, tok, cnt, fl, 4, blocking=True)
        return int(cnt.cpu().numpy().view(np.uint64)[0, 0] >> np.uint64(32))

    e0 = epoch_of_valid_call()
    for E, kw in ((5, {}), (4, {"producer": "preset"}), (4, {"flag_rows": 2048}), (4, {"peer_gbps": 1e-9})):
        with pytest.raises(sgt.SgtError) as ei:
            ctx.a2a_dispatch([x, x], [t, t], recv, tok, cnt, fl, E, **kw)
        assert ei.value.status in (sgt.SGT_EINVAL, sgt.SGT_EUNSUPPORTED)
    assert epoch_of_valid_call() == e0 + 1, "a rejected call advanced the context's epoch"
    odd = torch.zeros((8, 60), dtype=torch.bfloat16, device="cuda:0")   # 120-byte rows
    with pytest.raises(sgt.SgtError):
        ctx.a2a_dispatch([odd, odd], [t, t], recv, tok, cnt, fl, 4)
    cbuf = torch.zeros((4, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    g = torch.zeros((8, 2), dtype=torch.float32, device="cuda:0")
    out = torch.zeros((8, 64), dtype=torch.float32, device="cuda:0")
    with pytest.raises(sgt.SgtError):
        ctx.a2a_combine([cbuf[:2], cbuf[:2]], t, g, cbuf, t.clone(), out, fl, 2, out_dtype=sgt.SGT_BF16)


def test_dispatch_and_combine_of_zero_tokens(ctx):
    """T_r = 0: the dispatch still stores every count packet (count 0, this call's epoch); the combine is a no-op."""
    W, E, H, k = 4, 8, 64, 2
    X = [torch.empty((0, H), dtype=torch.bfloat16, device="cuda:0") for _ in range(W)]
    tk = [torch.empty((0, k), dtype=torch.int32, device="cuda:0") for _ in range(W)]
    recv = torch.empty((E // W, W, 0, H), dtype=torch.bfloat16, device="cuda:0")
    tok = torch.empty((E // W, W, 0), dtype=torch.int32, device="cuda:0")
    cnt = torch.full((E // W, W), -1, dtype=torch.int64, device="cuda:0")
    fl = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    assert sgt.a2a_flag_count(W, 0, E) == 0
    ctx.a2a_dispatch(X, tk, recv, tok, cnt, fl, E, rank=1, blocking=True)
    c = cnt.cpu().numpy().view(np.uint64)
    assert ((c & np.uint64(0xFFFFFFFF)) == 0).all() and ((c >> np.uint64(32)) > 0).all()
    assert len(set((c >> np.uint64(32)).ravel().tolist())) == 1
    out = torch.empty((0, H), dtype=torch.float32, device="cuda:0")
    ctx.a2a_combine([torch.empty((E // W, 0, H), dtype=torch.bfloat16, device="cuda:0")] * W, tk[0],
                    torch.empty((0, k), dtype=torch.float32, device="cuda:0"),
                    torch.empty((E, 0, H), dtype=torch.bfloat16, device="cuda:0"), tk[0].clone(), out, fl, W,
                    blocking=True)


@pytest.mark.parametrize("W,T_r,H,E,k,chunk,rank", [(4, 33, 64, 8, 1, 8, 3),     # one pick per token
                                                     (8, 40, 128, 8, 3, 16, 2)])  # one expert per rank
def test_a2a_degenerate_routings(ctx, orc, W, T_r, H, E, k, chunk, rank):
    X, topk, gates, back = _case(orc, W, T_r, H, E, k, seed=40)
    recv, tok, cnt, flags = run_dispatch(ctx, X, topk, E, rank=rank, flag_rows=chunk, peer_gbps=20.0)
    check_dispatch(orc, X, topk, E, rank, chunk, recv, tok, cnt, flags)
    cbuf, slot, out = run_combine(ctx, back, topk[rank], gates[rank], E, rank=rank, flag_rows=chunk, peer_gbps=20.0)
    check_combine(orc, back, topk[rank], gates[rank], E, cbuf, slot, out)


def test_a2a_every_token_to_one_expert(ctx, orc):
    """All tokens of every rank pick expert 5 first (and distinct others): block (5 - r*E_l, p) holds all T_r rows,
    the slot capacity, over a ragged last chunk."""
    W, T_r, H, E, k, chunk = 4, 45, 64, 16, 3, 8
    X, topk, gates, back = _case(orc, W, T_r, H, E, k, seed=41)
    for tk in topk:
        for t in range(T_r):
            others = [e for e in tk[t] if e != 5][:k - 1]
            tk[t] = [5] + others
    rank = 5 // (E // W)
    recv, tok, cnt, flags = run_dispatch(ctx, X, topk, E, rank=rank, flag_rows=chunk)
    check_dispatch(orc, X, topk, E, rank, chunk, recv, tok, cnt, flags)
    assert ((cnt[5 % (E // W)] & np.uint64(0xFFFFFFFF)) == T_r).all()
    cbuf, slot, out = run_combine(ctx, back, topk[0], gates[0], E, rank=0, flag_rows=chunk)
    check_combine(orc, back, topk[0], gates[0], E, cbuf, slot, out)
