"""Pins for the CPU oracle against facts fixed by mathematics and by the pages.

Nothing here re-types the oracle's formula: each check compares it with an
independent exact computation (Python rationals, integer matrix products), a
closed form (identity / permutation matrices), a library routine for a special
case (numpy concatenate, stable argsort), a hand-derived fixture (panel orders
from the pages' swizzle formula), or an invariant (arrival-order invariance of
the protocol emulation, with a planted mistake showing the check has teeth).
"""
from fractions import Fraction
import os

import numpy as np
import pytest

from signal_gated_tiled_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _vals(a):
    return I.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def _exact_gemm(A, B, b_layout):
    """Exact rational product (independent of the oracle): returns (value, sum|a||b|) as Fractions."""
    Av = _vals(A).astype(np.float64)
    Bv = _vals(B).astype(np.float64)
    if b_layout == "nk":
        Bv = Bv.T
    M, K = Av.shape
    N = Bv.shape[1]
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            m = Fraction(0)
            for k in range(K):
                p = Fraction(float(Av[i, k])) * Fraction(float(Bv[k, j]))
                s += p
                m += abs(p)
            out[i][j] = s
            mag[i][j] = m
    return out, mag


def _rand(shape, dtype, seed):
    ss = np.random.SeedSequence(seed)
    return I.uniform_f32(ss, shape) if dtype == "f32" else I.normal_bf16(ss, shape, 0.5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("b_layout", ["kn", "nk"])
@pytest.mark.parametrize("M,K,N", [(3, 5, 4), (7, 13, 6), (5, 33, 9)])
def test_gemm_against_exact_rationals(orc, dtype, b_layout, M, K, N):
    A = _rand((M, K), dtype, 11 + M)
    B = _rand((K, N), dtype, 97 + N)
    Bs = np.ascontiguousarray(B.T) if b_layout == "nk" else B
    C = orc.gemm(A, Bs, b_layout)
    exact, mag = _exact_gemm(A, Bs, b_layout)
    u = 2.0 ** -53
    for i in range(M):
        for j in range(N):
            err = abs(Fraction(float(C[i, j])) - exact[i][j])
            assert err <= Fraction(K) * Fraction(u) * mag[i][j] + Fraction(1, 2 ** 1074), (i, j)
    # a transposed operand or a shifted index gives a large error somewhere
    Cf = np.array([[float(x) for x in row] for row in exact])
    assert np.allclose(C, Cf, rtol=1e-12, atol=1e-12)


def test_allgather_is_row_concatenation(orc):
    shards = [_rand((6, 10), "bf16", s) for s in range(5)]
    A = orc.allgather(shards)
    assert A.shape == (30, 10)
    assert np.array_equal(A, np.concatenate(shards, axis=0))
    for p in range(5):
        assert np.array_equal(A[6 * p:6 * (p + 1)], shards[p])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_B_returns_gathered_rows(orc, dtype):
    shards = [_rand((8, 24), dtype, 40 + s) for s in range(3)]
    eye = np.eye(24, dtype=np.float32)
    B = eye if dtype == "f32" else I.f32_to_bf16_bits(eye)
    A_full, C = orc.ag_gemm(shards, B)
    assert np.array_equal(C, _vals(A_full).astype(np.float64))


def test_permutation_B_permutes_columns(orc):
    shards = [_rand((4, 16), "f32", 60 + s) for s in range(4)]
    perm = np.random.default_rng(3).permutation(16)
    Pm = np.zeros((16, 16), np.float32)
    Pm[perm, np.arange(16)] = 1.0          # column j of A*Pm is column perm[j] of A
    A_full, C = orc.ag_gemm(shards, Pm)
    assert np.array_equal(C, A_full[:, perm].astype(np.float64))
    A_full, C = orc.ag_gemm(shards, np.ascontiguousarray(Pm.T), b_layout="nk")
    assert np.array_equal(C, A_full[:, perm].astype(np.float64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_integer_inputs_match_integer_product(orc, dtype):
    ss = np.random.SeedSequence(5)
    a, b = ss.spawn(2)
    A = I.small_int(a, (37, 70), dtype=dtype)
    B = I.small_int(b, (70, 23), dtype=dtype)
    C = orc.gemm(A, B)
    ref = _vals(A).astype(np.int64) @ _vals(B).astype(np.int64)
    assert np.array_equal(C, ref.astype(np.float64))


def test_row_subset_matches_full(orc):
    A = _rand((40, 31), "bf16", 1)
    B = _rand((31, 12), "bf16", 2)
    full = orc.gemm(A, B)
    rows = [39, 0, 17, 17, 5]
    assert np.array_equal(orc.gemm(A, B, rows=rows), full[rows])
    assert np.array_equal(orc.gemm(A, B, threads=1), full)


def _read_swizzle_fixture():
    out = []
    with open(os.path.join(GOLDEN, "swizzle_orders.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, tail = line.split(":")
            order, W, tpp, rank = head.split()
            out.append((order, int(W), int(tpp), int(rank), [int(x) for x in tail.split()]))
    return out


@pytest.mark.parametrize("case", _read_swizzle_fixture())
def test_panel_order_matches_fixture(orc, case):
    order, W, tpp, rank, expect = case
    got = orc.panel_order(W, rank, rows_per_shard=tpp * 4, panel_rows=4, order=order)
    assert list(got) == expect
    assert sorted(got) == list(range(W * tpp))   # a permutation of the panels


@pytest.mark.parametrize("order", ["shard", "mesh"])
@pytest.mark.parametrize("rank", [0, 2, 3])
def test_protocol_is_invariant_to_arrival_order_and_delay(orc, order, rank):
    shards, B = I.make_ag(I.TINY)
    A_ref, C_ref = orc.ag_gemm(shards, B)
    for seed, delay, gp in [(0, 0.0, False), (1, 30.0, False), (7, 50.0, True), (123, 200.0, True), (9, 5.0, False)]:
        A_g, C = orc.ag_gemm_protocol(shards, B, rank=rank, flag_rows=16, panel_rows=16, seed=seed,
                                      max_delay_us=delay, global_perm=gp, order=order, n_consumers=3)
        assert np.array_equal(A_g, A_ref)
        assert np.array_equal(C, C_ref), (seed, delay, gp)


def test_protocol_panels_spanning_several_flags(orc):
    w = I.scaled(I.TINY, dtype="bf16", dist="normal", std=0.5)
    shards, B = I.make_ag(w)
    _, C_ref = orc.ag_gemm(shards, B)
    _, C = orc.ag_gemm_protocol(shards, B, rank=1, flag_rows=8, panel_rows=32, seed=4, max_delay_us=40.0)
    assert np.array_equal(C, C_ref)


def test_planted_mistake_is_caught(orc):
    """A consumer that skips the wait reads poison: the invariance check must fail."""
    shards, B = I.make_ag(I.TINY)
    _, C_ref = orc.ag_gemm(shards, B)
    _, C = orc.ag_gemm_protocol(shards, B, rank=0, seed=3, max_delay_us=3000.0, global_perm=True,
                                n_consumers=4, skip_wait=True)
    assert not np.array_equal(C, C_ref)


def _rs_inputs(dist_a="normal", peer="normal", W=4, M=32, K=24, N=20, dtype="bf16", seed=2):
    w = I.RSWorkload("t", W=W, M=M, K=K, N=N, dtype=dtype, dist=dist_a, std=0.5, peer_dist=peer, seed_index=seed)
    return I.make_rs(w)


def test_gemm_rs_exact_small(orc):
    A, B, parts = _rs_inputs(W=2, M=6, K=9, N=5)
    for rank in range(2):
        C = orc.gemm_rs(A, B, parts, rank)
        exact, mag = _exact_gemm(A[rank * 3:(rank + 1) * 3], B, "kn")
        for i in range(3):
            for j in range(5):
                v = exact[i][j] + sum(Fraction(float(parts[p][i, j])) for p in range(2) if p != rank)
                assert abs(Fraction(float(C[i, j])) - v) <= Fraction(2 ** -40) * (mag[i][j] + 8)


def test_gemm_rs_zero_A_is_sum_of_peers(orc):
    A, B, parts = _rs_inputs(dist_a="int", peer="int")
    A = np.zeros_like(A)
    for rank in range(4):
        C = orc.gemm_rs(A, B, parts, rank)
        ref = sum(parts[p].astype(np.float64) for p in range(4) if p != rank)
        assert np.array_equal(C, ref)


def test_gemm_rs_zero_peers_is_block_product(orc):
    A, B, parts = _rs_inputs(dist_a="int", peer="zero")
    full = _vals(A).astype(np.int64) @ _vals(B).astype(np.int64)
    for rank in range(4):
        C = orc.gemm_rs(A, B, parts, rank)
        assert np.array_equal(C, full[rank * 8:(rank + 1) * 8].astype(np.float64))


def test_gemm_rs_linear_in_peers(orc):
    A, B, parts = _rs_inputs(dist_a="int", peer="int")
    base = orc.gemm_rs(A, B, [np.zeros_like(p) for p in parts], 1)
    one = orc.gemm_rs(A, B, parts, 1)
    two = orc.gemm_rs(A, B, [2 * p for p in parts], 1)
    assert np.array_equal(two - base, 2 * (one - base))
    # the local rank's own entry is never read
    poisoned = [p.copy() for p in parts]
    poisoned[1][...] = np.nan
    assert np.array_equal(orc.gemm_rs(A, B, poisoned, 1), one)


def test_moe_route_matches_stable_sort(orc):
    w = I.scaled(I.MOE, T=256, W=4)
    _, _, logits = I.make_moe(w)
    ids, off, row_token = orc.moe_route(logits, w.topk)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :w.topk]
    assert np.array_equal(ids, ref)
    assert off[0] == 0 and off[-1] == w.T * w.topk
    assert np.all(np.diff(off) >= 0)
    for e in range(w.E):
        toks = row_token[off[e]:off[e + 1]]
        assert np.all(np.diff(toks) > 0)                 # ascending, no duplicates
        assert np.array_equal(np.sort(np.nonzero((ids == e).any(1))[0]), toks)
    counts = np.bincount(row_token, minlength=w.T)
    assert np.all(counts == w.topk)


def test_moe_route_ties_go_to_lower_id(orc):
    logits = np.zeros((3, 6), np.float32)
    logits[1, 4] = 1.0
    logits[2] = [0.5, 2.0, 0.5, 2.0, 0.5, 0.5]
    ids, off, rt = orc.moe_route(logits, 3)
    assert ids.tolist() == [[0, 1, 2], [4, 0, 1], [1, 3, 0]]
    # expert 0: tokens 0,1,2; expert 1: tokens 0,1,2; expert 2: token 0; 3: token 2; 4: token 1; 5: none
    assert off.tolist() == [0, 3, 6, 7, 8, 9, 9]
    assert rt.tolist() == [0, 1, 2, 0, 1, 2, 0, 2, 1]


def test_moe_skew_is_zipf_like():
    _, _, logits = I.make_moe(I.MOE)
    top = np.argsort(-logits, axis=1, kind="stable")[:, :I.MOE.topk]
    sizes = np.bincount(top.ravel(), minlength=I.MOE.E)
    assert sizes.sum() == I.MOE.T * I.MOE.topk
    assert sizes.max() > 4 * sizes.mean() and sizes.min() < sizes.mean() / 4


def test_moe_with_one_expert_is_ag_gemm(orc):
    w = I.scaled(I.MOE, T=64, H=48, I=40, E=1, topk=1, W=4)
    shards, We, logits = I.make_moe(w)
    X, ids, off, rt, Y = orc.moe_ag_gemm(shards, We, logits, 1)
    _, C = orc.ag_gemm(shards, We[0])
    assert np.array_equal(Y, C)


def test_moe_exact_small(orc):
    w = I.scaled(I.MOE, T=8, H=7, I=5, E=4, topk=2, W=2, std=0.5)
    shards, We, logits = I.make_moe(w)
    X, ids, off, rt, Y = orc.moe_ag_gemm(shards, We, logits, 2)
    for row in range(16):
        e = int(np.searchsorted(off, row, side="right") - 1)
        exact, mag = _exact_gemm(X[rt[row]:rt[row] + 1], We[e], "kn")
        for j in range(5):
            assert abs(Fraction(float(Y[row, j])) - exact[0][j]) <= Fraction(7 * 2 ** -53) * mag[0][j]
    # nk storage of the expert weights gives the same bits
    _, _, _, _, Y2 = orc.moe_ag_gemm(shards, np.ascontiguousarray(np.transpose(We, (0, 2, 1))), logits, 2,
                                     w_layout="nk")
    assert np.array_equal(Y, Y2)


# ---------------------------------------------------------------------------
# MoE GEMM + ReduceScatter (combine side)
# ---------------------------------------------------------------------------
def _group(ids, E):
    """Routing tables of a given pick matrix: rows grouped by expert ascending, tokens ascending inside."""
    T, k = ids.shape
    off = np.zeros(E + 1, np.int32)
    rows = []
    for e in range(E):
        off[e] = len(rows)
        rows += [t for t in range(T) for j in range(k) if ids[t, j] == e]
    off[E] = len(rows)
    return off, np.array(rows, np.int32)


def _moe_rs_small(seed=7, T=16, k=2, E=4, n_in=8, H=6, W=4, dist="int"):
    w = I.scaled(I.MOE_RS, T=T, topk=k, E=E, I=n_in, H=H, W=W, dist=dist, peer_dist="int", seed_index=seed)
    return w, I.make_moe_rs(w)


def test_moe_rs_single_expert_top1_is_dense_gemm_rs(orc):
    # one expert, one pick per token, gate 1: the grouped rows are the tokens in order, so P = Hg @ W2[0]
    # (a plain matrix product) and C adds the peers' blocks
    w, (Hg, W2, gate, logits, parts) = _moe_rs_small(T=16, k=1, E=1, n_in=8, H=6, W=4)
    ids = np.zeros((16, 1), np.int32)
    off, rt = _group(ids, 1)
    gate = np.ones((16, 1), np.float32)
    A = I.bf16_bits_to_f32(Hg).astype(np.float64)
    B = I.bf16_bits_to_f32(W2[0]).astype(np.float64)
    P_ref = A @ B
    for rank in range(4):
        C = orc.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, rank)
        blk = slice(rank * 4, rank * 4 + 4)
        C_ref = P_ref[blk] + sum(parts[p].astype(np.float64) for p in range(4) if p != rank)
        assert np.array_equal(C, C_ref)


def test_moe_rs_one_hot_routing_is_per_expert_products(orc):
    # token t picks expert t % E alone, with gate 2^-(t % 3): P[t] = gate * Hg[row] @ W2[t % E]
    w, (Hg, W2, gate, logits, parts) = _moe_rs_small(T=24, k=1, E=3, n_in=10, H=7, W=2)
    ids = (np.arange(24) % 3).astype(np.int32)[:, None]
    off, rt = _group(ids, 3)
    gate = (2.0 ** -(np.arange(24) % 3)).astype(np.float32)[:, None]
    P = orc.moe_gemm_rs_p(Hg, W2, gate, ids, off, rt, np.arange(24))
    A = I.bf16_bits_to_f32(Hg).astype(np.float64)
    for t in range(24):
        e = t % 3
        r = int(np.nonzero(rt[off[e]:off[e + 1]] == t)[0][0]) + int(off[e])
        ref = float(gate[t, 0]) * (A[r] @ I.bf16_bits_to_f32(W2[e]).astype(np.float64))
        assert np.array_equal(P[t], ref)


def test_moe_rs_gates_are_linear(orc):
    w, (Hg, W2, gate, logits, parts) = _moe_rs_small(T=16, k=3, E=5, n_in=8, H=6, W=4)
    ids, off, rt = orc.moe_route(logits, 3)
    g = (2.0 ** -np.random.default_rng(1).integers(0, 3, size=(16, 3))).astype(np.float32)
    C1 = orc.moe_gemm_rs(Hg, W2, g, ids, off, rt, parts, 1)
    C2 = orc.moe_gemm_rs(Hg, W2, 2 * g, ids, off, rt, parts, 1)
    peers = sum(parts[p].astype(np.float64) for p in range(4) if p != 1)
    assert np.array_equal(C2 - peers, 2 * (C1 - peers))


def test_moe_rs_expert_relabelling_is_invisible(orc):
    # renaming the experts (weights permuted alike, rows regrouped in the new expert order) leaves P unchanged
    w, (Hg, W2, gate, logits, parts) = _moe_rs_small(T=12, k=2, E=4, n_in=8, H=5, W=2)
    ids, off, rt = orc.moe_route(logits, 2)
    P = orc.moe_gemm_rs_p(Hg, W2, gate, ids, off, rt, np.arange(12))
    pi = np.array([2, 0, 3, 1])                      # expert e is called pi[e] after renaming
    ids2 = pi[ids].astype(np.int32)
    W22 = np.empty_like(W2)
    W22[pi] = W2
    off2, rt2 = _group(ids2, 4)
    # row of (t, new expert pi[e]) takes the old row of (t, e)
    Hg2 = np.empty_like(Hg)
    for e in range(4):
        for r in range(off[e], off[e + 1]):
            t = rt[r]
            r2 = int(np.nonzero(rt2[off2[pi[e]]:off2[pi[e] + 1]] == t)[0][0]) + int(off2[pi[e]])
            Hg2[r2] = Hg[r]
    P2 = orc.moe_gemm_rs_p(Hg2, W22, gate, ids2, off2, rt2, np.arange(12))
    assert np.array_equal(P, P2)


def test_moe_rs_pick_order_only_moves_gates(orc):
    # reversing each token's picks together with its gates leaves P unchanged (integer data: exact sums)
    w, (Hg, W2, gate, logits, parts) = _moe_rs_small(T=10, k=3, E=6, n_in=8, H=4, W=2)
    ids, off, rt = orc.moe_route(logits, 3)
    g = np.ones((10, 3), np.float32)
    P = orc.moe_gemm_rs_p(Hg, W2, g, ids, off, rt, np.arange(10))
    P2 = orc.moe_gemm_rs_p(Hg, W2, g[:, ::-1].copy(), ids[:, ::-1].copy(), off, rt, np.arange(10))
    assert np.array_equal(P, P2)


def test_moe_rs_planted_mistake_is_caught(orc):
    # a routing table that sends a pick to a group without the token is rejected
    w, (Hg, W2, gate, logits, parts) = _moe_rs_small(T=8, k=1, E=2, n_in=8, H=4, W=2)
    ids = np.zeros((8, 1), np.int32)
    off, rt = _group(ids, 2)
    bad = ids.copy()
    bad[3, 0] = 1
    with pytest.raises(ValueError):
        orc.moe_gemm_rs_p(Hg, W2, gate, bad, off, rt, np.arange(8))


# ---- low-latency packets (paper summary, "Method": data and flag share one 8-byte block) ----

def test_ll_pack_word_is_epoch_high_payload_low(orc):
    # closed form with Python integers: word = epoch * 2^32 + payload word
    rng = np.random.default_rng(11)
    payload = rng.integers(0, 2**32, size=37, dtype=np.uint64).astype(np.uint32)
    for epoch in (1, 7, 2**32 - 1):
        got = orc.ll_pack(payload, epoch)
        assert got.dtype == np.uint64 and got.size == payload.size
        assert [int(v) for v in got] == [epoch * 2**32 + int(w) for w in payload]


def test_ll_pack_bytes_of_a_worked_example(orc):
    # two payload words, epoch 5: little-endian bytes, payload first, flag second
    got = orc.ll_pack(np.array([0x11223344, 0xAABBCCDD], np.uint32), 5).tobytes()
    assert got == bytes([0x44, 0x33, 0x22, 0x11, 5, 0, 0, 0, 0xDD, 0xCC, 0xBB, 0xAA, 5, 0, 0, 0])


def test_ll_pack_of_bf16_rows_keeps_element_pairs(orc):
    # a bf16 payload packs two elements per word: the low half of each packet is
    # the pair's bytes as laid out in memory, so unpacking the low halves of a
    # row's packets gives the row back
    row = np.arange(1, 9, dtype=np.uint16)
    got = orc.ll_pack(row, 3)
    assert np.array_equal((got & 0xFFFFFFFF).astype(np.uint32).view(np.uint16), row)
    assert np.all(got >> 32 == 3)


def test_ll_buffer_slots_follow_the_gathered_rows(orc):
    rng = np.random.default_rng(12)
    shards = [rng.integers(0, 2**16, size=(4, 6), dtype=np.uint64).astype(np.uint16) for _ in range(3)]
    before = np.full(3 * 4 * 6 // 2, 99, np.uint64)
    got = orc.ll_buffer(shards, rank=1, epoch=9, chunk_rows=2, before=before)
    gathered = np.concatenate(shards)           # library routine for the row order
    words = gathered.reshape(-1).view(np.uint32)
    per = 4 * 6 // 2
    for p in range(3):
        seg = got[p * per:(p + 1) * per]
        if p == 1:
            assert np.all(seg == 99)              # the local slot is left as it was
        else:
            assert np.array_equal(seg & 0xFFFFFFFF, words[p * per:(p + 1) * per])
            assert np.all(seg >> 32 == 9)


def test_ll_planted_swap_is_caught(orc):
    # a packer that put the flag in the low half would fail the closed form above
    payload = np.array([1, 2, 3], np.uint32)
    good = orc.ll_pack(payload, 4)
    swapped = (good << np.uint64(32)) | (good >> np.uint64(32))
    assert [int(v) for v in swapped] != [4 * 2**32 + int(w) for w in payload]


# ---- ring AllReduce (semantics page, "Example: ring AllReduce with overlap") ----

def _ring_xs(W, N, kind="float", seed=21):
    rng = np.random.default_rng(seed)
    if kind == "int":
        return [rng.integers(-50, 51, size=N).astype(np.float32) for _ in range(W)]
    return [rng.standard_normal(N).astype(np.float32) for _ in range(W)]


@pytest.mark.parametrize("W", [1, 2, 3, 5, 8])
def test_ring_result_is_the_sum_on_every_rank(orc, W):
    xs = _ring_xs(W, W * 12)
    outs, _, _ = orc.ring_allreduce(xs)
    ref = np.sum(np.stack(xs).astype(np.float64), axis=0)           # library routine, fp64
    mag = np.sum(np.abs(np.stack(xs).astype(np.float64)), axis=0)
    for q in range(W):
        assert np.all(np.abs(outs[q] - ref) <= W * 2.0**-24 * mag + 1e-30), q


def test_ring_integer_inputs_are_exact(orc):
    xs = _ring_xs(8, 8 * 20, kind="int")
    outs, _, _ = orc.ring_allreduce(xs)
    ref = np.sum(np.stack(xs).astype(np.int64), axis=0)
    for o in outs:
        assert np.array_equal(o.astype(np.int64), ref)


def test_ring_sums_each_chunk_in_ring_order(orc):
    # W = 3, one element per chunk.  Chunk 0 starts at rank 0 and gains rank 1's, then rank 2's
    # value, each sum rounded to fp32: (2^24 + 1) + 1 rounds to 2^24 twice (ties to even), while
    # 2^24 + (1 + 1) would be 2^24 + 2.  Chunk 1 starts at rank 1: (1 + 2^24) + 1 rounds to 2^24 as
    # well; chunk 2 starts at rank 2: (1 + 1) + 2^24 = 2^24 + 2 exactly.
    xs = [np.array([2.0**24, 1.0, 1.0], np.float32), np.array([1.0, 1.0, 2.0**24], np.float32),
          np.array([1.0, 2.0**24, 1.0], np.float32)]
    outs, _, _ = orc.ring_allreduce(xs)
    for o in outs:
        assert o[0] == 2.0**24 and o[1] == 2.0**24 and o[2] == 2.0**24 + 2


def test_ring_closes_and_rank_view_matches(orc):
    for W in (2, 4, 7):
        xs = _ring_xs(W, W * 8, seed=22 + W)
        outs, inbox, outbox = orc.ring_allreduce(xs)
        for q in range(W):
            # what q sends is what q+1 receives
            assert np.array_equal(outbox[q], inbox[(q + 1) % W])
            # the rank's own recurrence, given what it receives, gives the same result and sends
            o, ob = orc.ring_rank(xs[q], inbox[q], q, W)
            assert np.array_equal(o, outs[q]) and np.array_equal(ob, outbox[q])


def _allreduce_pins_hold(orc, planted=""):
    """The pins of oracle.allreduce: (i) integer-valued fp32 vectors sum exactly, compared with an
    int64 sum; (ii) a hand-worked example whose fp32 running sum would lose the small terms:
    rank 0 holds 2^24, ranks 1..3 hold 1, so the exact sum 2^24 + 3 (representable in fp64) differs
    from every fp32 accumulation order that starts at 2^24 (2^24 + 1 rounds back to 2^24), and
    element 1 is rank 0's alone (-7.5, others 0)."""
    xs = _ring_xs(6, 6 * 40, kind="int", seed=91)
    ok_int = np.array_equal(orc.allreduce(xs, planted=planted), np.sum(np.stack(xs).astype(np.int64), axis=0))
    hand = [np.array([2.0**24, -7.5], np.float32)] + [np.array([1.0, 0.0], np.float32) for _ in range(3)]
    got = orc.allreduce(hand, planted=planted)
    ok_hand = got[0] == 16777219.0 and got[1] == -7.5
    return ok_int and ok_hand


def test_allreduce_pins(orc):
    assert _allreduce_pins_hold(orc)
    # the result is fp64 and has one element per input element
    out = orc.allreduce([np.ones(5, np.float32)] * 3)
    assert out.dtype == np.float64 and out.shape == (5,) and np.all(out == 3.0)


@pytest.mark.parametrize("planted", ["drop_first", "f32"])
def test_allreduce_planted_mistake_is_caught(orc, planted):
    assert not _allreduce_pins_hold(orc, planted=planted)


def test_ring_planted_mistake_is_caught(orc):
    xs = _ring_xs(4, 16, kind="int")
    outs, _, _ = orc.ring_allreduce(xs, planted="rs_chunk")
    ref = np.sum(np.stack(xs).astype(np.int64), axis=0)
    assert not all(np.array_equal(o.astype(np.int64), ref) for o in outs)


# ---- expert-parallel AllToAll ----

def _a2a_case(seed, W=4, E=8, T_r=13, k=3, H=5, invalid=False):
    rng = np.random.default_rng(seed)
    X = [I.f32_to_bf16_bits(rng.standard_normal((T_r, H)).astype(np.float32)) for _ in range(W)]
    topk = [np.array([rng.permutation(E)[:k] for _ in range(T_r)], np.int32) for _ in range(W)]
    if invalid:
        for tk in topk:
            tk[rng.integers(0, T_r, 3), rng.integers(0, k, 3)] = [-1, E, E + 7]
    return X, topk


@pytest.mark.parametrize("invalid", [False, True])
def test_a2a_dispatch_delivers_every_pick_once_to_its_owner(orc, invalid):
    from collections import Counter
    W, E = 4, 8
    X, topk = _a2a_case(1, W=W, E=E, invalid=invalid)
    E_l = E // W
    got = Counter()
    for r in range(W):
        recv, tok, cnt = orc.a2a_dispatch(X, topk, E, r)
        for l in range(E_l):
            for p in range(W):
                n = int(cnt[l, p])
                ts = tok[l, p, :n]
                assert (np.diff(ts) > 0).all() and (tok[l, p, n:] == -1).all()
                assert np.array_equal(recv[l, p, :n], X[p][ts])
                assert not recv[l, p, n:].any()
                got.update((p, int(t), r * E_l + l) for t in ts)
    want = Counter((p, t, int(e)) for p in range(W) for t in range(topk[p].shape[0]) for e in topk[p][t]
                   if 0 <= e < E)
    assert got == want
    assert sum(got.values()) == sum(int(((tk >= 0) & (tk < E)).sum()) for tk in topk)


def test_a2a_dispatch_blocks_concatenate_to_moe_groups(orc):
    # the expert groups of the (separately written, C) MoE routing over all ranks' tokens are the
    # dispatch blocks of that expert's owner, taken source by source
    W, E, T, k = 4, 16, 96, 4
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, off, row_token = orc.moe_route(logits, k)
    T_r, E_l = T // W, E // W
    X = [np.arange(T_r * 2, dtype=np.uint16).reshape(T_r, 2) for _ in range(W)]
    topk = [ids[p * T_r:(p + 1) * T_r] for p in range(W)]
    for r in range(W):
        _, tok, cnt = orc.a2a_dispatch(X, topk, E, r)
        for l in range(E_l):
            e = r * E_l + l
            cat = np.concatenate([p * T_r + tok[l, p, :cnt[l, p]] for p in range(W)])
            assert np.array_equal(cat, row_token[off[e]:off[e + 1]])


def _dense_combine(back, topk, gate, E):
    """Independent matrix form: G[t, e] = sum of the gates of t's picks of e; the slot of t in expert e's list
    is the running count (cumulative sum) of the tokens up to t that picked e, minus one."""
    W = len(back)
    E_l = E // W
    topk = np.asarray(topk)
    T_r = topk.shape[0]
    onehot = np.zeros((T_r, E), np.float64)
    G = np.zeros((T_r, E), np.float64)
    for j in range(topk.shape[1]):
        valid = (topk[:, j] >= 0) & (topk[:, j] < E)
        rows = np.nonzero(valid)[0]
        onehot[rows, topk[rows, j]] = 1.0
        G[rows, topk[rows, j]] += gate[rows, j].astype(np.float64)
    hit = onehot > 0
    slots = np.cumsum(hit, axis=0) - 1
    H = back[0].shape[2]
    out = np.zeros((T_r, H), np.float64)
    for e in range(E):
        Y = I.bf16_bits_to_f32(back[e // E_l][e % E_l]).astype(np.float64)
        sel = np.where(hit[:, e], slots[:, e], 0)
        out += (G[:, e] * hit[:, e])[:, None] * Y[sel]
    return out


@pytest.mark.parametrize("invalid", [False, True])
def test_a2a_combine_matches_dense_selection_form(orc, invalid):
    W, E, T_r, k, H = 4, 8, 13, 3, 6
    rng = np.random.default_rng(11)
    _, topk = _a2a_case(2, W=W, E=E, T_r=T_r, k=k, H=H, invalid=invalid)
    back = [I.f32_to_bf16_bits(rng.standard_normal((E // W, T_r, H)).astype(np.float32)) for _ in range(W)]
    gate = rng.random((T_r, k), dtype=np.float32)
    for r in (0, 3):
        out = orc.a2a_combine(back, topk[r], gate, E)
        ref = _dense_combine(back, topk[r], gate, E)
        assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_a2a_combine_of_identity_experts_returns_the_tokens(orc):
    # each expert sends back exactly the rows it received; gates that are powers of two summing to one
    # make every sum exact, so the combine must return each token's own row bit for bit
    W, E, T_r, k, H = 4, 8, 17, 4, 5
    X, topk = _a2a_case(3, W=W, E=E, T_r=T_r, k=k, H=H)
    gate = np.tile(np.array([0.5, 0.25, 0.125, 0.125], np.float32), (T_r, 1))
    recv = [orc.a2a_dispatch(X, topk, E, q)[0] for q in range(W)]
    for r in range(W):
        back = [recv[q][:, r] for q in range(W)]
        out = orc.a2a_combine(back, topk[r], gate, E)
        assert np.array_equal(out, I.bf16_bits_to_f32(X[r]).astype(np.float64))
        cbuf = orc.a2a_combine_recv(back, topk[r], E)
        for e in range(E):
            ts = orc.a2a_tokens(topk[r], e)
            assert np.array_equal(cbuf[e, :len(ts)], X[r][ts])


def test_a2a_slots_of_a_worked_example(orc):
    # three tokens, E = 4: token 0 picks (2, 0), token 1 picks (0, 3), token 2 picks (0, 2)
    topk = np.array([[2, 0], [0, 3], [0, 2]], np.int32)
    assert orc.a2a_slots(topk, 4).tolist() == [[0, 0], [1, 0], [2, 1]]


def test_a2a_planted_slot_mistake_is_caught(orc, monkeypatch):
    W, E, T_r, k, H = 4, 8, 13, 3, 6
    rng = np.random.default_rng(12)
    _, topk = _a2a_case(4, W=W, E=E, T_r=T_r, k=k, H=H)
    back = [I.f32_to_bf16_bits(rng.standard_normal((E // W, T_r, H)).astype(np.float32)) for _ in range(W)]
    gate = rng.random((T_r, k), dtype=np.float32)
    good = orc.a2a_slots
    # counting the token itself (a slot off by one) must break the agreement with the dense form
    monkeypatch.setattr(orc, "a2a_slots", lambda tk, E_: np.minimum(good(tk, E_) + 1, T_r - 1))
    out = orc.a2a_combine(back, topk[1], gate, E)
    assert not np.allclose(out, _dense_combine(back, topk[1], gate, E), rtol=1e-6, atol=1e-6)
