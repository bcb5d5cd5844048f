"""CPU oracle (test infrastructure only).

Plain, slow, obviously correct definitions of what the signal-gated tiled path
computes, in double precision, written in C (``oracle.c``) and wrapped here with
ctypes and numpy.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product path never does, and this
package imports nothing from the product.

Functions and the passage each follows (page titles as on the pages):

* ``allgather``      -- Triton-distributed semantics page, "AllGather + GEMM overlap":
                        the producer gathers every PE's tiles into one buffer.
* ``ag_gemm``        -- same section: C = AllGather(A) * B_local.
* ``ll_pack`` / ``ll_buffer`` -- paper summary, "Method" (low-latency protocol for
                        short messages): data and flag stored together in 8-byte
                        blocks; the packets an LL AllGather leaves in the receiver's
                        buffer.
* ``gemm_rs``        -- Triton-distributed semantics page, "GEMM + ReduceScatter overlap";
                        Triton-distributed paper summary, "Method" (intra-node
                        ReduceScatter in push mode): each rank reduces its own row block.
* ``moe_route`` / ``moe_ag_gemm`` -- paper summary, "Experiments" (MoE routing
                        operations) and the DITRON article, "three-level tiling"
                        (dynamic per-expert sizes): top-k routing, expert-grouped rows.
* ``moe_gemm_rs``    -- paper summary, "Experiments" (MoE ReduceScatter) and the semantics
                        page, "GEMM + ReduceScatter overlap": the combine side of an MoE
                        layer -- grouped rows times their expert's weight, each token's
                        rows summed with its gate weights, then the ReduceScatter over
                        token blocks.
* ``allreduce`` / ``ring_allreduce`` / ``ring_rank`` -- semantics page, "Example: ring
                        AllReduce with overlap": the sum over ranks, the ring's two
                        phases emulated over all ranks (the messages every rank
                        receives and sends), and one rank's steps given what it
                        receives.
* ``a2a_dispatch`` / ``a2a_slots`` / ``a2a_combine_recv`` / ``a2a_combine`` -- paper summary,
                        "Experiments" (expert-parallel AllToAll dispatch and combine) and the
                        complete guide, §4.2 (low-latency AllToAll for expert parallelism): each
                        token's row goes to the owner of every expert it picked, and comes back
                        as that expert's output, summed with the token's gate weights.
* ``ag_gemm_protocol`` -- semantics page, "Producer-consumer model", "Signal-based
                        synchronization", "Threadblock swizzle", "Token-based data
                        dependency"; paper summary, "Method" (AMD full-mesh swizzle):
                        the same C computed through host threads that copy tiles,
                        release flags, and wait on flags before reading.

bf16 arrays are numpy ``uint16`` bit patterns; fp32 arrays are ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
KN, NK = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (OpenMP over output rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wno-unused-function", _SRC, "-o", tmp, "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.orc_allgather.argtypes = [P, I32, I64, I64, P]
        lib.orc_ll_pack.argtypes = [P, I64, ctypes.c_uint32, P]
        lib.orc_gemm_rows.argtypes = [P, I32, P, I32, I32, I64, I64, I64, P, I64, P, I32]
        lib.orc_gemm_rs.argtypes = [P, I32, P, I32, I32, I64, I64, I64, P, I32, I32, P, I64, P, I32]
        lib.orc_moe_route.argtypes = [P, I64, I32, I32, P, P, P]
        lib.orc_moe_route.restype = I32
        lib.orc_moe_gemm_rows.argtypes = [P, P, I32, I64, I64, I32, P, P, P, I64, P, I32]
        lib.orc_moe_gemm_rs.argtypes = [P, P, I32, I64, I32, I64, I64, I32, P, P, P, P, P, I32, I32, P, I64, P, P,
                                        I32]
        lib.orc_moe_gemm_rs.restype = I32
        lib.orc_ag_gemm_protocol.argtypes = [P, I32, I32, I32, P, I32, I32, I64, I64, I64, I64, I64,
                                             ctypes.c_uint64, D, I32, I32, I32, I32, P, P]
        lib.orc_ag_gemm_protocol.restype = I32
        lib.orc_max_threads.restype = I32
        lib.orc_panel_order.argtypes = [I32, I32, I64, I64, I32, P]
        lib.orc_panel_order.restype = I32
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().orc_max_threads())


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError("oracle inputs are bf16 bits (uint16) or float32, got %s" % a.dtype)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _rows(rows):
    if rows is None:
        return None, None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, _ptr(r), len(r)


def _lay(layout: str) -> int:
    return {"kn": KN, "nk": NK}[layout]


def allgather(shards) -> np.ndarray:
    """Stack the row shards in shard order (shard p -> rows [p*R, (p+1)*R))."""
    shards = [np.ascontiguousarray(s) for s in shards]
    R, K = shards[0].shape
    out = np.empty((R * len(shards), K), dtype=shards[0].dtype)
    _load().orc_allgather(_ptr_array(shards), len(shards), R, K * shards[0].itemsize, _ptr(out))
    return out


def ll_pack(payload: np.ndarray, epoch: int) -> np.ndarray:
    """Low-latency packets of a payload (any dtype, a whole number of 4-byte words): one uint64
    per payload word, the word in bits 0..31 and the epoch in bits 32..63."""
    words = np.ascontiguousarray(payload).reshape(-1).view(np.uint32)
    out = np.empty(words.size, dtype=np.uint64)
    _load().orc_ll_pack(_ptr(words), words.size, int(epoch), _ptr(out))
    return out


def ll_buffer(shards, rank: int, epoch: int, chunk_rows: int, before: np.ndarray = None) -> np.ndarray:
    """Expected LL receive buffer after an LL AllGather (as uint64 words): each remote shard's
    rows, chunk by chunk (chunk_rows rows, in gathered-row order), as packets of `epoch`; the
    local shard's slot keeps what it held (`before`, zeros by default)."""
    R = shards[0].shape[0]
    assert R % chunk_rows == 0
    out = np.zeros(sum(s.size * s.itemsize for s in shards) // 4, dtype=np.uint64) if before is None \
        else np.array(before, dtype=np.uint64).reshape(-1)
    per = shards[0].size * shards[0].itemsize // 4
    for p, s in enumerate(shards):
        if p != rank:
            out[p * per:(p + 1) * per] = ll_pack(s, epoch)
    return out


def gemm(A: np.ndarray, B: np.ndarray, b_layout: str = "kn", rows=None, threads: int = 0) -> np.ndarray:
    """C = A * B in float64 (ascending-k sums); only the listed rows of A if given."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    M, K = A.shape
    N = B.shape[1] if b_layout == "kn" else B.shape[0]
    assert (B.shape[0] if b_layout == "kn" else B.shape[1]) == K
    r, rp, nr = _rows(rows)
    C = np.empty((nr if r is not None else M, N), np.float64)
    _load().orc_gemm_rows(_ptr(A), _dt(A), _ptr(B), _dt(B), _lay(b_layout), M, K, N, rp, nr, _ptr(C), threads)
    return C


def ag_gemm(shards, B, b_layout: str = "kn", rows=None, threads: int = 0):
    """(A_full, C) for C = AllGather(shards) * B; C holds only `rows` if given."""
    A_full = allgather(shards)
    return A_full, gemm(A_full, B, b_layout, rows, threads)


def gemm_rs(A_local, B, partials, rank: int, b_layout: str = "kn", rows=None, threads: int = 0) -> np.ndarray:
    """C_shard for `rank`: block `rank` of A_local*B plus every other rank's partial block."""
    A = np.ascontiguousarray(A_local)
    B = np.ascontiguousarray(B)
    W = len(partials)
    M, K = A.shape
    N = B.shape[1] if b_layout == "kn" else B.shape[0]
    assert M % W == 0
    parts = [np.ascontiguousarray(p, dtype=np.float32) for p in partials]
    for p in parts:
        assert p.shape == (M // W, N)
    r, rp, nr = _rows(rows)
    C = np.empty((nr if r is not None else M // W, N), np.float64)
    _load().orc_gemm_rs(_ptr(A), _dt(A), _ptr(B), _dt(B), _lay(b_layout), M, K, N, _ptr_array(parts), W, rank,
                        rp, nr, _ptr(C), threads)
    return C


def moe_route(logits: np.ndarray, topk: int):
    """(topk_ids T x k, expert_off E+1, row_token T*k) by descending logit, ties to the lower id."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, topk), np.int32)
    off = np.empty(E + 1, np.int32)
    row_token = np.empty(T * topk, np.int32)
    rc = _load().orc_moe_route(_ptr(logits), T, E, topk, _ptr(ids), _ptr(off), _ptr(row_token))
    if rc != 0:
        raise ValueError("bad top-k")
    return ids, off, row_token


def moe_gemm(X_full, W_experts, expert_off, row_token, w_layout: str = "kn", rows=None, threads: int = 0):
    """Y[row] = X_full[row_token[row]] * W_e for the expert e owning `row` (float64)."""
    X = np.ascontiguousarray(X_full, dtype=np.uint16)
    Wt = np.ascontiguousarray(W_experts, dtype=np.uint16)
    E = Wt.shape[0]
    H = X.shape[1]
    I = Wt.shape[2] if w_layout == "kn" else Wt.shape[1]
    off = np.ascontiguousarray(expert_off, dtype=np.int32)
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    r, rp, nr = _rows(rows)
    Y = np.empty((nr if r is not None else int(off[E]), I), np.float64)
    _load().orc_moe_gemm_rows(_ptr(X), _ptr(Wt), _lay(w_layout), H, I, E, _ptr(off), _ptr(rt), rp, nr, _ptr(Y),
                              threads)
    return Y


def moe_ag_gemm(shards, W_experts, logits, topk: int, w_layout: str = "kn", rows=None, threads: int = 0):
    """(X_full, topk_ids, expert_off, row_token, Y) for the MoE AllGather-grouped-GEMM."""
    X_full = allgather(shards)
    ids, off, rt = moe_route(logits, topk)
    return X_full, ids, off, rt, moe_gemm(X_full, W_experts, off, rt, w_layout, rows, threads)


def moe_gemm_rs(Hg, W2, gate, topk_ids, expert_off, row_token, partials, rank: int, w_layout: str = "kn",
                tokens=None, want_p: bool = False, threads: int = 0):
    """C for `rank` (its T/W tokens x H, float64), and P (tokens x H) when want_p.

    Hg: grouped rows (rows x I bf16), W2: E x I x H ("kn") or E x H x I ("nk") bf16, gate: T x k float32,
    topk_ids: T x k, expert_off: E+1, row_token: rows; partials: W arrays of (T/W) x H float32 ([rank] unused).
    tokens: token indices to compute (default: the rank's block).
    """
    Hg = np.ascontiguousarray(Hg, dtype=np.uint16)
    W2 = np.ascontiguousarray(W2, dtype=np.uint16)
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    off = np.ascontiguousarray(expert_off, dtype=np.int32)
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    T, k = ids.shape
    E = W2.shape[0]
    I = Hg.shape[1]
    H = W2.shape[2] if w_layout == "kn" else W2.shape[1]
    W = len(partials)
    assert T % W == 0
    parts = [np.ascontiguousarray(p, dtype=np.float32) if p is not None else np.zeros((T // W, H), np.float32)
             for p in partials]
    if tokens is None:
        tokens = np.arange(rank * (T // W), (rank + 1) * (T // W), dtype=np.int64)
    tk = np.ascontiguousarray(tokens, dtype=np.int64)
    C = np.empty((len(tk), H), np.float64)
    P = np.empty((len(tk), H), np.float64) if want_p else None
    rc = _load().orc_moe_gemm_rs(_ptr(Hg), _ptr(W2), _lay(w_layout), T, k, I, H, E, _ptr(ids), _ptr(gate), _ptr(off),
                                 _ptr(rt), _ptr_array(parts), W, rank, _ptr(tk), len(tk),
                                 _ptr(P) if want_p else None, _ptr(C), threads)
    if rc != 0:
        raise ValueError("moe_gemm_rs: bad routing tables or tokens (%d)" % rc)
    return (C, P) if want_p else C


def moe_gemm_rs_p(Hg, W2, gate, topk_ids, expert_off, row_token, tokens, w_layout: str = "kn", threads: int = 0):
    """P rows (the combined partial, float64) for any tokens, without the ReduceScatter."""
    Hg = np.ascontiguousarray(Hg, dtype=np.uint16)
    W2 = np.ascontiguousarray(W2, dtype=np.uint16)
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    off = np.ascontiguousarray(expert_off, dtype=np.int32)
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    T, k = ids.shape
    E = W2.shape[0]
    I = Hg.shape[1]
    H = W2.shape[2] if w_layout == "kn" else W2.shape[1]
    tk = np.ascontiguousarray(tokens, dtype=np.int64)
    P = np.empty((len(tk), H), np.float64)
    rc = _load().orc_moe_gemm_rs(_ptr(Hg), _ptr(W2), _lay(w_layout), T, k, I, H, E, _ptr(ids), _ptr(gate), _ptr(off),
                                 _ptr(rt), None, 1, 0, _ptr(tk), len(tk), _ptr(P), None, threads)
    if rc != 0:
        raise ValueError("moe_gemm_rs: bad routing tables (%d)" % rc)
    return P


def panel_order(W: int, rank: int, rows_per_shard: int, panel_rows: int, order: str = "shard") -> np.ndarray:
    """Order in which the emulated consumer takes the row panels."""
    out = np.empty(W * rows_per_shard // panel_rows, np.int64)
    if _load().orc_panel_order(W, rank, rows_per_shard, panel_rows, {"shard": 0, "mesh": 1}[order], _ptr(out)):
        raise ValueError("bad panel-order arguments")
    return out


def ag_gemm_protocol(shards, B, rank: int, b_layout: str = "kn", flag_rows: int = 16, panel_rows: int = 16,
                     seed: int = 0, max_delay_us: float = 0.0, global_perm: bool = False, order: str = "shard",
                     n_consumers: int = 4, skip_wait: bool = False):
    """(A_gathered, C) computed through the emulated signal protocol.

    The gathered buffer starts as NaN poison, so a consumer that read a tile
    before its flag would produce NaN or different bits.  ``skip_wait`` drops
    the consumer's wait (a deliberately wrong oracle, for tests of the tests).
    """
    shards = [np.ascontiguousarray(s) for s in shards]
    B = np.ascontiguousarray(B)
    W = len(shards)
    R, K = shards[0].shape
    M = R * W
    N = B.shape[1] if b_layout == "kn" else B.shape[0]
    dt = _dt(shards[0])
    A_g = np.empty((M, K), shards[0].dtype)
    A_g.view(np.uint16 if dt == BF16 else np.uint32)[...] = 0x7FC0 if dt == BF16 else 0x7FC00000
    C = np.empty((M, N), np.float64)
    rc = _load().orc_ag_gemm_protocol(_ptr_array(shards), W, rank, dt, _ptr(B), _dt(B), _lay(b_layout), M, K, N,
                                      flag_rows, panel_rows, seed, max_delay_us, int(global_perm),
                                      {"shard": 0, "mesh": 1}[order], n_consumers, int(skip_wait), _ptr(A_g), _ptr(C))
    if rc != 0:
        raise ValueError("bad protocol arguments")
    return A_g, C


# ---- ring AllReduce (semantics page, "Example: ring AllReduce with overlap") ----

def allreduce(xs, planted: str = "") -> np.ndarray:
    """The plain definition: the elementwise sum of the ranks' vectors, in double precision.

    ``planted`` (tests only, to show the pins catch a plausible mistake): "drop_first" leaves out
    rank 0's vector, "f32" accumulates in single precision."""
    acc = np.float32 if planted == "f32" else np.float64
    out = np.zeros(np.asarray(xs[0]).size, dtype=acc)
    for q, x in enumerate(xs):
        if planted == "drop_first" and q == 0:
            continue
        out += np.asarray(x, dtype=acc).reshape(-1)
    return out.astype(np.float64)


def _f32_add(a, b):
    """One fp32 addition: the sum in double precision rounded once to fp32.  Double has more than
    2 * 24 + 2 bits of precision, so this equals the correctly rounded fp32 sum."""
    return (np.asarray(a, np.float64) + np.asarray(b, np.float64)).astype(np.float32)


def ring_allreduce(xs, planted: str = ""):
    """Emulate the ring over all W ranks, step by step in the pages' two phases.

    Chunk c of a vector is [c*C, (c+1)*C), C = N / W.  Rank q receives from q-1 and sends to q+1.
    ReduceScatter step s = 0..W-2: q sends chunk q-s (its own x at s = 0, else what it reduced at
    step s-1) and receives chunk q-s-1, adding its own x to it in fp32; after W-1 steps q holds the
    full chunk q+1.  AllGather step s = 0..W-2: q sends chunk q+1-s (the chunk it finished, then
    what it received the step before) and receives the full chunk q-s.

    Returns (outs, inboxes, outboxes): per rank the fp32 result, the 2(W-1) messages it received
    and the 2(W-1) it sent (message k = s in the ReduceScatter, W-1+s in the AllGather).
    ``planted`` (tests only): "rs_chunk" receives chunk q-s instead of q-s-1.
    """
    xs = [np.asarray(x, np.float32).reshape(-1) for x in xs]
    W = len(xs)
    N = xs[0].size
    assert N % W == 0
    C = N // W

    def ch(v, c):
        c %= W
        return v[c * C:(c + 1) * C]

    outs = [np.full(N, np.nan, np.float32) for _ in range(W)]
    if W == 1:
        outs[0][:] = xs[0]
        return outs, [np.zeros((0, C), np.float32)], [np.zeros((0, C), np.float32)]
    inbox = [np.zeros((2 * (W - 1), C), np.float32) for _ in range(W)]
    outbox = [np.zeros((2 * (W - 1), C), np.float32) for _ in range(W)]
    reduced = [None] * W
    for s in range(W - 1):
        for q in range(W):
            outbox[q][s] = ch(xs[q], q) if s == 0 else reduced[q]
        for q in range(W):
            got = outbox[(q - 1) % W][s]
            inbox[q][s] = got
            c = q - s if planted == "rs_chunk" else q - s - 1
            reduced[q] = _f32_add(ch(xs[q], c), got)
    for q in range(W):
        ch(outs[q], q + 1)[:] = reduced[q]
    last = list(reduced)
    for s in range(W - 1):
        k = W - 1 + s
        for q in range(W):
            outbox[q][k] = last[q]
        for q in range(W):
            got = outbox[(q - 1) % W][k]
            inbox[q][k] = got
            ch(outs[q], q - s)[:] = got
            last[q] = got
    return outs, inbox, outbox


def ring_rank(x, inbox, rank: int, W: int):
    """One rank's steps given the messages it receives (inbox: 2(W-1) x C, message k in row k):
    returns (out, outbox) as that rank computes and sends them."""
    x = np.asarray(x, np.float32).reshape(-1)
    N = x.size
    C = N // W
    out = np.full(N, np.nan, np.float32)
    if W == 1:
        out[:] = x
        return out, np.zeros((0, C), np.float32)
    inbox = np.asarray(inbox, np.float32).reshape(2 * (W - 1), C)
    outbox = np.zeros((2 * (W - 1), C), np.float32)

    def sl(c):
        c %= W
        return slice(c * C, (c + 1) * C)

    outbox[0] = x[sl(rank)]
    for k in range(W - 1):
        c = rank - k - 1
        v = _f32_add(x[sl(c)], inbox[k])
        if k < W - 2:
            outbox[k + 1] = v
        else:
            out[sl(c)] = v
            outbox[W - 1] = v
    for s in range(W - 1):
        k = W - 1 + s
        out[sl(rank - s)] = inbox[k]
        if s < W - 2:
            outbox[k + 1] = inbox[k]
    return out, outbox


# ---- expert-parallel AllToAll (paper summary, "Experiments": AllToAll dispatch and combine measured against
#      DeepEP; complete guide, §4.2: low-latency AllToAll for expert parallelism) ----

def a2a_owner(e, E: int, W: int):
    """Rank that holds expert e: the E experts are split into W contiguous blocks of E / W."""
    return np.asarray(e) // (E // W)


def a2a_tokens(topk: np.ndarray, e: int) -> np.ndarray:
    """Ascending indices of the tokens (rows of topk) that picked expert e (a token counts once)."""
    topk = np.asarray(topk)
    return np.nonzero((topk == e).any(axis=1))[0].astype(np.int32)


def a2a_dispatch(X, topk, E: int, rank: int, before=None):
    """The dispatch as rank `rank` receives it.

    X: W arrays T_r x H (any dtype; rows are copied as bits); topk: W arrays T_r x k of expert ids (ids outside
    [0, E) select nothing).  For local expert l (global e = rank * E/W + l) and source p, slot i of block (l, p)
    holds X[p][tok_i], tok_0 < tok_1 < ... being the tokens of p that picked e.
    Returns (recv E_l x W x T_r x H, recv_token E_l x W x T_r, count E_l x W).  Slots past the count keep
    `before` (default zeros) and their token entries are -1.
    """
    W = len(X)
    E_l = E // W
    T_r, H = np.asarray(X[0]).shape
    recv = np.zeros((E_l, W, T_r, H), np.asarray(X[0]).dtype) if before is None else np.array(before, copy=True)
    tok = np.full((E_l, W, T_r), -1, np.int32)
    count = np.zeros((E_l, W), np.int64)
    for l in range(E_l):
        e = rank * E_l + l
        for p in range(W):
            ts = a2a_tokens(topk[p], e)
            n = len(ts)
            count[l, p] = n
            tok[l, p, :n] = ts
            recv[l, p, :n] = np.asarray(X[p])[ts]
    return recv, tok, count


def a2a_slots(topk: np.ndarray, E: int) -> np.ndarray:
    """slot[t, j]: the position of token t in expert topk[t, j]'s list of this rank's tokens, i.e. the number of
    tokens before t that picked that expert; -1 for ids outside [0, E)."""
    topk = np.asarray(topk)
    T_r, k = topk.shape
    slot = np.full((T_r, k), -1, np.int64)
    seen = np.zeros(E, np.int64)
    for t in range(T_r):
        picked = set()
        for j in range(k):
            e = int(topk[t, j])
            if 0 <= e < E:
                slot[t, j] = seen[e]
                picked.add(e)
        for e in picked:
            seen[e] += 1
    return slot


def a2a_combine_recv(back, topk, E: int, before=None):
    """What the combine's senders leave in this rank's receive buffer: for expert e (owner q, local index l),
    rows [0, n_e) of back[q][l] at cbuf[e], n_e = this rank's tokens that picked e.  back: W arrays
    E_l x T_r x H.  Rows past n_e keep `before` (default zeros)."""
    W = len(back)
    E_l = E // W
    _, T_r, H = np.asarray(back[0]).shape
    cbuf = np.zeros((E, T_r, H), np.asarray(back[0]).dtype) if before is None else np.array(before, copy=True)
    for e in range(E):
        n = len(a2a_tokens(topk, e))
        cbuf[e, :n] = np.asarray(back[e // E_l])[e % E_l, :n]
    return cbuf


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns to float64 (exact): a bf16 value is the upper half of the fp32 with the same bits."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def a2a_combine(back, topk, gate, E: int):
    """The combine on this rank: out[t] = sum over picks j of gate[t, j] * Y_e[slot(t, j)], e = topk[t, j],
    Y_e = back[owner(e)][e mod E/W] (bf16 bits), in float64, picks in order; ids outside [0, E) add nothing."""
    W = len(back)
    E_l = E // W
    topk = np.asarray(topk)
    gate = np.asarray(gate, np.float32)
    T_r, k = topk.shape
    H = np.asarray(back[0]).shape[2]
    slot = a2a_slots(topk, E)
    out = np.zeros((T_r, H), np.float64)
    for t in range(T_r):
        for j in range(k):
            e = int(topk[t, j])
            if not 0 <= e < E:
                continue
            y = _bf16_to_f64(np.asarray(back[e // E_l])[e % E_l, slot[t, j]])
            out[t] += np.float64(gate[t, j]) * y
    return out
