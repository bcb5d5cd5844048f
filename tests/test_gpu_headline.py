"""Parity of the benchmarked calls themselves, at their full shapes, on every output element.

* AllGather + GEMM at the Llama-3-70B MLP share (W 8, M 16384, K 8192, N 3584, B stored N x K), overlapped,
  8 K chunks per signal tile, 153.6 GB/s per simulated link with up to 27 us of jitter per tile: exactly the
  benchmark's headline call, for rank 0 and rank 5.  Every row of C against the fp64 oracle (Triton-distributed
  semantics page, "AllGather + GEMM overlap": C = AllGather(A) * B_local), and with integer-valued inputs bit for
  bit on every row.
* GEMM + ReduceScatter at the Qwen3-32B MLP share (M 8192, K 3200, N 5120, B stored N x K, 7 fp32 peer
  partials), peers resident and paced at 50 GB/s per link: every element of C_shard and of partial_out
  against the oracle (semantics page, "GEMM + ReduceScatter overlap").
"""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")

import signal_gated_tiled_amd as sgt  # noqa: E402
from signal_gated_tiled_amd import inputs as I  # noqa: E402
from gpu_util import TOL_BF16, assert_close, dev, host, poison_like  # noqa: E402

K_CHUNKS = 8   # the benchmark's setting


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = sgt.Context(0)
    yield c
    c.close()


_cache = {}


def _llama(orc, dist):
    """Inputs (B stored N x K) and the oracle's gathered A and C for every row; the oracle's result does not
    depend on the rank (a rank only changes the order of the work), so one computation serves both ranks."""
    if dist not in _cache:
        w = I.scaled(I.LLAMA_AG, dist=dist)
        shards, B = I.make_ag(w, B_layout="nk")
        A_ref, C_ref = orc.ag_gemm(shards, B, b_layout="nk")
        _cache[dist] = (w, shards, B, A_ref, C_ref)
    return _cache[dist]


def _headline_call(ctx, w, dA, dB, rank, seed):
    """The benchmark's overlapped step: producer on its own stream, K-chunked signal tiles, paced links."""
    Ag = poison_like(torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda:0"))
    C = poison_like(torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0"))
    flags = torch.zeros(sgt.ag_flag_count(w.W, w.M, w.K, k_chunks=K_CHUNKS), dtype=torch.int32, device="cuda:0")
    ctx.ag_gemm(dA, dB, Ag, C, flags, rank=rank, b_layout="nk", producer="cu", k_chunks=K_CHUNKS,
                peer_gbps=w.peer_gbps, jitter_us=w.jitter_us, arrival_seed=seed, blocking=True)
    torch.cuda.synchronize()
    return Ag, C, host(flags)


def _compare_all_rows(C_gpu: np.ndarray, C_ref: np.ndarray, exact: bool, what: str, block: int = 2048):
    """Every element, a block of rows at a time: bit-exact (integer inputs) or the bf16 tolerance
    (each element within 1e-2 (|ref| + 1), relative Frobenius over the whole matrix at most 2e-3)."""
    num = den = 0.0
    for r0 in range(0, C_ref.shape[0], block):
        g = C_gpu[r0:r0 + block].astype(np.float64)
        ref = C_ref[r0:r0 + block]
        assert np.isfinite(g).all(), "%s: non-finite values in rows %d.." % (what, r0)
        if exact:
            bad = g != ref
        else:
            bad = np.abs(g - ref) > TOL_BF16["max_coef"] * (np.abs(ref) + 1.0)
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError("%s: %d elements off in rows %d..%d, first at row %d col %d: gpu %r ref %r" %
                                 (what, int(bad.sum()), r0, r0 + block, r0 + i[0], i[1], g[tuple(i)], ref[tuple(i)]))
        num += float(np.sum((g - ref) ** 2))
        den += float(np.sum(ref ** 2))
    rf = (num / den) ** 0.5 if den > 0 else num ** 0.5
    assert rf <= TOL_BF16["rel_fro"], "%s: relative Frobenius %.3e" % (what, rf)
    return rf


@pytest.mark.parametrize("rank", [0, 5])
def test_headline_call_every_row(ctx, orc, rank):
    w, shards, B, A_ref, C_ref = _llama(orc, "normal")
    dA, dB = [dev(s) for s in shards], dev(B)
    Ag, C, fl = _headline_call(ctx, w, dA, dB, rank, seed=11 + rank)
    assert np.array_equal(host(Ag), A_ref), "gathered buffer"
    assert len(fl) == (w.M // 256) * K_CHUNKS and (fl == fl[0]).all() and fl[0] > 0, "flags hold the epoch"
    rf = _compare_all_rows(host(C), C_ref, exact=False, what="headline C rank %d" % rank)
    print("headline rank %d: relative Frobenius %.3e over %d x %d" % (rank, rf, w.M, w.N), flush=True)


@pytest.mark.parametrize("sdma", [dict(producer="sdma"), dict(producer="sdma", sdma_peers=3)],
                         ids=["engines", "engines+cu"])
def test_headline_call_copy_engines_every_row(ctx, orc, sdma):
    """The headline call with the copy-engine producer (all remote peers, or three of them with CU
    workgroups moving the other four): every row against the oracle."""
    w, shards, B, A_ref, C_ref = _llama(orc, "normal")
    dA, dB = [dev(s) for s in shards], dev(B)
    Ag = poison_like(torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda:0"))
    C = poison_like(torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0"))
    flags = torch.zeros(sgt.ag_flag_count(w.W, w.M, w.K, k_chunks=K_CHUNKS), dtype=torch.int32, device="cuda:0")
    ctx.ag_gemm(dA, dB, Ag, C, flags, rank=2, b_layout="nk", k_chunks=K_CHUNKS, peer_gbps=w.peer_gbps,
                jitter_us=w.jitter_us, arrival_seed=31, blocking=True, **sdma)
    torch.cuda.synchronize()
    assert np.array_equal(host(Ag), A_ref), "gathered buffer"
    _compare_all_rows(host(C), C_ref, exact=False, what="headline C, copy engines")


@pytest.mark.parametrize("rank", [0, 5])
def test_headline_call_integer_inputs_bit_exact(ctx, orc, rank):
    """Inputs in [-3, 3] are exact in bf16 and every partial sum is an integer below 2^24, so fp32
    accumulation is exact in any order: C must equal the oracle bit for bit on every row."""
    w, shards, B, A_ref, C_ref = _llama(orc, "int")
    dA, dB = [dev(s) for s in shards], dev(B)
    Ag, C, _ = _headline_call(ctx, w, dA, dB, rank, seed=21 + rank)
    assert np.array_equal(host(Ag), A_ref), "gathered buffer"
    _compare_all_rows(host(C), C_ref, exact=True, what="headline integer C rank %d" % rank)


# ---------------------------------------------------------------- GEMM + ReduceScatter, full shape, N x K

_rs_cache = {}


def _rs(orc):
    if "rs" not in _rs_cache:
        w = I.GEMM_RS
        A, B, parts = I.make_rs(w, B_layout="nk")
        P_ref = orc.gemm(A, B, b_layout="nk")
        _rs_cache["rs"] = (w, A, B, parts, P_ref)
    return _rs_cache["rs"]


@pytest.mark.parametrize("mode", ["resident", "paced_50gbps"])
@pytest.mark.parametrize("rank", [3, 6])
def test_gemm_rs_full_shape_every_element(ctx, orc, mode, rank):
    w, A, B, parts, P_ref = _rs(orc)
    ng, npf = sgt.rs_flag_count(w.W, w.M, w.N)
    P = poison_like(torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0"))
    Cs = poison_like(torch.empty((w.M // w.W, w.N), dtype=torch.float32, device="cuda:0"))
    gf = torch.zeros(ng, dtype=torch.int32, device="cuda:0")
    pf = torch.zeros(npf, dtype=torch.int32, device="cuda:0")
    dparts = [dev(p) if q != rank else None for q, p in enumerate(parts)]
    if mode == "resident":
        ctx.gemm_rs(dev(A), dev(B), dparts, P, Cs, gf, pf, rank=rank, b_layout="nk", blocking=True)
    else:
        inbox = [poison_like(torch.empty_like(p)) if p is not None else None for p in dparts]
        ctx.gemm_rs_paced(dev(A), dev(B), dparts, inbox, P, Cs, gf, pf, rank=rank, b_layout="nk", peer_gbps=50.0,
                          arrival_seed=rank, blocking=True)
        for q in range(w.W):
            if q != rank:
                assert torch.equal(inbox[q].view(torch.int32), dparts[q].view(torch.int32)), "inbox %d" % q
    torch.cuda.synchronize()
    _compare_all_rows(host(P), P_ref, exact=False, what="partial_out (%s)" % mode)
    assert_close(host(Cs), orc.gemm_rs(A, B, parts, rank, b_layout="nk"), what="C_shard (%s)" % mode, **TOL_BF16)
    g, p = host(gf), host(pf)
    assert (g == g[0]).all() and g[0] != 0
    nb = len(p) // w.W
    for q in range(w.W):
        if q != rank:
            assert (p[q * nb:(q + 1) * nb] == g[0]).all(), "peer %d flags" % q
