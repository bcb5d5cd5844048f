"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no gather, no product, no reduction, no routing).  Both the
HIP path and the CPU oracle receive the arrays built here.

Conventions
-----------
* bf16 tensors are carried as ``numpy.uint16`` arrays holding the bf16 bit
  patterns; fp32 tensors as ``numpy.float32``.
* A bf16 value "~N(0, s)" is an fp32 draw from numpy's PCG64 normal generator,
  scaled by ``s`` and rounded to bf16 with round-to-nearest-even.
* Each workload uses ``SeedSequence(1000 + index)`` and spawns one child stream
  per tensor in a fixed order, so a tensor never depends on the sizes of the
  tensors drawn before it.

The workloads mirror the shapes of the tensor-parallel MLP layers that the
Triton-distributed pages benchmark (Qwen3-32B and Llama-3-70B MLPs, and a MoE
layer): one GPU's share of each layer, with the peer shards held locally.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# bit patterns used to poison buffers that a kernel must overwrite
POISON_BF16 = np.uint16(0x7FC0)        # bf16 quiet NaN
POISON_F32 = np.uint32(0x7FC00000)     # fp32 quiet NaN


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def normal_bf16(ss, shape, std: float) -> np.ndarray:
    g = _rng(ss)
    return f32_to_bf16_bits(g.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def normal_f32(ss, shape, std: float = 1.0) -> np.ndarray:
    g = _rng(ss)
    return g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)


def uniform_f32(ss, shape, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    g = _rng(ss)
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def small_int(ss, shape, lo: int = -3, hi: int = 3, dtype: str = "bf16") -> np.ndarray:
    """Integer values in [lo, hi]; exact in bf16 and fp32."""
    g = _rng(ss)
    v = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def _draw(kind: str, ss, shape, dtype: str, std: float):
    if kind == "int":
        return small_int(ss, shape, dtype=dtype)
    if dtype == "f32":
        return uniform_f32(ss, shape) if kind == "uniform" else normal_f32(ss, shape, std)
    return normal_bf16(ss, shape, std)


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class AGWorkload:
    """C = AllGather_rows(A shards) @ B_local, one GPU's share."""
    name: str
    W: int
    M: int
    K: int
    N: int
    dtype: str = "bf16"          # input dtype: "bf16" or "f32"
    dist: str = "normal"         # "normal" (std), "uniform" [-1,1], "int" {-3..3}
    std: float = 0.02
    peer_gbps: float = 0.0       # simulated per-peer link rate; 0 = unthrottled
    jitter_us: float = 0.0
    flag_rows: int = 0           # rows per signal tile; 0 = library default
    seed_index: int = 0

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


@dataclasses.dataclass(frozen=True)
class RSWorkload:
    """C_shard = (A_local @ B)[block r] + sum of peer partial blocks."""
    name: str
    W: int
    M: int
    K: int
    N: int
    dtype: str = "bf16"
    dist: str = "normal"
    std: float = 0.02
    peer_dist: str = "normal"    # "normal" N(0,1) fp32, "int", "zero"
    seed_index: int = 2

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


@dataclasses.dataclass(frozen=True)
class MoEWorkload:
    """Y = X_gathered[rows grouped by expert] @ W_e (up-projection side)."""
    name: str
    W: int
    T: int
    H: int
    I: int
    E: int
    topk: int
    std: float = 0.02
    zipf_alpha: float = 1.0
    dist: str = "normal"
    peer_gbps: float = 0.0
    seed_index: int = 4

    @property
    def flops(self) -> float:
        return 2.0 * self.T * self.topk * self.H * self.I


@dataclasses.dataclass(frozen=True)
class MoERSWorkload:
    """Combine side of the MoE layer: P[t] = sum_j gate[t, j] * Hg[row(t, j)] @ W2_e, then ReduceScatter."""
    name: str
    W: int
    T: int
    I: int      # input width of the down projection (the up projection's output)
    H: int      # output width (hidden)
    E: int
    topk: int
    std: float = 0.02
    zipf_alpha: float = 1.0
    dist: str = "normal"
    peer_dist: str = "normal"
    seed_index: int = 5

    @property
    def flops(self) -> float:
        return 2.0 * self.T * self.topk * self.I * self.H


@dataclasses.dataclass(frozen=True)
class RingWorkload:
    """Ring AllReduce of W ranks' fp32 vectors of N elements, one rank's share."""
    name: str
    W: int
    N: int
    peer_gbps: float = 0.0      # the left neighbour's link; 0 = unthrottled
    jitter_us: float = 0.0
    dist: str = "normal"        # "normal" N(0,1) or "int" {-8..8}
    seed_index: int = 7

    @property
    def bytes_per_rank(self) -> int:
        return 4 * self.N


@dataclasses.dataclass(frozen=True)
class A2AWorkload:
    """Expert-parallel AllToAll of one MoE layer, one rank's share: the dispatch of every rank's tokens to the
    owners of the experts they picked, and the combine of the expert outputs back into this rank's tokens."""
    name: str
    W: int
    T: int          # tokens over all ranks (T / W per rank)
    H: int
    E: int
    topk: int
    std: float = 0.02
    zipf_alpha: float = 1.0
    peer_gbps: float = 0.0
    chunk_rows: int = 32
    seed_index: int = 8

    @property
    def tokens_per_rank(self) -> int:
        return self.T // self.W


# The five workloads (index = seed offset).  Shapes follow the pages' model
# shapes: Qwen3-32B MLP (hidden 5120, intermediate 25600), Llama-3-70B MLP
# (hidden 8192, intermediate 28672), each split 8 ways.
TINY = AGWorkload("ag_tiny_f32_w4", W=4, M=256, K=256, N=128, dtype="f32", dist="uniform",
                  flag_rows=16, jitter_us=50.0, seed_index=0)
QWEN_AG = AGWorkload("ag_qwen32b_mlp_w8", W=8, M=8192, K=5120, N=3200, peer_gbps=50.0, seed_index=1)
GEMM_RS = RSWorkload("gemm_rs_qwen32b_mlp_w8", W=8, M=8192, K=3200, N=5120, seed_index=2)
LLAMA_AG = AGWorkload("ag_llama3_70b_mlp_w8", W=8, M=16384, K=8192, N=3584, peer_gbps=153.6,
                      jitter_us=27.0, seed_index=3)
MOE = MoEWorkload("moe_ag_grouped_w8", W=8, T=4096, H=2048, I=768, E=64, topk=8, peer_gbps=50.0,
                  seed_index=4)

# The down projection of the same MoE layer (the next workload on the pages' list).
MOE_RS = MoERSWorkload("moe_gemm_rs_w8", W=8, T=4096, I=768, H=2048, E=64, topk=8, seed_index=5)

# The ring AllReduce of the pages' second example at the Llama-3-70B row-parallel output of 2048 tokens
# (2048 x 8192 fp32 per rank), over the 153.6 GB/s link from the left neighbour.
RING = RingWorkload("ring_allreduce_llama3_70b_w8", W=8, N=2048 * 8192, peer_gbps=153.6, seed_index=7)

# The AllToAll dispatch and combine of the same MoE layer with expert parallelism over the 8 ranks (8 experts
# per rank), links at 50 GB/s per peer.
A2A = A2AWorkload("a2a_moe_ep8", W=8, T=4096, H=2048, E=64, topk=8, peer_gbps=50.0, seed_index=8)

WORKLOADS = {w.name: w for w in (TINY, QWEN_AG, GEMM_RS, LLAMA_AG, MOE, MOE_RS, RING, A2A)}


def _streams(seed_index: int, n: int, salt: int = 0):
    return np.random.SeedSequence(1000 + seed_index, spawn_key=(salt,)).spawn(n) if salt else \
        np.random.SeedSequence(1000 + seed_index).spawn(n)


def make_ag(w: AGWorkload, salt: int = 0, B_layout: str = "kn"):
    """Return (shards, B) for an AG workload.

    shards: list of W arrays, each (M/W) x K.  B: K x N ("kn") or N x K ("nk",
    the same matrix stored transposed, as a Linear layer's weight).
    """
    assert w.M % w.W == 0
    ss = _streams(w.seed_index, w.W + 1, salt)
    rows = w.M // w.W
    shards = [_draw(w.dist, ss[p], (rows, w.K), w.dtype, w.std) for p in range(w.W)]
    B = _draw(w.dist, ss[w.W], (w.K, w.N), w.dtype, w.std)
    if B_layout == "nk":
        B = np.ascontiguousarray(B.T)
    return shards, B


def make_rs(w: RSWorkload, salt: int = 0, B_layout: str = "kn"):
    """Return (A_local, B, partials) for a GEMM-RS workload.

    partials: list of W fp32 arrays of (M/W) x N (the peers' contributions to
    this rank's row block); the entry at the local rank is never read.
    """
    assert w.M % w.W == 0
    ss = _streams(w.seed_index, 2 + w.W, salt)
    A = _draw(w.dist, ss[0], (w.M, w.K), w.dtype, w.std)
    B = _draw(w.dist, ss[1], (w.K, w.N), w.dtype, w.std)
    mb = w.M // w.W
    partials = []
    for p in range(w.W):
        if w.peer_dist == "zero":
            partials.append(np.zeros((mb, w.N), np.float32))
        elif w.peer_dist == "int":
            partials.append(small_int(ss[2 + p], (mb, w.N), -8, 8, dtype="f32"))
        else:
            partials.append(normal_f32(ss[2 + p], (mb, w.N), 1.0))
    if B_layout == "nk":
        B = np.ascontiguousarray(B.T)
    return A, B, partials


def make_moe(w: MoEWorkload, salt: int = 0, W_layout: str = "kn"):
    """Return (X shards, W_experts, logits).

    logits[t, e] = g[t, e] + beta[e], g ~ N(0, 1) and beta[e] = -alpha * ln(1 + pi(e))
    for a seeded permutation pi: a Zipf-like skew of expert popularity.
    W_experts: E x H x I ("kn") or E x I x H ("nk").
    """
    assert w.T % w.W == 0
    ss = _streams(w.seed_index, w.W + 3, salt)
    rows = w.T // w.W
    shards = [_draw(w.dist, ss[p], (rows, w.H), "bf16", w.std) for p in range(w.W)]
    We = _draw(w.dist, ss[w.W], (w.E, w.H, w.I), "bf16", w.std)
    g = _rng(ss[w.W + 1]).standard_normal(size=(w.T, w.E), dtype=np.float32)
    perm = _rng(ss[w.W + 2]).permutation(w.E)
    beta = (-w.zipf_alpha * np.log1p(perm.astype(np.float64))).astype(np.float32)
    logits = (g + beta[None, :]).astype(np.float32)
    if W_layout == "nk":
        We = np.ascontiguousarray(np.transpose(We, (0, 2, 1)))
    return shards, We, logits


def make_moe_rs(w: MoERSWorkload, salt: int = 0, W_layout: str = "kn"):
    """Return (Hg, W2, gate, logits, partials).

    Hg: (T * topk) x I bf16, the grouped rows (row r belongs to whatever (expert, token) the routing of
    `logits` puts at r).  W2: E x I x H ("kn") or E x H x I ("nk") bf16.  gate: T x topk float32 in (0, 1),
    one weight per pick.  logits: as in make_moe.  partials: W arrays of (T/W) x H float32.
    """
    assert w.T % w.W == 0
    ss = _streams(w.seed_index, 5 + w.W, salt)
    Hg = _draw(w.dist, ss[0], (w.T * w.topk, w.I), "bf16", w.std * 50 if w.dist == "normal" else w.std)
    W2 = _draw(w.dist, ss[1], (w.E, w.I, w.H), "bf16", w.std)
    gate = _rng(ss[2]).random(size=(w.T, w.topk), dtype=np.float32)
    g = _rng(ss[3]).standard_normal(size=(w.T, w.E), dtype=np.float32)
    perm = _rng(ss[4]).permutation(w.E)
    beta = (-w.zipf_alpha * np.log1p(perm.astype(np.float64))).astype(np.float32)
    logits = (g + beta[None, :]).astype(np.float32)
    mb = w.T // w.W
    partials = []
    for p in range(w.W):
        if w.peer_dist == "zero":
            partials.append(np.zeros((mb, w.H), np.float32))
        elif w.peer_dist == "int":
            partials.append(small_int(ss[5 + p], (mb, w.H), -8, 8, dtype="f32"))
        else:
            partials.append(normal_f32(ss[5 + p], (mb, w.H), 1.0))
    if W_layout == "nk":
        W2 = np.ascontiguousarray(np.transpose(W2, (0, 2, 1)))
    return Hg, W2, gate, logits, partials


def make_ring(w: RingWorkload, salt: int = 0):
    """Return the W ranks' vectors (fp32, N each)."""
    assert w.N % w.W == 0
    ss = _streams(w.seed_index, w.W, salt)
    if w.dist == "int":
        return [small_int(ss[p], (w.N,), -8, 8, dtype="f32") for p in range(w.W)]
    return [normal_f32(ss[p], (w.N,), 1.0) for p in range(w.W)]


def make_ring_messages(w: RingWorkload, salt: int = 0):
    """Stand-ins for the left neighbour's 2(W-1) messages of N / W floats each, N(0,1) (the timed
    work does not depend on their values; parity tests build consistent ones with the oracle)."""
    ss = _streams(w.seed_index, 1, salt + 1000)
    return normal_f32(ss[0], (2 * (w.W - 1), w.N // w.W), 1.0)


def make_a2a(w: A2AWorkload, salt: int = 0):
    """Return (X, logits, gate, back).

    X: W arrays of (T/W) x H bf16 ~N(0, std), the ranks' tokens.  logits: T x E float32, as in make_moe (Gaussian
    plus a seeded Zipf-like popularity skew); rank p's tokens are rows [p*T/W, (p+1)*T/W).  gate: T x topk float32
    in (0, 1), one weight per pick.  back: W arrays of (E/W) x (T/W) x H bf16 ~N(0, 1), stand-ins for the expert
    outputs that each expert owner sends back to this rank (slot i of expert l: this rank's i-th token routed to
    it; only the first count rows are ever read).
    """
    assert w.T % w.W == 0 and w.E % w.W == 0
    ss = _streams(w.seed_index, 2 * w.W + 3, salt)
    T_r, E_l = w.T // w.W, w.E // w.W
    X = [normal_bf16(ss[p], (T_r, w.H), w.std) for p in range(w.W)]
    g = _rng(ss[w.W]).standard_normal(size=(w.T, w.E), dtype=np.float32)
    perm = _rng(ss[w.W + 1]).permutation(w.E)
    beta = (-w.zipf_alpha * np.log1p(perm.astype(np.float64))).astype(np.float32)
    logits = (g + beta[None, :]).astype(np.float32)
    gate = _rng(ss[w.W + 2]).random(size=(w.T, w.topk), dtype=np.float32)
    back = [normal_bf16(ss[w.W + 3 + q], (E_l, T_r, w.H), 1.0) for q in range(w.W)]
    return X, logits, gate, back


def scaled(w, **kw):
    """A copy of a workload with some fields replaced (used for reduced test sizes)."""
    return dataclasses.replace(w, **kw)


def gb(nbytes: float) -> float:
    return nbytes / 1e9


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("dataclasses", "math", "np", "annotations")]
