"""ctypes binding of libsgt (include/sgt.h): argument marshalling only.

Every computation happens in the HIP library; this module checks tensor
devices, dtypes and contiguity, passes raw device pointers, sizes and options
through the C ABI, and turns status codes into exceptions.  PyTorch provides
device memory and streams.  If ``libsgt.so`` is missing the calls raise; there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsgt.so")

SGT_OK, SGT_EINVAL, SGT_EUNSUPPORTED, SGT_ETIMEDOUT, SGT_EHIP, SGT_ENOMEM = 0, -1, -2, -3, -4, -5
SGT_F32, SGT_BF16 = 0, 1
SGT_KN, SGT_NK = 0, 1
PRODUCERS = {"cu": 0, "preset": 1, "serial": 2, "sdma": 3}
ORDERS = {"mesh": 0, "shard": 1}
LAYOUTS = {"kn": SGT_KN, "nk": SGT_NK}
ARRIVALS = {"inorder": 0, "per_peer": 1, "global": 2}


class SgtError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), msg))
        self.status = status


_STATUS = {0: "SGT_OK", -1: "SGT_EINVAL", -2: "SGT_EUNSUPPORTED", -3: "SGT_ETIMEDOUT", -4: "SGT_EHIP",
           -5: "SGT_ENOMEM"}


class Opts(ctypes.Structure):
    """Mirror of ``sgt_opts``."""
    _fields_ = [
        ("rank", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("b_layout", ctypes.c_int32), ("producer", ctypes.c_int32), ("order", ctypes.c_int32),
        ("flag_rows", ctypes.c_int32), ("producer_cus", ctypes.c_int32), ("consumer_cus", ctypes.c_int32),
        ("blocking", ctypes.c_int32), ("peer_gbps", ctypes.c_double), ("jitter_us", ctypes.c_double),
        ("timeout_ms", ctypes.c_double), ("arrival_seed", ctypes.c_uint64), ("withhold_peer", ctypes.c_int32),
        ("rs_tile", ctypes.c_int32), ("arrival_order", ctypes.c_int32), ("tile_waves", ctypes.c_int32),
        ("tile_rows", ctypes.c_int32), ("k_chunks", ctypes.c_int32), ("sdma_peers", ctypes.c_int32),
        ("trace", ctypes.c_void_p), ("consumer_events", ctypes.c_void_p * 2),
    ]


_lib = None
P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64


def lib() -> ctypes.CDLL:
    """Load libsgt.so (built in-tree by ``python -m signal_gated_tiled_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsgt.so is not built (%s); run `python -m signal_gated_tiled_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.sgt_version.restype = ctypes.c_char_p
        L.sgt_status_str.restype = ctypes.c_char_p
        L.sgt_status_str.argtypes = [ctypes.c_int]
        L.sgt_last_error.restype = ctypes.c_char_p
        L.sgt_opts_init.argtypes = [ctypes.POINTER(Opts)]
        L.sgt_ctx_create.argtypes = [ctypes.POINTER(P), ctypes.c_int]
        L.sgt_ctx_destroy.argtypes = [P]
        L.sgt_sync.argtypes = [P]
        L.sgt_ag_flag_count.argtypes = [ctypes.c_int, I64, I64, ctypes.POINTER(Opts)]
        L.sgt_ag_flag_count.restype = I64
        L.sgt_ag_panel_rows.argtypes = [ctypes.c_int, I64, I64, I64, ctypes.POINTER(Opts)]
        L.sgt_ag_panel_rows.restype = I32
        L.sgt_panel_order.argtypes = [ctypes.c_int, ctypes.c_int, I64, I32, ctypes.c_int, P, I64]
        L.sgt_panel_order.restype = I64
        L.sgt_trace_words.argtypes = [ctypes.c_int, I64, I64, I64, ctypes.POINTER(Opts)]
        L.sgt_trace_words.restype = I64
        L.sgt_moe_trace_words.argtypes = [ctypes.c_int, I64, I64, I64, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(Opts)]
        L.sgt_moe_trace_words.restype = I64
        L.sgt_ag_gemm.argtypes = [P, P, P, P, P, P, ctypes.c_int, I64, I64, I64, ctypes.POINTER(Opts), P]
        L.sgt_rs_flag_count.argtypes = [ctypes.c_int, I64, I64, ctypes.POINTER(Opts), ctypes.POINTER(I64),
                                        ctypes.POINTER(I64)]
        L.sgt_gemm_rs.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, I64, I64, I64, ctypes.POINTER(Opts), P]
        L.sgt_gemm_rs_paced.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_int, I64, I64, I64,
                                        ctypes.POINTER(Opts), P]
        L.sgt_moe_gemm_rs.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int, I64, ctypes.c_int, I64,
                                      I64, ctypes.c_int, ctypes.POINTER(Opts), P]
        L.sgt_moe_gemm_rs_paced.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int, I64,
                                            ctypes.c_int, I64, I64, ctypes.c_int, ctypes.POINTER(Opts), P]
        L.sgt_moe_ag_gemm.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_int, I64, I64, I64, ctypes.c_int,
                                      ctypes.c_int, ctypes.POINTER(Opts), P]
        L.sgt_allgather.argtypes = [P, P, P, P, ctypes.c_int, I64, I64, ctypes.POINTER(Opts), P]
        L.sgt_ll_allgather.argtypes = [P, P, P, P, ctypes.c_int, I64, I64, ctypes.POINTER(Opts), P]
        L.sgt_ll_buffer_bytes.argtypes = [ctypes.c_int, I64, I64, ctypes.POINTER(Opts)]
        L.sgt_ll_buffer_bytes.restype = I64
        L.sgt_ring_allreduce.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, I64, ctypes.POINTER(Opts), P]
        L.sgt_ring_flag_count.argtypes = [ctypes.c_int, I64, ctypes.POINTER(I64)]
        L.sgt_ring_flag_count.restype = I64
        L.sgt_a2a_dispatch.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, I64, I64, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(Opts), P]
        L.sgt_a2a_combine.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, I64, I64, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(Opts), P]
        L.sgt_a2a_flag_count.argtypes = [ctypes.c_int, I64, ctypes.c_int, ctypes.POINTER(Opts)]
        L.sgt_a2a_flag_count.restype = I64
        L.sgt_rs_trace_words.argtypes = [ctypes.c_int, I64, I64, ctypes.POINTER(Opts)]
        L.sgt_rs_trace_words.restype = I64
        L.sgt_gemm_rs_static.argtypes = [P, P, P, P, P, ctypes.c_int, I64, I64, I64, ctypes.POINTER(Opts), P]
        L.sgt_gemm_rs_static_scratch_bytes.argtypes = []
        L.sgt_gemm_rs_static_scratch_bytes.restype = I64
        for f in ("sgt_ctx_create", "sgt_ctx_destroy", "sgt_sync", "sgt_ag_gemm", "sgt_rs_flag_count", "sgt_gemm_rs",
                  "sgt_gemm_rs_paced", "sgt_moe_ag_gemm", "sgt_moe_gemm_rs",
                  "sgt_moe_gemm_rs_paced", "sgt_allgather", "sgt_ll_allgather", "sgt_ring_allreduce",
                  "sgt_a2a_dispatch", "sgt_a2a_combine", "sgt_gemm_rs_static"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def version() -> str:
    return lib().sgt_version().decode()


def _check(status: int):
    if status != SGT_OK:
        raise SgtError(status, lib().sgt_last_error().decode())


def make_opts(rank: int = 0, in_dtype: int = SGT_BF16, out_dtype: int = SGT_F32, b_layout: str = "kn",
              producer: str = "cu", order: str = "mesh", flag_rows: int = 0, producer_cus: int = 0,
              consumer_cus: int = 0, blocking: bool = False, peer_gbps: float = 0.0, jitter_us: float = 0.0,
              timeout_ms: float = 2000.0, arrival_seed: int = 0, withhold_peer: int = -1, rs_tile: int = 0,
              trace: int = 0, consumer_events=None, arrival_order: str = "inorder", tile_waves: int = 0,
              tile_rows: int = 0, k_chunks: int = 0, sdma_peers: int = 0) -> Opts:
    o = Opts()
    lib().sgt_opts_init(ctypes.byref(o))
    o.rank, o.in_dtype, o.out_dtype = rank, in_dtype, out_dtype
    o.b_layout = LAYOUTS[b_layout]
    o.producer = PRODUCERS[producer]
    o.order = ORDERS[order]
    o.flag_rows, o.producer_cus, o.consumer_cus = flag_rows, producer_cus, consumer_cus
    o.blocking = 1 if blocking else 0
    o.peer_gbps, o.jitter_us, o.timeout_ms = float(peer_gbps), float(jitter_us), float(timeout_ms)
    o.arrival_seed = int(arrival_seed)
    o.withhold_peer = withhold_peer
    o.rs_tile = rs_tile
    o.arrival_order = ARRIVALS[arrival_order]
    o.tile_waves = tile_waves
    o.tile_rows = tile_rows
    o.k_chunks = k_chunks
    o.sdma_peers = sdma_peers
    o.trace = trace or None
    if consumer_events is not None:
        o.consumer_events[0] = _event_handle(consumer_events[0])
        o.consumer_events[1] = _event_handle(consumer_events[1])
    return o


def _event_handle(ev) -> int:
    """Raw hipEvent_t of a torch.cuda.Event, or an int handle.

    A torch event is recorded once here (so torch creates it and accepts it in
    elapsed_time); the library records it again at the consumer launch.
    """
    if isinstance(ev, int):
        return ev
    ev.record()
    return int(ev.cuda_event)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SGT_BF16
    if t.dtype == torch.float32:
        return SGT_F32
    raise TypeError("tensors must be bfloat16 or float32, got %s" % t.dtype)


def _dev_ptr(t, name: str, device=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    return t.data_ptr()


def _stream_handle(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def ag_flag_count(W: int, M: int, K: int, **kw) -> int:
    o = make_opts(**kw)
    n = lib().sgt_ag_flag_count(W, M, K, ctypes.byref(o))
    if n < 0:
        _check(int(n))
    return int(n)


def ag_panel_rows(W: int, M: int, K: int, N: int, **kw) -> int:
    o = make_opts(**kw)
    return int(lib().sgt_ag_panel_rows(W, M, K, N, ctypes.byref(o)))


def panel_order(W: int, rank: int, M: int, panel_rows: int, order: str = "mesh"):
    n = -(-M // panel_rows)
    buf = (ctypes.c_int32 * max(n, 1))()
    r = lib().sgt_panel_order(W, rank, M, panel_rows, ORDERS[order], ctypes.cast(buf, P), n)
    if r < 0:
        _check(int(r))
    return [int(buf[i]) for i in range(int(r))]


def trace_words(W: int, M: int, K: int, N: int, **kw) -> int:
    o = make_opts(**kw)
    n = lib().sgt_trace_words(W, M, K, N, ctypes.byref(o))
    if n < 0:
        _check(int(n))
    return int(n)


def moe_trace_words(W: int, T: int, H: int, I: int, E: int, topk: int, **kw) -> int:
    o = make_opts(**kw)
    n = lib().sgt_moe_trace_words(W, T, H, I, E, topk, ctypes.byref(o))
    if n < 0:
        _check(int(n))
    return int(n)


def ll_buffer_bytes(W: int, M: int, K: int, **kw) -> int:
    """Bytes of the LL receive buffer of an ll_allgather call (twice the gathered bytes)."""
    o = make_opts(**kw)
    n = lib().sgt_ll_buffer_bytes(W, M, K, ctypes.byref(o))
    if n < 0:
        raise SgtError(SGT_EINVAL, "invalid LL AllGather shape or options")
    return int(n)


def ring_flag_count(W: int, N: int):
    """(flag words, tile elements) of a ring AllReduce of N fp32 elements over W ranks."""
    t = I64()
    n = lib().sgt_ring_flag_count(W, N, ctypes.byref(t))
    if n < 0:
        raise SgtError(SGT_EINVAL, "invalid ring AllReduce shape (N a multiple of W, N / W a multiple of 4)")
    return int(n), int(t.value)


def a2a_flag_count(W: int, T_r: int, E: int, **kw) -> int:
    """Flag words of an AllToAll dispatch or combine (E x ceil(T_r / chunk rows))."""
    o = make_opts(**kw)
    n = lib().sgt_a2a_flag_count(W, T_r, E, ctypes.byref(o))
    if n < 0:
        raise SgtError(SGT_EINVAL, "invalid AllToAll shape or options")
    return int(n)


def rs_trace_words(W: int, M: int, N: int, rs_tile: int = 0) -> int:
    """Words (uint64) of the optional trace buffer of a GEMM+ReduceScatter call."""
    o = make_opts(rs_tile=rs_tile)
    n = lib().sgt_rs_trace_words(W, M, N, ctypes.byref(o))
    if n < 0:
        raise SgtError(SGT_EINVAL, "invalid GEMM+ReduceScatter shape")
    return int(n)


def rs_flag_count(W: int, M: int, N: int, rs_tile: int = 0):
    o = make_opts(rs_tile=rs_tile)
    g, p = I64(), I64()
    _check(lib().sgt_rs_flag_count(W, M, N, ctypes.byref(o), ctypes.byref(g), ctypes.byref(p)))
    return int(g.value), int(p.value)


def gemm_rs_static(A_local, B, partials: Sequence, partial_out, C_shard, *, stream=None, **kw):
    """sgt_gemm_rs_static: GEMM + ReduceScatter with resident peers and no allocation (flags, counter and
    status in the library's per-device static scratch; no context).  Runs on the tensors' device, which must
    be the current one."""
    import torch
    dev = B.device
    if torch.cuda.current_device() != dev.index:
        raise ValueError("gemm_rs_static runs on the current device (%d); the tensors are on %s" %
                         (torch.cuda.current_device(), dev))
    W = len(partials)
    M, K = A_local.shape
    lay = kw.get("b_layout", "kn")
    N = B.shape[1] if lay == "kn" else B.shape[0]
    kw.setdefault("in_dtype", _dtype_code(B))
    o = make_opts(**kw)
    ptrs = (P * W)(*[_dev_ptr(p, "partials[%d]" % i, dev) if p is not None else 0 for i, p in enumerate(partials)])
    _check(lib().sgt_gemm_rs_static(_dev_ptr(A_local, "A_local", dev), _dev_ptr(B, "B", dev), ctypes.cast(ptrs, P),
                                    _dev_ptr(partial_out, "partial_out", dev), _dev_ptr(C_shard, "C_shard", dev), W,
                                    M, K, N, ctypes.byref(o), _stream_handle(stream)))


def gemm_rs_static_scratch_bytes() -> int:
    return int(lib().sgt_gemm_rs_static_scratch_bytes())


class Context:
    """An sgt context on one device (its epoch counter, producer stream, status word)."""

    def __init__(self, device: int = 0):
        self._h = P()
        self.device = device
        _check(lib().sgt_ctx_create(ctypes.byref(self._h), device))

    def close(self):
        if self._h:
            _check(lib().sgt_ctx_destroy(self._h))
            self._h = P()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sync(self):
        """Wait for the context's work; raises SgtError(SGT_ETIMEDOUT) after an expired wait."""
        _check(lib().sgt_sync(self._h))

    def ag_gemm(self, A_shards: Sequence, B, A_gathered, C, flags, *, stream=None, **kw):
        """AllGather + GEMM: A_gathered = stack(A_shards); C = A_gathered @ B (B is K x N, or N x K
        with b_layout='nk').  Options as in sgt_opts (rank, producer, order, peer_gbps, ...)."""
        dev = B.device
        W = len(A_shards)
        M = A_gathered.shape[0]
        K = A_gathered.shape[1]
        lay = kw.get("b_layout", "kn")
        N = B.shape[1] if lay == "kn" else B.shape[0]
        kw.setdefault("in_dtype", _dtype_code(B))
        if "out_dtype" not in kw:
            kw["out_dtype"] = _dtype_code(C) if C is not None else SGT_F32
        o = make_opts(**kw)
        ptrs = (P * W)(*[_dev_ptr(a, "A_shards[%d]" % i, dev) for i, a in enumerate(A_shards)])
        _check(lib().sgt_ag_gemm(self._h, ctypes.cast(ptrs, P), _dev_ptr(B, "B", dev),
                                 _dev_ptr(A_gathered, "A_gathered", dev), _dev_ptr(C, "C", dev),
                                 _dev_ptr(flags, "flags", dev), W, M, K, N, ctypes.byref(o), _stream_handle(stream)))

    def allgather(self, shards: Sequence, gathered, flags, *, stream=None, **kw):
        """Flag-based AllGather: gathered = stack(shards); one flag per chunk of flag_rows rows
        (ag_flag_count with the same options).  Options as in sgt_opts."""
        dev = gathered.device
        W = len(shards)
        M, K = gathered.shape[0], gathered.shape[1]
        kw.setdefault("in_dtype", _dtype_code(gathered))
        o = make_opts(**kw)
        ptrs = (P * W)(*[_dev_ptr(a, "shards[%d]" % i, dev) for i, a in enumerate(shards)])
        _check(lib().sgt_allgather(self._h, ctypes.cast(ptrs, P), _dev_ptr(gathered, "gathered", dev),
                                   _dev_ptr(flags, "flags", dev), W, M, K, ctypes.byref(o), _stream_handle(stream)))

    def ll_allgather(self, shards: Sequence, ll_buf, gathered, *, stream=None, **kw):
        """Low-latency AllGather: the peers' chunks arrive as 8-byte {payload, epoch} packets in
        ll_buf (ll_buffer_bytes bytes, zeroed once); gathered = stack(shards)."""
        dev = gathered.device
        W = len(shards)
        M, K = gathered.shape[0], gathered.shape[1]
        kw.setdefault("in_dtype", _dtype_code(gathered))
        o = make_opts(**kw)
        ptrs = (P * W)(*[_dev_ptr(a, "shards[%d]" % i, dev) for i, a in enumerate(shards)])
        _check(lib().sgt_ll_allgather(self._h, ctypes.cast(ptrs, P), _dev_ptr(ll_buf, "ll_buf", dev),
                                      _dev_ptr(gathered, "gathered", dev), W, M, K, ctypes.byref(o),
                                      _stream_handle(stream)))

    def ring_allreduce(self, x, left_msgs, inbox, outbox, out, flags, W: int, *, stream=None, **kw):
        """One rank's share of a ring AllReduce: out = sum over ranks (fp32).  left_msgs / inbox /
        outbox: 2(W-1) messages of N / W floats; flags: ring_flag_count(W, N)[0] words.  left_msgs
        may be None with producer='preset' (the inbox already holds the messages)."""
        dev = x.device
        kw.setdefault("in_dtype", SGT_F32)
        kw.setdefault("out_dtype", SGT_F32)
        o = make_opts(**kw)
        _check(lib().sgt_ring_allreduce(self._h, _dev_ptr(x, "x", dev), _dev_ptr(left_msgs, "left_msgs", dev),
                                        _dev_ptr(inbox, "inbox", dev), _dev_ptr(outbox, "outbox", dev),
                                        _dev_ptr(out, "out", dev), _dev_ptr(flags, "flags", dev), W, x.numel(),
                                        ctypes.byref(o), _stream_handle(stream)))

    def gemm_rs(self, A_local, B, partials: Sequence, partial_out, C_shard, gflags, pflags, *, stream=None, **kw):
        """GEMM + ReduceScatter: partial_out = A_local @ B (fp32); C_shard = partial_out[block rank] +
        sum of the other ranks' partials."""
        dev = B.device
        W = len(partials)
        M, K = A_local.shape
        lay = kw.get("b_layout", "kn")
        N = B.shape[1] if lay == "kn" else B.shape[0]
        kw.setdefault("in_dtype", _dtype_code(B))
        o = make_opts(**kw)
        ptrs = (P * W)(*[_dev_ptr(p, "partials[%d]" % i, dev) if p is not None else 0
                         for i, p in enumerate(partials)])
        _check(lib().sgt_gemm_rs(self._h, _dev_ptr(A_local, "A_local", dev), _dev_ptr(B, "B", dev),
                                 ctypes.cast(ptrs, P), _dev_ptr(partial_out, "partial_out", dev),
                                 _dev_ptr(C_shard, "C_shard", dev), _dev_ptr(gflags, "gflags", dev),
                                 _dev_ptr(pflags, "pflags", dev), W, M, K, N, ctypes.byref(o),
                                 _stream_handle(stream)))

    def gemm_rs_paced(self, A_local, B, peer_blocks: Sequence, inbox: Sequence, partial_out, C_shard, gflags, pflags, *,
                      stream=None, **kw):
        """GEMM+ReduceScatter with the peers' blocks copied into `inbox` at the simulated link rate."""
        dev = A_local.device
        W = len(peer_blocks)
        M, K = A_local.shape
        lay = kw.get("b_layout", "kn")
        N = B.shape[1] if lay == "kn" else B.shape[0]
        kw.setdefault("in_dtype", _dtype_code(B))
        o = make_opts(**kw)
        src = (P * W)(*[_dev_ptr(p, "peer_blocks[%d]" % i, dev) if p is not None else 0
                        for i, p in enumerate(peer_blocks)])
        dst = (P * W)(*[_dev_ptr(p, "inbox[%d]" % i, dev) if p is not None else 0 for i, p in enumerate(inbox)])
        _check(lib().sgt_gemm_rs_paced(self._h, _dev_ptr(A_local, "A_local", dev), _dev_ptr(B, "B", dev),
                                       ctypes.cast(src, P), ctypes.cast(dst, P),
                                       _dev_ptr(partial_out, "partial_out", dev), _dev_ptr(C_shard, "C_shard", dev),
                                       _dev_ptr(gflags, "gflags", dev), _dev_ptr(pflags, "pflags", dev), W, M, K, N,
                                       ctypes.byref(o), _stream_handle(stream)))

    def moe_gemm_rs(self, Hg, W2, gate, topk_ids, expert_off, row_token, partials: Sequence, Y, partial_out,
                    C_shard, gflags, pflags, *, stream=None, inbox: Optional[Sequence] = None, **kw):
        """MoE GEMM + ReduceScatter (combine side); see sgt_moe_gemm_rs.  Y may be fp32 or bf16 (its dtype sets
        out_dtype).  With `inbox`, `partials` are the peers' blocks and arrive into `inbox` at the simulated link
        rate (sgt_moe_gemm_rs_paced)."""
        dev = Hg.device
        W = len(partials)
        rows, n_in = Hg.shape
        T, topk = topk_ids.shape
        lay = kw.get("b_layout", "kn")
        E = W2.shape[0]
        H = W2.shape[2] if lay == "kn" else W2.shape[1]
        if rows != T * topk:
            raise ValueError("Hg has %d rows, expected T * topk = %d" % (rows, T * topk))
        kw.setdefault("in_dtype", _dtype_code(Hg))
        kw.setdefault("out_dtype", _dtype_code(Y))   # Y fp32, or bf16 to halve its traffic
        o = make_opts(**kw)
        parts = (P * W)(*[_dev_ptr(p, "partials[%d]" % i, dev) if p is not None else 0
                          for i, p in enumerate(partials)])
        if inbox is not None:
            box = (P * W)(*[_dev_ptr(p, "inbox[%d]" % i, dev) if p is not None else 0 for i, p in enumerate(inbox)])
            _check(lib().sgt_moe_gemm_rs_paced(self._h, _dev_ptr(Hg, "Hg", dev), _dev_ptr(W2, "W2", dev),
                                               _dev_ptr(gate, "gate", dev), _dev_ptr(topk_ids, "topk_ids", dev),
                                               _dev_ptr(expert_off, "expert_off", dev),
                                               _dev_ptr(row_token, "row_token", dev), ctypes.cast(parts, P),
                                               ctypes.cast(box, P), _dev_ptr(Y, "Y", dev),
                                               _dev_ptr(partial_out, "partial_out", dev),
                                               _dev_ptr(C_shard, "C_shard", dev), _dev_ptr(gflags, "gflags", dev),
                                               _dev_ptr(pflags, "pflags", dev), W, T, topk, n_in, H, E,
                                               ctypes.byref(o), _stream_handle(stream)))
            return
        _check(lib().sgt_moe_gemm_rs(self._h, _dev_ptr(Hg, "Hg", dev), _dev_ptr(W2, "W2", dev),
                                     _dev_ptr(gate, "gate", dev), _dev_ptr(topk_ids, "topk_ids", dev),
                                     _dev_ptr(expert_off, "expert_off", dev), _dev_ptr(row_token, "row_token", dev),
                                     ctypes.cast(parts, P), _dev_ptr(Y, "Y", dev),
                                     _dev_ptr(partial_out, "partial_out", dev), _dev_ptr(C_shard, "C_shard", dev),
                                     _dev_ptr(gflags, "gflags", dev), _dev_ptr(pflags, "pflags", dev), W, T, topk,
                                     n_in, H, E, ctypes.byref(o), _stream_handle(stream)))

    def moe_ag_gemm(self, X_shards: Sequence, W_experts, logits, X_gathered, Y, expert_off, row_token, topk_ids,
                    shard_flags, *, topk: int, stream=None, **kw):
        """MoE AllGather + grouped GEMM (routing by top-k of logits, rows grouped by expert)."""
        dev = W_experts.device
        W = len(X_shards)
        T, H = X_gathered.shape
        E = W_experts.shape[0]
        lay = kw.get("b_layout", "kn")
        I = W_experts.shape[2] if lay == "kn" else W_experts.shape[1]
        kw.setdefault("in_dtype", SGT_BF16)
        if "out_dtype" not in kw:
            kw["out_dtype"] = _dtype_code(Y)
        o = make_opts(**kw)
        ptrs = (P * W)(*[_dev_ptr(x, "X_shards[%d]" % i, dev) for i, x in enumerate(X_shards)])
        _check(lib().sgt_moe_ag_gemm(self._h, ctypes.cast(ptrs, P), _dev_ptr(W_experts, "W_experts", dev),
                                     _dev_ptr(logits, "logits", dev), _dev_ptr(X_gathered, "X_gathered", dev),
                                     _dev_ptr(Y, "Y", dev), _dev_ptr(expert_off, "expert_off", dev),
                                     _dev_ptr(row_token, "row_token", dev), _dev_ptr(topk_ids, "topk_ids", dev),
                                     _dev_ptr(shard_flags, "shard_flags", dev), W, T, H, I, E, topk,
                                     ctypes.byref(o), _stream_handle(stream)))

    def a2a_dispatch(self, X: Sequence, topk: Sequence, recv, recv_token, recv_count, flags, E: int, *, stream=None,
                     **kw):
        """Expert-parallel AllToAll dispatch as rank `rank` receives it.  X: W tensors T_r x H (bf16 or fp32);
        topk: W int32 tensors T_r x k; recv: E/W x W x T_r x H; recv_token: E/W x W x T_r int32;
        recv_count: E/W x W int64 packets (epoch << 32 | count); flags: a2a_flag_count words."""
        dev = recv.device
        W = len(X)
        T_r, H = X[0].shape[0], X[0].shape[1]
        k = topk[0].shape[1]
        kw.setdefault("in_dtype", _dtype_code(X[0]))
        o = make_opts(**kw)
        xp = (P * W)(*[_dev_ptr(a, "X[%d]" % i, dev) for i, a in enumerate(X)])
        tp = (P * W)(*[_dev_ptr(t, "topk[%d]" % i, dev) for i, t in enumerate(topk)])
        _check(lib().sgt_a2a_dispatch(self._h, ctypes.cast(xp, P), ctypes.cast(tp, P), _dev_ptr(recv, "recv", dev),
                                      _dev_ptr(recv_token, "recv_token", dev), _dev_ptr(recv_count, "recv_count", dev),
                                      _dev_ptr(flags, "flags", dev), W, T_r, H, E, k, ctypes.byref(o),
                                      _stream_handle(stream)))

    def a2a_combine(self, back: Optional[Sequence], topk, gate, cbuf, slot_of, out, flags, W: int, *, stream=None,
                    **kw):
        """Expert-parallel AllToAll combine on rank `rank`: out[t] = sum_j gate[t, j] * (row slot(t, j) of expert
        topk[t, j]).  back: W bf16 tensors E/W x T_r x H (None with producer='preset': cbuf already holds the
        rows); topk, gate: T_r x k (int32, fp32); cbuf: E x T_r x H bf16; slot_of: T_r x k int32 (written);
        out: T_r x H fp32; flags: a2a_flag_count words."""
        dev = out.device
        T_r, H = out.shape[0], out.shape[1]
        k = topk.shape[1]
        E = cbuf.shape[0]
        kw.setdefault("in_dtype", SGT_BF16)
        kw.setdefault("out_dtype", SGT_F32)
        o = make_opts(**kw)
        if back is not None:
            bp = (P * W)(*[_dev_ptr(b, "back[%d]" % i, dev) for i, b in enumerate(back)])
            bptr = ctypes.cast(bp, P)
        else:
            bptr = None
        _check(lib().sgt_a2a_combine(self._h, bptr, _dev_ptr(topk, "topk", dev), _dev_ptr(gate, "gate", dev),
                                     _dev_ptr(cbuf, "cbuf", dev), _dev_ptr(slot_of, "slot_of", dev),
                                     _dev_ptr(out, "out", dev), _dev_ptr(flags, "flags", dev), W, T_r, H, E, k,
                                     ctypes.byref(o), _stream_handle(stream)))
