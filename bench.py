#!/usr/bin/env python3
"""Benchmark of the signal-gated tiled AllGather+GEMM on one MI355X.

Step = one overlapped sgt_ag_gemm call at the Llama-3-70B MLP share
(W = 8 shards, M = 16384 rows, K = 8192, N = 3584, bf16 ~ N(0, 0.02), fp32
accumulate and output): the producer kernel moves the 7 peer shards into the
gathered buffer at 153.6 GB/s per simulated peer with per-tile jitter up to
27 us and releases one flag per signal tile; the persistent MFMA consumer
waits on each panel's flags.  Inputs are resident in HBM before timing.

Prints one JSON line.  `value` is TFLOP/s of the overlapped step (2 M N K per
step).  Alongside: the same consumer with the data pre-resident and flags
preset (the GEMM alone), the serial producer-then-consumer run, the overlap
efficiency E = T(GEMM alone) / T(overlapped) from interleaved pairs and its
ceiling E_max, median and p10/p90 of the per-call times, an arrival sweep
(unthrottled, 153.6 and 50 GB/s per peer), MALL-flushed timings, the consumer
kernel's roofline (timed with HIP events recorded on its own stream around its
launch), the GEMM+ReduceScatter workload (M = 8192, K = 3200, N = 5120, 7
fp32 peer partials, resident and paced at 50 GB/s) with its reduction window,
the MoE AllGather + grouped GEMM workload, measured copy and hipBLASLt
ceilings, and the CPU oracle timed on a bounded sample of rows.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "AG-GEMM/GEMM-RS bf16 TFLOP/s, % MFMA peak, overlap efficiency vs GEMM-only"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0
K_CHUNKS = 8                # column chunks of K per AllGather signal tile on the headline workload


# HBM traffic of the consumer from the committed counter summary: valid only
# while the consumer's sources are the ones the counters were taken on.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "ag_consumer_bf16_llama70b_traffic.md")
CONSUMER_SOURCES = ["ag_gemm.hip", "mfma_tile.hpp", "signal.hpp", "sched.hpp", "common.hpp"]


def consumer_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in CONSUMER_SOURCES:
        with open(os.path.join(ROOT, "signal_gated_tiled_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per consumer dispatch (FETCH + WRITE, copy-calibrated), or None when the
    summary is missing or was taken on other consumer sources."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("consumer_source_sha256_16") != consumer_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, steps: int):
    """A plain copy of known size (fp32, 1 GiB read + 1 GiB written per launch) whose FETCH_SIZE and
    WRITE_SIZE counters scale the consumer's."""
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4, "launches": steps,
                                           "kernel": "torch.neg (vectorized elementwise)"}}), flush=True)


def _events(n, torch):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


LAST_HOST_MS = []


@contextlib.contextmanager
def no_gc():
    """Python's cyclic garbage collector off inside a timed loop (as timeit does): in a process holding
    torch's objects one full collection takes tens of milliseconds, which would land inside one call.  The
    collection runs once, before the warm-up (a collection between the warm-up and a timed block leaves the
    GPU idle long enough for its clock to drop); inside an outer no_gc() this does nothing."""
    if not gc.isenabled():
        yield
        return
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


# Under sustained load the engine clock settles within about a tenth of a second: after an idle gap (a
# workload's host-side setup, or a garbage collection of tens of milliseconds) the first ~100 calls of the
# Llama GEMM ran 3% slower than the rest, and the first 30 up to 10%.  Every warm-up therefore runs for at
# least this long (and at least its W calls), and nothing idles the GPU between it and the timed blocks.
WARM_S = 0.25


def warm(fn, warmup, torch, ctx):
    """fn(i, None) for i = 0, 1, ... until at least `warmup` calls and WARM_S seconds have passed (the host
    waits for the GPU after every 32 calls, so the seconds are the GPU's); returns the number of calls."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < WARM_S:
        fn(i, None)
        i += 1
        if i % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if ctx is not None:
        ctx.sync()
    return i


def timed(fn, steps, warmup, torch, ctx):
    """Run fn(i, events) warmup times (and for at least WARM_S seconds), then two blocks of `steps` calls.

    The first block records HIP events around every consumer launch (the kernel times).  The second passes
    no events: its wall time between two synchronizations is the step time (a timing event recorded around
    every call costs the stream up to tens of microseconds per call, so it is kept out of the step; running
    it second also lets the clocks settle under the load first).
    Returns (ms per step, mean consumer-kernel ms, per-call kernel ms).
    """
    with no_gc():
        return _timed(fn, steps, warmup, torch, ctx)


def _timed(fn, steps, warmup, torch, ctx):
    evk = _events(steps, torch)
    warm(fn, warmup, torch, ctx)
    for i in range(steps):
        fn(warmup + i, evk[i])
    torch.cuda.synchronize()
    ctx.sync()
    kern = [a.elapsed_time(b) for a, b in evk]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    host = [0.0] * steps
    t0.record()
    for i in range(steps):
        h0 = time.perf_counter()
        fn(warmup + steps + i, None)
        host[i] = time.perf_counter() - h0
    t1.record()
    torch.cuda.synchronize()
    ctx.sync()
    step_ms = t0.elapsed_time(t1) / steps
    # host time of each call in the step-timed block (ms): a call whose host side stalls shows here
    LAST_HOST_MS[:] = [h * 1e3 for h in host]
    return step_ms, statistics.mean(kern), kern


def timed_blocks(fn, steps, warmup, torch, ctx, blocks=3):
    """timed() whose step time is the median over `blocks` event-free blocks: for calls of tens of
    microseconds, where one host stall inside a single block would dominate its mean."""
    with no_gc():
        step, mean_k, kern = _timed(fn, steps, warmup, torch, ctx)
        steps_ms = [step]
        for b in range(blocks - 1):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for i in range(steps):
                fn(warmup + (b + 2) * steps + i, None)
            t1.record()
            torch.cuda.synchronize()
            ctx.sync()
            steps_ms.append(t0.elapsed_time(t1) / steps)
    return statistics.median(steps_ms), mean_k, kern


def spread(vals):
    """Median and 10th / 90th percentiles of a list of times."""
    v = sorted(vals)
    q = statistics.quantiles(v, n=10, method="inclusive") if len(v) > 1 else [v[0]] * 9
    return {"median": statistics.median(v), "p10": q[0], "p90": q[8], "n": len(v)}


def pairs(fn_a, fn_b, n, torch, ctx):
    """Interleave n calls of fn_a and fn_b (each given its consumer events); per-call kernel times of each.

    Pairs taken back to back see the same clock and thermal state, so their ratio is not biased by drift
    between two blocks of runs."""
    with no_gc():
        ev = _events(2 * n, torch)
        warm(lambda i, _: (fn_a(i, None), fn_b(i, None)), 1, torch, ctx)
        for i in range(n):
            fn_a(i, ev[2 * i])
            fn_b(i, ev[2 * i + 1])
    torch.cuda.synchronize()
    ctx.sync()
    return [a.elapsed_time(b) for a, b in ev[0::2]], [a.elapsed_time(b) for a, b in ev[1::2]]


def flushed(fn, n, torch, ctx, scrub):
    """Per call: overwrite a 512 MiB buffer (evicts the 256 MB MALL and the L2s), then time the whole call
    (producer fork to join) with events on the calling stream; returns the per-call times."""
    out = []
    for i in range(n):
        scrub.fill_(i & 0x7F)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i, None)
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    ctx.sync()
    return out


def device_clocks():
    """Engine and memory clocks as rocm-smi reports them right now (None if it is unavailable)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
    except Exception:  # noqa: BLE001 - a missing tool only drops this field
        return None
    lines = [ln.strip() for ln in r.stdout.splitlines() if "clock level" in ln.lower()]
    return lines or None


def power_under_load(fn, torch, ctx, samples=3):
    """Board power and per-XCD engine clocks as amd-smi reads them while fn runs back to back (after a warm-up):
    under sustained dense MFMA load the package sits at its power limit, which sets the clock.  amd-smi reads
    instantaneous values and the overlapped call's phases draw differently (copies, then the GEMM's tail), so
    it is read `samples` times in a row and the readings are reported with their maximum.  None if the tool is
    unavailable."""
    import re
    import subprocess

    def smi():
        return subprocess.Popen(["amd-smi", "metric", "-g", "0", "-p", "-c"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    outs = []
    with no_gc():
        warm(fn, 1, torch, ctx)
        t0 = time.perf_counter()
        proc, i = None, 0
        try:
            while len(outs) < samples:
                fn(i, None)
                i += 1
                if i % 8:
                    continue
                torch.cuda.synchronize()
                el = time.perf_counter() - t0
                if el > 30.0:
                    break
                if proc is None:
                    if el > 0.2:
                        proc = smi()
                elif proc.poll() is not None:
                    outs.append(proc.communicate(timeout=20)[0] or "")
                    proc = smi() if len(outs) < samples else None
        except (OSError, subprocess.SubprocessError):  # no amd-smi: only this field is dropped
            if proc is not None:
                proc.kill()
            return None
        if proc is not None:
            proc.kill()
        torch.cuda.synchronize()
        ctx.sync()
    pw, clk = [], []
    for out in outs:
        m = re.search(r"SOCKET_POWER:\s*(\d+)", out)
        c = [int(x) for x in re.findall(r"GFX_\d+:\s*CLK:\s*(\d+)\s*MHz", out)]
        if m:
            pw.append(int(m.group(1)))
        if c:
            clk.append(round(sum(c) / len(c)))
    if not pw:
        return None
    return {"socket_power_w": max(pw), "socket_power_w_samples": pw, "gfx_clk_mhz_mean_samples": clk,
            "calls": i, "note": "amd-smi read %d times in a row while the overlapped Llama call ran back to back; "
                                "socket_power_w is the largest reading" % len(pw)}


def microbench(torch, A, B_kn, steps):
    """Measured ceilings on this device: a 1 GiB device copy and hipBLASLt's bf16 GEMM (torch.matmul) at the
    headline shape, both timed with events; context for the hand-written kernels, not part of the method."""
    n = 1 << 28
    x = torch.empty(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    x.fill_(1.0)
    with no_gc():
        warm(lambda i, _: y.copy_(x), 2, torch, None)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    copy_ms = a.elapsed_time(b) / steps
    del x, y
    M, K = A.shape
    N = B_kn.shape[1]
    with no_gc():
        warm(lambda i, _: torch.matmul(A, B_kn), 2, torch, None)
    a.record()
    for _ in range(steps):
        C = torch.matmul(A, B_kn)
    b.record()
    torch.cuda.synchronize()
    mm_ms = a.elapsed_time(b) / steps
    del C
    return {"copy_1gib_gbs": 2 * 4 * n / (copy_ms * 1e-3) / 1e9,
            "copy_note": "read + write bytes of a 1 GiB fp32 device copy / time",
            "hipblaslt_bf16_gemm_tflops": 2.0 * M * N * K / (mm_ms * 1e-3) / 1e12,
            "hipblaslt_note": "torch.matmul of the resident gathered A (bf16) by a row-major K x N bf16 B, bf16 "
                              "output, same M, K, N"}


def cpu_baseline(shards, B, M, N, K, seconds: float, b_layout: str = "kn"):
    """The oracle (concat + fp64 loops over output rows), timed on a bounded sample of rows."""
    import numpy as np
    import oracle
    threads = oracle.max_threads()
    t = time.perf_counter()
    A_full = oracle.allgather(shards)
    t_gather = time.perf_counter() - t
    # candidate rows interleaved over the whole matrix (every shard early in the list)
    rows = np.concatenate([np.arange(r, M, 64, dtype=np.int64) for r in range(64)])
    n = max(threads, 8)
    t = time.perf_counter()
    oracle.gemm(A_full, B, b_layout=b_layout, rows=rows[:n])
    dt = time.perf_counter() - t
    n2 = int(min(len(rows), max(n, n * seconds / max(dt, 1e-3))))
    t = time.perf_counter()
    oracle.gemm(A_full, B, b_layout=b_layout, rows=rows[:n2])
    dt = time.perf_counter() - t
    flops = 2.0 * n2 * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d output rows of C (all %d columns, K=%d) by the fp64 oracle loop, %.1f s; "
                      "plus the %d-shard concat (%.2f s)" % (n2, M, N, K, dt, len(shards), t_gather),
            "seconds": dt}


def cpu_host_details(I):
    """The host the CPU oracle ran on (model, threads) and the oracle on the tiny fp32 workload with one
    thread and with all (whole workload, median of 5)."""
    import oracle
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    w = I.TINY
    shards, B = I.make_ag(w)
    out = {"cpu_model": model, "threads": oracle.max_threads(), "os_cpus": os.cpu_count()}
    for name, th in (("tiny_ag_gemm_1_thread_ms", 1), ("tiny_ag_gemm_all_threads_ms", 0)):
        ts = []
        for _ in range(5):
            t = time.perf_counter()
            oracle.gemm(oracle.allgather(shards), B, threads=th)
            ts.append((time.perf_counter() - t) * 1e3)
        out[name] = statistics.median(ts)
    return out


def release_times(ctx, call, trace_words, n_tiles, torch, n=3, local_flags=0):
    """The last signal tile's release, in microseconds from the call's first in-kernel stamp (a consumer
    tile's wait start or a release, whichever is earlier), median over n traced calls; also the first
    release of a remote signal tile (flags from local_flags on: rank 0's shard holds the first ones).  The
    trace holds 4 words per consumer tile, then one release stamp per signal tile (100 MHz clock)."""
    import numpy as np
    last, span, first, clock = [], [], [], []
    tr = torch.zeros(trace_words, dtype=torch.int64, device="cuda:0")
    for i in range(n):
        tr.zero_()
        call(i, tr.data_ptr())
        torch.cuda.synchronize()
        ctx.sync()
        t = tr.cpu().numpy().view(np.uint64).astype(np.int64)
        tiles = t[:4 * n_tiles].reshape(-1, 4)
        rel = t[4 * n_tiles:]
        t0 = min(tiles[:, 0].min(), rel.min())
        last.append((rel.max() - t0) / 100.0)
        span.append((tiles[:, 2].max() - t0) / 100.0)
        first.append((rel[local_flags:].min() - t0) / 100.0)
        # engine clock: each tile's cycles (bits 16.. of its last word) over its duration
        dur_us = (tiles[:, 2] - tiles[:, 0]) / 100.0
        cyc = tiles[:, 3] >> 16
        ok = (dur_us > 0) & (cyc > 0)
        if ok.any():
            clock.append(float(np.median(cyc[ok] / dur_us[ok])))
    del tr
    return {"last_release_us": statistics.median(last), "first_remote_release_us": statistics.median(first),
            "consumer_end_us": statistics.median(span), "n": n,
            "clock_mhz": statistics.median(clock) if clock else None}


def trace_clocks(traces, n_tiles):
    """Engine clock (MHz) of each traced call in `traces` (one AllGather trace per row): the median over its
    tiles of cycles / duration; None for a call without cycle counts."""
    import numpy as np
    out = []
    for row in traces.cpu().numpy().view(np.uint64).astype(np.int64):
        tiles = row[:4 * n_tiles].reshape(-1, 4)
        dur_us = (tiles[:, 2] - tiles[:, 0]) / 100.0
        cyc = tiles[:, 3] >> 16
        ok = (dur_us > 0) & (cyc > 0)
        out.append(float(np.median(cyc[ok] / dur_us[ok])) if ok.any() else None)
    return out


def trace_clock(call, trace_words, n_tiles, torch, ctx, n=3):
    """Median engine clock (MHz) over n traced calls: each tile's cycle count over its duration."""
    import numpy as np
    tr = torch.zeros(trace_words, dtype=torch.int64, device="cuda:0")
    out = []
    for i in range(n):
        tr.zero_()
        call(i, tr.data_ptr())
        torch.cuda.synchronize()
        ctx.sync()
        tiles = tr.cpu().numpy().view(np.uint64).astype(np.int64)[:4 * n_tiles].reshape(-1, 4)
        dur_us = (tiles[:, 2] - tiles[:, 0]) / 100.0
        cyc = tiles[:, 3] >> 16
        ok = (dur_us > 0) & (cyc > 0)
        if ok.any():
            out.append(float(np.median(cyc[ok] / dur_us[ok])))
    del tr
    return statistics.median(out) if out else None


def bench_engines(ctx, shards, B, Ag, C, flags, rank, lay, kc, link, alone_ms, flops, shape, args, torch, sgt):
    """The headline's overlapped step with the copy-engine producer (SGT_PROD_SDMA): every remote peer through
    the copy engines, and hybrids where the first sdma_peers peers go through the copy engines and the others
    through CU producer workgroups; per variant the step time, its overlap efficiency against the GEMM alone,
    the consumer kernel's time and when the first remote and the last signal tile were released."""
    W, M, K, N = shape
    engines = {}
    for name, kw in (("engines_all_peers", dict(producer="sdma")),
                     ("engines_2_peers_cu_5", dict(producer="sdma", sdma_peers=2)),
                     ("engines_3_peers_cu_4", dict(producer="sdma", sdma_peers=3))):
        e_ms, e_k, e_l = timed(lambda i, ev: ctx.ag_gemm(shards, B, Ag, C, flags, rank=rank, b_layout=lay,
                                                         consumer_events=ev, k_chunks=kc, arrival_seed=5000 + i,
                                                         **link, **kw), max(6, args.steps // 2), 3, torch, ctx)
        e_rel = release_times(ctx, lambda i, tr: ctx.ag_gemm(shards, B, Ag, C, flags, rank=rank, b_layout=lay,
                                                              k_chunks=kc, arrival_seed=6000 + i, trace=tr,
                                                              **link, **kw),
                              sgt.trace_words(W, M, K, N, k_chunks=kc), (M // 256) * (-(-N // 256)), torch,
                              local_flags=sgt.ag_flag_count(W, M, K, k_chunks=kc) // W)
        engines[name] = {"step_ms": e_ms, "tflops_step": flops / (e_ms * 1e-3) / 1e12,
                         "overlap_efficiency_step": alone_ms / e_ms, "consumer_kernel_ms": spread(e_l),
                         "first_remote_release_us": e_rel["first_remote_release_us"],
                         "last_release_us": e_rel["last_release_us"], "consumer_end_us": e_rel["consumer_end_us"]}
    assert torch.equal(Ag.view(torch.int16), torch.cat(shards).view(torch.int16)), "gathered buffer (copy engines)"
    return engines


def bench_ag_other(ctx, up, args, torch, sgt, I, lay):
    """The other AllGather workloads: the Qwen3-32B MLP share at 50 GB/s per peer (the link floor exceeds the
    GEMM, so E is bounded well below 1) and the tiny fp32 case (launch-bound)."""
    out = {}
    for w, kw in ((I.QWEN_AG, dict(b_layout=lay)), (I.TINY, dict(b_layout="kn"))):
        shards_h, B_h = I.make_ag(w, B_layout=kw["b_layout"])
        shards = [up(x) for x in shards_h]
        B = up(B_h)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        Ag = torch.empty((w.M, w.K), dtype=dt, device="cuda:0")
        C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
        fr = getattr(w, "flag_rows", 0)
        # K-chunked signal tiles where the tile supports them (bf16, B as N x K, whole 256-row panels per shard)
        kc = K_CHUNKS if (w.dtype == "bf16" and kw["b_layout"] == "nk" and w.K % (128 * K_CHUNKS) == 0
                          and (w.M // w.W) % 256 == 0) else 0
        flags = torch.zeros(sgt.ag_flag_count(w.W, w.M, w.K, flag_rows=fr, k_chunks=kc), dtype=torch.int32,
                            device="cuda:0")
        link = dict(peer_gbps=w.peer_gbps, jitter_us=w.jitter_us, flag_rows=fr, k_chunks=kc)
        if w is I.TINY:
            link["arrival_order"] = "global"

        def ag(producer, **k2):
            def fn(i, ev):
                ctx.ag_gemm(shards, B, Ag, C, flags, rank=0, producer=producer, consumer_events=ev, **kw, **k2)
            return fn
        over_ms, _, over_l = timed(lambda i, ev: ag("cu", arrival_seed=i + 1, **link)(i, ev), args.steps,
                                   args.warmup, torch, ctx)
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        ov_l, al_l = pairs(lambda i, ev: ag("cu", arrival_seed=500 + i, **link)(i, ev),
                           ag("preset", consumer_cus=n_cu - max(8, n_cu // 8)), args.steps, torch, ctx)
        assert torch.equal(Ag.view(torch.int16 if w.dtype == "bf16" else torch.int32),
                           torch.cat(shards).view(torch.int16 if w.dtype == "bf16" else torch.int32)), w.name
        floor_us = (w.M // w.W) * w.K * (2 if w.dtype == "bf16" else 4) / (w.peer_gbps * 1e9) * 1e6 \
            if w.peer_gbps else 0.0
        flops = 2.0 * w.M * w.N * w.K
        al = statistics.median(al_l)
        bm = 256 if w.dtype == "bf16" else 64
        grid = n_cu - max(8, n_cu // 8)
        tiles = -(-w.M // bm) * -(-w.N // bm)
        # after the link floor the last panel's tiles still compute their last chunk (a whole tile without chunks)
        tail = al * 1e3 * grid / tiles / (kc if kc else 1)
        out[w.name] = {
            "M": w.M, "K": w.K, "N": w.N, "W": w.W, "dtype": w.dtype, "k_chunks": kc,
            "peer_gbps": w.peer_gbps or None,
            "jitter_us": w.jitter_us, "step_ms": over_ms, "tflops_step": flops / (over_ms * 1e-3) / 1e12,
            "overlapped_kernel_ms": spread(over_l), "pairs_alone_kernel_ms": spread(al_l),
            "overlap_efficiency": al / statistics.median(ov_l),
            "overlap_efficiency_max": (al * 1e3 / max(al * 1e3, floor_us + tail) if floor_us else 1.0),
            "link_floor_us": floor_us,
        }
        del shards, B, Ag, C, flags
    out["note"] = ("overlap_efficiency_max estimates the ceiling: the GEMM alone over the link floor plus the "
                   "work left once the last data lands (one tile time, or one K chunk of it with K-chunked signal "
                   "tiles; tiles that run alone at the end run faster, so a measured value can exceed it "
                   "slightly); "
                   "the tiny fp32 case is latency-bound and checked mainly for correctness")
    return out


def bench_ll(ctx, up, args, torch, sgt, I):
    """Low-latency (packet) AllGather against the flag-based one at decode sizes: Llama-3-70B hidden size
    (K = 8192, bf16), W = 8, 1 to 1024 tokens per rank, chunks of 1 row (16 KiB) and of 4 rows (64 KiB),
    32 or 96 workgroups for the simulated peers and as many for the receiver (96 lets the peers' side
    deliver LL's doubled bytes at the 153.6 GB/s link rate).

    Per call: the whole call's time (back to back, stream-ordered), the kernel's time, and from an
    in-kernel trace the time from the producer's first write to the receiver's last chunk seen and the
    per-chunk latency (remote chunks: producer's first write of the chunk to the receiver seeing all of it).
    """
    import numpy as np
    out = {}
    W, K = 8, 8192
    for tokens in (1, 16, 128, 1024):
        M = W * tokens
        w = I.AGWorkload("ll", W=W, M=M, K=K, N=0, seed_index=6)
        shards = [up(s) for s in I.make_ag(w)[0]]
        ref = torch.cat(shards)
        G = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
        ll = torch.zeros(sgt.ll_buffer_bytes(W, M, K) // 8, dtype=torch.int64, device="cuda:0")
        row = {"M": M, "K": K, "W": W, "tokens_per_rank": tokens, "payload_mib": M * K * 2 / 2**20}
        best = {}
        variants = [(fr, cus, link, gbps) for fr in sorted({1, min(tokens, 4)}) for cus in (32, 96)
                    for link, gbps in (("unthrottled", 0.0), ("153.6GBps", 153.6))
                    if cus == 96 or gbps == 0.0]
        for fr, cus, link, gbps in variants:
            n = M // fr
            fl = torch.zeros(sgt.ag_flag_count(W, M, K, flag_rows=fr), dtype=torch.int32, device="cuda:0")
            tr = torch.zeros(2 * n, dtype=torch.int64, device="cuda:0")
            per_shard = tokens // fr
            if True:
                for kind in ("ll", "flag"):
                    def call(i, ev, trace=0, kind=kind, gbps=gbps, fr=fr, fl=fl, cus=cus):
                        kw = dict(rank=0, flag_rows=fr, peer_gbps=gbps, consumer_events=ev, trace=trace,
                                  producer_cus=cus, consumer_cus=cus)
                        if kind == "ll":
                            ctx.ll_allgather(shards, ll, G, **kw)
                        else:
                            ctx.allgather(shards, G, fl, **kw)
                    step_ms, _, kern = timed(call, args.steps, 5, torch, ctx)
                    G.zero_()
                    call(0, None, trace=tr.data_ptr())
                    torch.cuda.synchronize()
                    ctx.sync()
                    assert torch.equal(G, ref), "gathered rows differ (%s, %d tokens)" % (kind, tokens)
                    t = tr.cpu().numpy().reshape(n, 2).astype(np.float64)
                    remote = np.arange(n) >= per_shard          # rank 0: chunks past the first shard
                    lat = (t[remote, 1] - t[remote, 0]) / 100.0  # 100 MHz ticks -> us
                    r = {"call_us": step_ms * 1e3,
                         "kernel_us": {k: v * 1e3 if k != "n" else v for k, v in spread(kern).items()},
                         "first_write_to_last_seen_us": (t[:, 1].max() - t[:, 0].min()) / 100.0,
                         "chunk_latency_us": spread(list(lat))}
                    key = "%s_%s" % (kind, link)
                    row["%s_chunk%dkib_wg%d" % (key, fr * K * 2 // 1024, cus)] = r
                    if key not in best or r["first_write_to_last_seen_us"] < best[key][2]:
                        best[key] = (fr * K * 2 // 1024, cus, r["first_write_to_last_seen_us"],
                                     r["chunk_latency_us"]["median"], r["call_us"])
        row["best"] = {k: {"chunk_kib": v[0], "workgroups_each_side": v[1], "first_write_to_last_seen_us": v[2],
                           "chunk_latency_median_us": v[3], "call_us": v[4]} for k, v in best.items()}
        out["ll_ag_decode_%dtok" % tokens] = row
    # where LL stops paying: per token count, each method at its best chunk and grid (unthrottled links)
    cross = {}
    for key, row in out.items():
        b = row.get("best", {})
        if "ll_unthrottled" in b and "flag_unthrottled" in b:
            cross[row["tokens_per_rank"]] = (b["ll_unthrottled"]["first_write_to_last_seen_us"],
                                             b["flag_unthrottled"]["first_write_to_last_seen_us"])
    up_to = 0   # the largest size up to which LL wins at every measured size
    for tk, (l_us, f_us) in sorted(cross.items()):
        if l_us >= f_us:
            break
        up_to = tk
    out["crossover"] = {
        "per_tokens_per_rank": {str(tk): {"ll_us": v[0], "flag_us": v[1]} for tk, v in sorted(cross.items())},
        "ll_faster_up_to_tokens_per_rank": up_to,
        "note": "first write to last chunk seen, in-kernel; above this size the flag-based AllGather is the one "
                "to use",
    }
    out["note"] = ("LL packets carry their epoch, so the receiver reads data and arrival in one load; the flag path "
                   "copies, waits for the stores' acknowledgement, publishes a flag, and the receiver polls it. "
                   "LL moves twice the bytes on the link and unpacks on the receiver. call_us is host-bound "
                   "(argument marshalling and one launch) at these sizes; the in-kernel figures compare the methods.")
    return out


def bench_ring(ctx, up, args, torch, sgt, I, resident_only=False):
    """One rank's share of the signal-gated ring AllReduce: 2048 x 8192 fp32 per rank, W = 8, the left
    neighbour's link at 153.6 GB/s.

    Kernel alone (messages resident, flags preset) against HBM; the overlapped call against the link floor
    (2(W-1) messages of N/W floats over one link); the serial call (all messages land, then the kernel).
    """
    w = I.RING
    W, N = w.W, w.N
    C = N // W
    x = up(I.make_ring(w)[0])
    msgs = up(I.make_ring_messages(w)).reshape(-1)
    inbox = torch.empty(2 * (W - 1) * C, dtype=torch.float32, device="cuda:0")
    outbox = torch.empty_like(inbox)
    out = torch.empty(N, dtype=torch.float32, device="cuda:0")
    nf, tile = sgt.ring_flag_count(W, N)
    flags = torch.zeros(nf, dtype=torch.int32, device="cuda:0")

    def call(producer, **kw):
        def fn(i, ev):
            ctx.ring_allreduce(x, msgs, inbox, outbox, out, flags, W, rank=0, producer=producer,
                               consumer_events=ev, **kw)
        return fn

    res = {"workload": w.name, "N": N, "W": W, "tile_elems": tile, "peer_gbps": w.peer_gbps}
    # algorithmic bytes of one rank per chunk element: first send 8, ReduceScatter steps 12 (the last 16),
    # AllGather steps 12 (the last 8)
    alg = (32 + 24 * (W - 2)) * C
    inbox.copy_(msgs)
    step, mean_k, kern = timed(call("preset"), args.steps, 5, torch, ctx)
    k = spread(kern)
    res["resident"] = {"step_ms": step, "kernel_ms": k, "hbm_gbps": alg / (k["median"] * 1e-3) / 1e9,
                       "hbm_frac": alg / (k["median"] * 1e-3) / 8e12, "algorithmic_mb": alg / 1e6}
    if resident_only:
        return res
    floor_us = 2 * (W - 1) * C * 4 / (w.peer_gbps * 1e3)
    for name, kw in (("overlapped_153.6GBps", dict(peer_gbps=w.peer_gbps)),
                     ("serial_153.6GBps", dict(peer_gbps=w.peer_gbps)),
                     ("overlapped_unthrottled", dict())):
        prod = "serial" if name.startswith("serial") else "cu"
        step, _, kern = timed(call(prod, **kw), max(10, args.steps // 2), 3, torch, ctx)
        r = {"step_ms": step, "kernel_ms": spread(kern)}
        if "153.6" in name:
            r["link_floor_us"] = floor_us
            r["efficiency_vs_link_floor"] = floor_us / (step * 1e3)
        res[name] = r
    # check this rank's result against its own steps (torch on the device, the same fp32 additions)
    owned = 1 % W
    exp_owned = x[owned * C:(owned + 1) * C] + msgs[(W - 2) * C:(W - 1) * C]
    assert torch.equal(out[owned * C:(owned + 1) * C], exp_owned), "owned chunk"
    for s_ in range(W - 1):
        c = (0 - s_) % W
        k_ = W - 1 + s_
        assert torch.equal(out[c * C:(c + 1) * C], msgs[k_ * C:(k_ + 1) * C]), "gathered chunk %d" % c
    res["note"] = ("overlapped: every tile waits only on its own arrival flag, so the reduction and forwarding "
                   "hide under the link; serial: the messages land first, then the same kernel runs")
    return res


def moe_routing(ctx, up, torch, sgt, I):
    """(expert_off, row_token, topk_ids) of the MoE workload's tokens from one MoE AllGather + grouped GEMM call
    (the library's GPU routing)."""
    m = I.MOE
    dev = "cuda:0"
    sh_h, We_h, lg_h = I.make_moe(m)
    Xg = torch.empty((m.T, m.H), dtype=torch.bfloat16, device=dev)
    Y = torch.empty((m.T * m.topk, m.I), dtype=torch.float32, device=dev)
    off = torch.empty(m.E + 1, dtype=torch.int32, device=dev)
    rt = torch.empty(m.T * m.topk, dtype=torch.int32, device=dev)
    ids = torch.empty((m.T, m.topk), dtype=torch.int32, device=dev)
    fl = torch.zeros(sgt.ag_flag_count(m.W, m.T, m.H), dtype=torch.int32, device=dev)
    ctx.moe_ag_gemm([up(s) for s in sh_h], up(We_h), up(lg_h), Xg, Y, off, rt, ids, fl, topk=m.topk, blocking=True)
    return off, rt, ids


def bench_a2a(ctx, up, args, torch, sgt, I, tables):
    """Expert-parallel AllToAll of the same MoE layer on rank 0 (W 8, 512 tokens per rank, hidden 2048 bf16,
    top-8 of 64 experts, 8 per rank, 32-row chunks): the dispatch and the combine, each with links at 50 GB/s
    per peer and unthrottled, against the link floor (the busiest link's bytes over its rate) and HBM."""
    import numpy as np
    w = I.A2A
    W, T_r, H, E, k = w.W, w.tokens_per_rank, w.H, w.E, w.topk
    E_l = E // W
    rank = 0
    dev = "cuda:0"
    _, _, ids = tables   # the MoE AllGather side's GPU routing of the layer's 4096 tokens (T x k)
    X_h, _, gate_h, back_h = I.make_a2a(w)
    X = [up(x) for x in X_h]
    topk = [ids[p * T_r:(p + 1) * T_r].contiguous() for p in range(W)]
    gate = up(gate_h[rank * T_r:(rank + 1) * T_r])
    back = [up(b) for b in back_h]
    recv = torch.empty((E_l, W, T_r, H), dtype=torch.bfloat16, device=dev)
    tok = torch.empty((E_l, W, T_r), dtype=torch.int32, device=dev)
    cnt = torch.zeros((E_l, W), dtype=torch.int64, device=dev)
    nf = sgt.a2a_flag_count(W, T_r, E, flag_rows=w.chunk_rows)
    dfl = torch.zeros(nf, dtype=torch.int32, device=dev)
    cbuf = torch.empty((E, T_r, H), dtype=torch.bfloat16, device=dev)
    slot = torch.empty((T_r, k), dtype=torch.int32, device=dev)
    out = torch.empty((T_r, H), dtype=torch.float32, device=dev)
    cfl = torch.zeros(nf, dtype=torch.int32, device=dev)
    row = H * 2

    def disp(**kw):
        def fn(i, ev):
            ctx.a2a_dispatch(X, topk, recv, tok, cnt, dfl, E, rank=rank, flag_rows=w.chunk_rows,
                             consumer_events=ev, **kw)
        return fn

    def comb(**kw):
        def fn(i, ev):
            ctx.a2a_combine(back if kw.get("producer") != "preset" else None, topk[rank], gate, cbuf, slot, out,
                            cfl, W, rank=rank, flag_rows=w.chunk_rows, consumer_events=ev, **kw)
        return fn

    res = {"workload": w.name, "W": W, "tokens_per_rank": T_r, "H": H, "E": E, "topk": k, "rank": rank,
           "chunk_rows": w.chunk_rows, "routing": "the MoE AllGather side's GPU routing of the same 4096 tokens"}
    n_steps = max(10, args.steps // 2)
    # dispatch
    d_link = {}
    for name, kw in (("paced_50GBps", dict(peer_gbps=w.peer_gbps)), ("unthrottled", dict())):
        step, _, kern = timed_blocks(disp(**kw), n_steps, 3, torch, ctx)
        d_link[name] = {"step_ms": step, "kernel_ms": spread(kern)}
    counts = (cnt.cpu().numpy() & 0xFFFFFFFF).astype(np.int64)           # E_l x W
    link_rows = counts.sum(axis=0)                                        # rows per source link
    remote = [p for p in range(W) if p != rank]
    floor_us = max(link_rows[p] for p in remote) * row / (w.peer_gbps * 1e3)
    rows = int(counts.sum())
    # algorithmic bytes: every received row read once and written once, the W routing tables read, the
    # token lists and count packets written
    d_bytes = 2 * rows * row + W * T_r * k * 4 + rows * 4 + E * 8
    d_link["paced_50GBps"]["link_floor_us"] = floor_us
    d_link["paced_50GBps"]["efficiency_vs_link_floor"] = floor_us / (d_link["paced_50GBps"]["kernel_ms"]["median"]
                                                                     * 1e3)
    u = d_link["unthrottled"]["kernel_ms"]["median"]
    d_link["unthrottled"]["hbm_gbps"] = d_bytes / (u * 1e-3) / 1e9
    d_link["unthrottled"]["hbm_frac"] = d_bytes / (u * 1e-3) / 1e9 / PEAK_HBM_GBS
    d_link["rows_received"] = rows
    d_link["rows_per_link_min_max"] = [int(link_rows.min()), int(link_rows.max())]
    d_link["algorithmic_bytes"] = d_bytes
    # spot check: a few received blocks against the tokens they name (bits)
    for l, p in ((0, 1), (E_l - 1, W - 1), (3, rank)):
        n = int(counts[l, p])
        assert torch.equal(recv[l, p, :n].view(torch.int16), X[p][tok[l, p, :n].long()].view(torch.int16)), \
            "dispatch block (%d, %d)" % (l, p)
    res["dispatch"] = d_link
    # combine
    c_res = {}
    for name, kw in (("paced_50GBps", dict(peer_gbps=w.peer_gbps)),
                     ("serial_50GBps", dict(peer_gbps=w.peer_gbps, producer="serial")),
                     ("unthrottled", dict()), ("receiver_alone", dict(producer="preset"))):
        step, _, kern = timed_blocks(comb(**kw), n_steps, 3, torch, ctx)
        c_res[name] = {"step_ms": step, "kernel_ms": spread(kern)}
    ids_r = topk[rank].cpu().numpy()
    n_e = np.array([int(((ids_r == e).any(axis=1)).sum()) for e in range(E)])
    c_link = n_e.reshape(W, E_l).sum(axis=1)                              # rows per owner link
    c_floor = max(c_link[q] for q in remote) * row / (w.peer_gbps * 1e3)
    c_res["paced_50GBps"]["link_floor_us"] = c_floor
    c_res["paced_50GBps"]["efficiency_vs_link_floor"] = c_floor / (c_res["paced_50GBps"]["kernel_ms"]["median"]
                                                                   * 1e3)
    c_res["serial_50GBps"]["link_floor_us"] = c_floor
    # receiver bytes: k bf16 rows read and one fp32 row written per token, the routing, gate and slot tables
    r_bytes = T_r * k * row + T_r * H * 4 + T_r * k * 12
    ra = c_res["receiver_alone"]["kernel_ms"]["median"]
    c_res["receiver_alone"]["hbm_gbps"] = r_bytes / (ra * 1e-3) / 1e9
    c_res["receiver_alone"]["hbm_frac"] = r_bytes / (ra * 1e-3) / 1e9 / PEAK_HBM_GBS
    c_res["receiver_algorithmic_bytes"] = r_bytes
    c_res["rows_per_link_min_max"] = [int(c_link.min()), int(c_link.max())]
    # spot check: token 0's output from its picks' rows in the receive buffer (fp32 on the device)
    s0 = slot[0].long()
    e0 = topk[rank][0].long()
    ref0 = torch.zeros(H, dtype=torch.float32, device=dev)
    for j in range(k):
        ref0 = torch.addcmul(ref0, gate[0, j].expand(H), cbuf[e0[j], s0[j]].float())
    assert torch.allclose(out[0], ref0, rtol=1e-5, atol=1e-5), "combine token 0"
    res["combine"] = c_res
    res["note"] = ("senders simulate the peers: each (link, expert) block travels in 32-row chunks, each flagged "
                   "when its link would deliver it; the combine receiver waits per token only on the chunks "
                   "of its picks")
    del recv, cbuf, back, X
    return res


def bench_moe(ctx, up, args, torch, sgt, I, lay):
    """MoE AllGather + grouped GEMM (T 4096 tokens in 8 shards, H 2048, I 768, 64 experts, top-8, Zipf-skewed
    logits), overlapped at 50 GB/s per simulated peer; the grouped consumer's MFMA and HBM roofline fractions."""
    import numpy as np
    m = I.MOE
    dev = "cuda:0"
    sh_h, We_h, lg_h = I.make_moe(m, W_layout=lay)
    sh = [up(s) for s in sh_h]
    We, lg = up(We_h), up(lg_h)
    Xg = torch.empty((m.T, m.H), dtype=torch.bfloat16, device=dev)
    Y = torch.empty((m.T * m.topk, m.I), dtype=torch.float32, device=dev)
    off = torch.empty(m.E + 1, dtype=torch.int32, device=dev)
    rt = torch.empty(m.T * m.topk, dtype=torch.int32, device=dev)
    ids = torch.empty((m.T, m.topk), dtype=torch.int32, device=dev)
    fl = torch.zeros(sgt.ag_flag_count(m.W, m.T, m.H), dtype=torch.int32, device=dev)

    def call(producer, **kw):
        def fn(i, ev):
            ctx.moe_ag_gemm(sh, We, lg, Xg, Y, off, rt, ids, fl, topk=m.topk, b_layout=lay, producer=producer,
                            consumer_events=ev, **kw)
        return fn

    link = dict(peer_gbps=m.peer_gbps)
    over_ms, over_k, _ = timed(lambda i, ev: call("cu", arrival_seed=i + 1, **link)(i, ev), args.steps, args.warmup,
                               torch, ctx)
    alone_ms, alone_k, _ = timed(call("preset"), args.steps, args.warmup, torch, ctx)
    serial_ms, _, _ = timed(lambda i, ev: call("serial", arrival_seed=i + 1, **link)(i, ev),
                            max(3, args.steps // 4), 2, torch, ctx)
    # the overlapped call's consumer runs on the whole chip (its last workgroups take the producer's CUs as
    # the producer finishes), so the GEMM alone is timed on the whole chip too
    ov_l, al_l = pairs(lambda i, ev: call("cu", arrival_seed=2000 + i, **link)(i, ev), call("preset"), args.steps,
                       torch, ctx)
    ov_k, al_k = statistics.median(ov_l), statistics.median(al_l)
    # spot checks (parity itself is the tests' job): gathered bits, and group offsets that cover T * topk rows
    assert torch.equal(Xg.view(torch.int16), torch.cat(sh).view(torch.int16)), "MoE gathered buffer mismatch"
    off_h = off.cpu().numpy()
    assert off_h[0] == 0 and off_h[-1] == m.T * m.topk and (np.diff(off_h) >= 0).all(), "MoE group offsets"
    flops = m.flops
    hbm = m.E * m.H * m.I * 2 + m.T * m.H * 2 + m.T * m.topk * m.I * 4   # weights + tokens once + Y (fp32)
    groups = np.diff(off_h)
    # rows the matrix cores compute: 256-row tiles, the last tile of a group 128 rows when at most 128 are left
    rem = groups % 256
    used_rows = int(np.sum(groups // 256) * 256 + np.sum(np.where(rem == 0, 0, np.where(rem <= 128, 128, 256))))
    out = {
        "workload": m.name, "T": m.T, "H": m.H, "I": m.I, "E": m.E, "topk": m.topk, "W": m.W,
        "peer_gbps": m.peer_gbps, "gflop": flops / 1e9, "algorithmic_hbm_bytes": hbm,
        "group_rows_min_max": [int(groups.min()), int(groups.max())],
        "mfma_rows_computed_over_routed": used_rows / float(m.T * m.topk),
        "step_ms": over_ms, "tflops_step": flops / (over_ms * 1e-3) / 1e12,
        "consumer_kernel_ms": over_k,
        "consumer_mfma_frac": flops / (over_k * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "consumer_hbm_frac": hbm / (over_k * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "resident_consumer_mfma_frac": flops / (alone_k * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "resident_consumer_hbm_frac": hbm / (alone_k * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "consumer_frac_note": "consumer_*: the overlapped call's consumer kernel, which also waits for its tokens; "
                              "resident_consumer_*: the same kernel with the tokens resident (its own timed block)",
        "preset_step_ms": alone_ms, "preset_consumer_kernel_ms": alone_k,
        "serial_ms": serial_ms, "speedup_vs_serial": serial_ms / over_ms,
        "overlap_efficiency": al_k / ov_k,
        "overlap_efficiency_note": "median consumer-kernel time with the tokens resident and flags preset (whole "
                                   "chip, as the overlapped consumer) over that of the overlapped call, interleaved "
                                   "pairs; routing excluded",
        "step_overlap_efficiency": alone_ms / over_ms,
        "pairs_kernel_ms": spread(ov_l), "pairs_preset_kernel_ms": spread(al_l),
        "link_floor_us": (m.T // m.W) * m.H * 2 / (m.peer_gbps * 1e9) * 1e6,
    }
    del sh, We, lg, Xg, Y
    return out, (off, rt, ids)


def bench_moe_rs(ctx, up, args, torch, sgt, I, lay, tables, resident_only=False):
    """MoE GEMM + ReduceScatter (combine side) of the same layer: T 4096 tokens, top-8 of 64 experts, I 768 ->
    H 2048, W 8; routing tables from the AllGather side's GPU routing; peers' partials resident."""
    import numpy as np
    m = I.MOE_RS
    dev = "cuda:0"
    off, rt, ids = tables
    Hg_h, W2_h, gate_h, _, parts_h = I.make_moe_rs(m, W_layout=lay)
    Hg, W2, gate = up(Hg_h), up(W2_h), up(gate_h)
    rank = 0
    parts = [up(p) if q != rank else None for q, p in enumerate(parts_h)]
    rows = m.T * m.topk
    Y = torch.empty((rows, m.H), dtype=torch.float32, device=dev)
    P = torch.empty((m.T, m.H), dtype=torch.float32, device=dev)
    Cs = torch.empty((m.T // m.W, m.H), dtype=torch.float32, device=dev)
    ng, npf = sgt.rs_flag_count(m.W, m.T, m.H, rs_tile=128)
    gf = torch.zeros(ng, dtype=torch.int32, device=dev)
    pf = torch.zeros(npf, dtype=torch.int32, device=dev)

    def fn(i, ev):
        ctx.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, Y, P, Cs, gf, pf, rank=rank, b_layout=lay,
                        consumer_events=ev)
    step_ms, kern_ms, kern = timed(fn, args.steps, args.warmup, torch, ctx)
    if resident_only:
        return {"step_ms": step_ms, "kernel_ms": spread(kern)}
    # the peers' partials arriving at 50 GB/s per link into an inbox
    gbps = 50.0
    inbox = [torch.empty_like(p) if p is not None else None for p in parts]

    def fn_paced(i, ev):
        ctx.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, Y, P, Cs, gf, pf, rank=rank, b_layout=lay,
                        consumer_events=ev, inbox=inbox, peer_gbps=gbps, arrival_seed=i + 1)
    pc_ms, _, pc_k = timed(fn_paced, max(4, args.steps // 2), 2, torch, ctx)
    assert torch.equal(inbox[1], parts[1]), "paced inbox mismatch"
    del inbox
    # Y stored in bf16 (half the bytes written and read back; P and C stay fp32)
    Yb = torch.empty((rows, m.H), dtype=torch.bfloat16, device=dev)

    def fn_b(i, ev):
        ctx.moe_gemm_rs(Hg, W2, gate, ids, off, rt, parts, Yb, P, Cs, gf, pf, rank=rank, b_layout=lay,
                        consumer_events=ev)
    yb_ms, _, yb_k = timed(fn_b, args.steps, args.warmup, torch, ctx)
    hbm_b = rows * m.I * 2 + m.E * m.I * m.H * 2 + 2 * rows * m.H * 2 + m.T * m.H * 4 + (m.W + 1) * (m.T // m.W) * m.H * 4
    del Yb
    flops = m.flops
    # algorithmic HBM bytes: Hg and W2 read once, Y written and read back once, P written, this rank's block of
    # P read back with the W-1 peers' blocks, C written
    blk = (m.T // m.W) * m.H * 4
    hbm = rows * m.I * 2 + m.E * m.I * m.H * 2 + 2 * rows * m.H * 4 + m.T * m.H * 4 + (m.W + 1) * blk
    med = statistics.median(kern)
    return {
        "workload": m.name, "T": m.T, "I": m.I, "H": m.H, "E": m.E, "topk": m.topk, "W": m.W,
        "routing": "the AllGather side's GPU routing of the same tokens (group sizes as above)",
        "gflop": flops / 1e9, "algorithmic_hbm_bytes": hbm,
        "step_ms": step_ms, "tflops_step": flops / (step_ms * 1e-3) / 1e12,
        "kernel_ms": spread(kern),
        "kernel_mfma_frac": flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "kernel_hbm_frac": hbm / (med * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "paced_50gbps": {"peer_gbps": gbps, "step_ms": pc_ms, "kernel_ms": spread(pc_k),
                         "tflops": flops / (pc_ms * 1e-3) / 1e12,
                         "link_floor_us": (m.T // m.W) * m.H * 4 / (gbps * 1e9) * 1e6},
        "y_bf16": {"step_ms": yb_ms, "kernel_ms": spread(yb_k), "tflops": flops / (yb_ms * 1e-3) / 1e12,
                   "algorithmic_hbm_bytes": hbm_b,
                   "kernel_hbm_frac": hbm_b / (statistics.median(yb_k) * 1e-3) / 1e9 / PEAK_HBM_GBS,
                   "kernel_mfma_frac": flops / (statistics.median(yb_k) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "note": "one persistent kernel: grouped GEMM tiles, gate-weighted combine tiles gated on their GEMM "
                "column, signal-gated reduction of this rank's block; peers' partials resident (and paced)",
    }


def kernel_pass(name, ctx, up, args, torch, sgt, I, lay):
    """One workload's kernels with resident data and preset flags only, for counter passes (a counter run
    serializes kernels, so a call whose consumer waits on a producer on another stream cannot run under it).
    Prints the per-call kernel times."""
    dev = "cuda:0"
    res = {"kernel_pass": name}
    if name in ("moe", "moe_rs", "a2a"):
        m = I.MOE
        sh_h, We_h, lg_h = I.make_moe(m, W_layout=lay)
        sh = [up(x) for x in sh_h]
        We, lg = up(We_h), up(lg_h)
        Xg = torch.cat(sh)
        Y = torch.empty((m.T * m.topk, m.I), dtype=torch.float32, device=dev)
        off = torch.empty(m.E + 1, dtype=torch.int32, device=dev)
        rt = torch.empty(m.T * m.topk, dtype=torch.int32, device=dev)
        ids = torch.empty((m.T, m.topk), dtype=torch.int32, device=dev)
        fl = torch.zeros(sgt.ag_flag_count(m.W, m.T, m.H), dtype=torch.int32, device=dev)

        def moe(i, ev):
            ctx.moe_ag_gemm(sh, We, lg, Xg, Y, off, rt, ids, fl, topk=m.topk, b_layout=lay, producer="preset",
                            consumer_events=ev)
        step, _, kern = timed(moe, args.steps, args.warmup, torch, ctx)
        res["moe_ag_grouped_preset"] = {"step_ms": step, "consumer_kernel_ms": spread(kern)}
        tables = (off, rt, ids)
        if name == "moe_rs":
            res["moe_gemm_rs"] = bench_moe_rs(ctx, up, args, torch, sgt, I, lay, tables, resident_only=True)
        if name == "a2a":
            # every AllToAll call is one stream's work (its senders run in the same launch or before it)
            res["a2a"] = bench_a2a(ctx, up, args, torch, sgt, I, tables)
    elif name == "gemm_rs":
        r = I.GEMM_RS
        A_h, B_h, parts_h = I.make_rs(r, B_layout=lay)
        A, B = up(A_h), up(B_h)
        parts = [up(p) if q != 0 else None for q, p in enumerate(parts_h)]
        ng, npf = sgt.rs_flag_count(r.W, r.M, r.N)
        P = torch.empty((r.M, r.N), dtype=torch.float32, device=dev)
        Cs = torch.empty((r.M // r.W, r.N), dtype=torch.float32, device=dev)
        gf = torch.zeros(ng, dtype=torch.int32, device=dev)
        pf = torch.zeros(npf, dtype=torch.int32, device=dev)
        step, _, kern = timed(lambda i, ev: ctx.gemm_rs(A, B, parts, P, Cs, gf, pf, rank=0, b_layout=lay,
                                                        consumer_events=ev), args.steps, args.warmup, torch, ctx)
        res["gemm_rs"] = {"step_ms": step, "kernel_ms": spread(kern)}
    elif name == "ring":
        res["ring"] = bench_ring(ctx, up, args, torch, sgt, I, resident_only=True)
    else:
        raise SystemExit("unknown kernel pass %r" % name)
    print(json.dumps(res), flush=True)


def bench_gemm_rs(ctx, up, args, torch, sgt, I, lay, rank):
    """GEMM + ReduceScatter on the Qwen-32B MLP share (M 8192, K 3200, N 5120, W 8): the call with the peers'
    partials resident, the same GEMM alone, interleaved pairs, the reduction window from the kernel's own
    stamps, and the call with the peers paced at 50 GB/s per link."""
    import numpy as np
    dev = "cuda:0"
    r = I.GEMM_RS
    A_h, Brs_h, parts_h = I.make_rs(r, B_layout=lay)
    A = up(A_h)
    Brs = up(Brs_h)
    parts = [up(p) if q != rank else None for q, p in enumerate(parts_h)]
    ng, npf = sgt.rs_flag_count(r.W, r.M, r.N)
    P = torch.empty((r.M, r.N), dtype=torch.float32, device=dev)
    Cs = torch.empty((r.M // r.W, r.N), dtype=torch.float32, device=dev)
    gf = torch.zeros(ng, dtype=torch.int32, device=dev)
    pf = torch.zeros(npf, dtype=torch.int32, device=dev)
    rs_ms, rs_kern_ms, _ = timed(lambda i, ev: ctx.gemm_rs(A, Brs, parts, P, Cs, gf, pf, rank=rank, b_layout=lay,
                                                           consumer_events=ev), args.steps, args.warmup, torch,
                                 ctx)
    # the same GEMM alone (no signalling epilogue, no reduction): the AllGather consumer on resident data
    A_shards = list(A.view(r.W, r.M // r.W, r.K).unbind(0))
    fl2 = torch.zeros(sgt.ag_flag_count(r.W, r.M, r.K), dtype=torch.int32, device=dev)
    Cg = torch.empty((r.M, r.N), dtype=torch.float32, device=dev)
    A_parts = [a.contiguous() for a in A_shards]
    g_ms, _, _ = timed(lambda i, ev: ctx.ag_gemm(A_parts, Brs, A, Cg, fl2, rank=rank, b_layout=lay,
                                                 producer="preset", consumer_events=ev), args.steps,
                       args.warmup, torch, ctx)
    # interleaved pairs: GEMM+RS call, then the same GEMM alone
    rs_l, g_l = pairs(lambda i, ev: ctx.gemm_rs(A, Brs, parts, P, Cs, gf, pf, rank=rank, b_layout=lay,
                                                consumer_events=ev),
                      lambda i, ev: ctx.ag_gemm(A_parts, Brs, A, Cg, fl2, rank=rank, b_layout=lay,
                                                producer="preset", consumer_events=ev), args.steps, torch, ctx)
    rs_pair, g_pair = statistics.median(rs_l), statistics.median(g_l)
    red_bytes = (r.M // r.W) * r.N * 4 * (r.W + 1)   # read local block + W-1 peers, write C_shard
    # reduction window from the kernel's own stamps (100 MHz clock): first reduction start to last end
    nw = sgt.rs_trace_words(r.W, r.M, r.N)
    tr = torch.zeros(nw, dtype=torch.int64, device=dev)
    ctx.gemm_rs(A, Brs, parts, P, Cs, gf, pf, rank=rank, b_layout=lay, trace=tr.data_ptr(), blocking=True)
    t = tr.cpu().numpy().view(np.uint64).reshape(-1, 3)
    n_g = (r.W * (-(-(r.M // r.W) // 256))) * (-(-r.N // 256))
    red_t, gem_t = t[n_g:].astype(np.int64), t[:n_g].astype(np.int64)
    red_win_us = (red_t[:, 1].max() - red_t[:, 0].min()) / 100.0
    red_item_us = (red_t[:, 1] - red_t[:, 0]) / 100.0
    # paced peers at 50 GB/s per link (the comm-bound variant): peers' blocks copied into an inbox
    gbps_rs = 50.0
    inbox = [torch.empty_like(p) if p is not None else None for p in parts]
    pc_ms, pc_k, pc_l = timed(lambda i, ev: ctx.gemm_rs_paced(A, Brs, parts, inbox, P, Cs, gf, pf, rank=rank,
                                                              b_layout=lay, peer_gbps=gbps_rs,
                                                              consumer_events=ev),
                              max(4, args.steps // 2), 2, torch, ctx)
    res = {
        "workload": r.name, "M": r.M, "K": r.K, "N": r.N, "W": r.W,
        "step_ms": rs_ms, "kernel_ms": rs_kern_ms,
        "tflops": r.flops / (rs_ms * 1e-3) / 1e12,
        "pct_peak": 100.0 * r.flops / (rs_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "gemm_alone_ms": g_ms,
        "overlap_efficiency": g_pair / rs_pair,
        "overlap_efficiency_note": "median kernel time of the GEMM alone over that of GEMM+RS, interleaved pairs",
        "overlap_efficiency_blocks": g_ms / rs_ms,
        "pairs_kernel_ms": spread(rs_l), "pairs_gemm_alone_kernel_ms": spread(g_l),
        "reduction_algorithmic_bytes": red_bytes,
        "reduction_window_us": float(red_win_us),
        "reduction_window_gbs": red_bytes / (red_win_us * 1e-6) / 1e9,
        "reduction_item_us": spread(red_item_us.tolist()),
        "reduction_note": "window = first reduction-item start to last end in one traced call (the items run "
                          "while other workgroups finish GEMM tiles, so the rate is a lower bound); an item is "
                          "a 32-row band of a 128 x 128 signal tile; its stamps cover its stream (the claim and "
                          "the flag peek of the next item overlap it)",
        "gemm_tiles_end_us": float((gem_t[:, 1].max() - gem_t[:, 0].min()) / 100.0),
        "paced_50gbps": {"peer_gbps": gbps_rs, "step_ms": pc_ms, "kernel_ms": spread(pc_l),
                         "tflops": r.flops / (pc_ms * 1e-3) / 1e12,
                         "link_floor_us": (r.M // r.W) * r.N * 4 / (gbps_rs * 1e9) * 1e6},
    }
    assert torch.equal(inbox[(rank + 1) % r.W], parts[(rank + 1) % r.W]), "paced inbox mismatch"
    del inbox, tr
    del A, Brs, parts, P, Cs, Cg
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rs", action="store_true", help="skip the GEMM+ReduceScatter workload")
    ap.add_argument("--rs-only", action="store_true", help="only the GEMM+ReduceScatter workload")
    ap.add_argument("--no-moe", action="store_true", help="skip the MoE AllGather + grouped GEMM workload")
    ap.add_argument("--no-ll", action="store_true", help="skip the low-latency AllGather comparison")
    ap.add_argument("--ll-only", action="store_true", help="only the low-latency AllGather comparison")
    ap.add_argument("--no-ring", action="store_true", help="skip the ring AllReduce")
    ap.add_argument("--ring-only", action="store_true", help="only the ring AllReduce")
    ap.add_argument("--no-a2a", action="store_true", help="skip the expert-parallel AllToAll")
    ap.add_argument("--a2a-only", action="store_true", help="only the expert-parallel AllToAll")
    ap.add_argument("--b-layout", default="nk", choices=["kn", "nk"],
                    help="B as N x K (a Linear layer's weight, default) or K x N")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only a plain 1 GiB device copy (counter calibration for the traffic figure)")
    ap.add_argument("--consumer-alone", action="store_true",
                    help="only the headline's consumer kernel on resident data with flags preset, on the grid the "
                         "overlapped call gives it (for counter passes, which serialize kernels and so cannot "
                         "run the overlapped call)")
    ap.add_argument("--kernel-pass", default=None, choices=["moe", "moe_rs", "gemm_rs", "ring", "a2a"],
                    help="only one workload's kernels with resident data and preset flags (for counter passes)")
    ap.add_argument("--moe-only", action="store_true", help="only the MoE AllGather and combine workloads")
    ap.add_argument("--engines-only", action="store_true",
                    help="only the headline's overlapped step with the CU producer and the copy-engine variants")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the overlapped steps (for a profiler run whose kernel list is exactly the timed one)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the tensor-parallel layer on one MI355X (the peers are "
              "simulated in its HBM); a run on %d GPUs is not supported" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import signal_gated_tiled_amd as sgt
    from signal_gated_tiled_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    if args.copy_calibration:
        copy_calibration(torch, max(1, args.steps))
        return

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    if args.kernel_pass:
        with sgt.Context(0) as c:
            kernel_pass(args.kernel_pass, c, up, args, torch, sgt, I, args.b_layout)
        return
    if args.moe_only:
        with sgt.Context(0) as c:
            moe, tables = bench_moe(c, up, args, torch, sgt, I, args.b_layout)
            print(json.dumps({"moe_ag_grouped": moe}), flush=True)
            print(json.dumps({"moe_gemm_rs": bench_moe_rs(c, up, args, torch, sgt, I, args.b_layout, tables)}),
                  flush=True)
        return
    if args.rs_only:
        with sgt.Context(0) as c:
            print(json.dumps({"gemm_rs": bench_gemm_rs(c, up, args, torch, sgt, I, args.b_layout, 0)}), flush=True)
        return
    if args.a2a_only:
        with sgt.Context(0) as c:
            print(json.dumps({"a2a": bench_a2a(c, up, args, torch, sgt, I, moe_routing(c, up, torch, sgt, I))}),
                  flush=True)
        return
    if args.ll_only or args.ring_only:
        with sgt.Context(0) as c:
            if args.ll_only:
                print(json.dumps({"ll_allgather": bench_ll(c, up, args, torch, sgt, I)}))
            else:
                print(json.dumps({"ring_allreduce": bench_ring(c, up, args, torch, sgt, I)}))
        return

    w = I.LLAMA_AG
    W, M, K, N = w.W, w.M, w.K, w.N
    lay = args.b_layout
    shards_h, B_h = I.make_ag(w, B_layout=lay)
    shards = [up(s) for s in shards_h]
    B = up(B_h)
    Ag = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    # signal tiles of one 256-row panel x one of K_CHUNKS column chunks of K: a tile whose panel is still
    # arriving starts on the chunks already in (the same bits as whole-row signal tiles)
    kc = K_CHUNKS if lay == "nk" else 0
    flags = torch.zeros(sgt.ag_flag_count(W, M, K, k_chunks=kc), dtype=torch.int32, device=dev)
    rank = 0
    flops = 2.0 * M * N * K
    ctx = sgt.Context(0)

    def ag(producer, **kw):
        def fn(i, ev):
            ctx.ag_gemm(shards, B, Ag, C, flags, rank=rank, b_layout=lay, producer=producer,
                        consumer_events=ev, k_chunks=kc, **kw)
        return fn

    link = dict(peer_gbps=w.peer_gbps, jitter_us=w.jitter_us)
    if args.consumer_alone:
        Ag.copy_(torch.cat(shards))
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        grid = n_cu - max(8, n_cu // 8)
        ms, kern_ms, _ = timed(ag("preset", consumer_cus=grid), args.steps, args.warmup, torch, ctx)
        print(json.dumps({"workload": w.name, "consumer_alone_ms": ms, "consumer_kernel_ms": kern_ms, "grid": grid,
                          "tflops": flops / (kern_ms * 1e-3) / 1e12}), flush=True)
        ctx.close()
        return
    # the instrumented block's calls also write a trace each, whose per-tile cycle counts give the engine clock
    # of exactly the calls the kernel times come from
    n_tr = sgt.trace_words(W, M, K, N, k_chunks=kc)
    over_tr = torch.zeros((args.steps, n_tr), dtype=torch.int64, device=dev)

    def over_fn(i, ev):
        tr = over_tr[i - args.warmup].data_ptr() if ev is not None else 0
        ag("cu", arrival_seed=i + 1, trace=tr, **link)(i, ev)
    over_ms, over_kern_ms, over_list = timed(over_fn, args.steps, args.warmup, torch, ctx)
    over_clock = trace_clocks(over_tr, (M // 256) * (-(-N // 256)))
    del over_tr
    over_host = spread(LAST_HOST_MS) if LAST_HOST_MS else None
    over_host_max = max(LAST_HOST_MS) if LAST_HOST_MS else None
    if args.headline_only:
        print(json.dumps({"workload": w.name, "overlapped_ms": over_ms, "consumer_kernel_ms": over_kern_ms,
                          "tflops": flops / (over_ms * 1e-3) / 1e12,
                          "clock_mhz": [round(c) if c else None for c in over_clock],
                          "host_call_ms": [round(h, 3) for h in LAST_HOST_MS]}), flush=True)
        ctx.close()
        return
    if args.engines_only:
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        a_ms, _, _ = timed(ag("preset", consumer_cus=n_cu - max(8, n_cu // 8)), args.steps, args.warmup, torch, ctx)
        rel = release_times(ctx, lambda i, tr: ctx.ag_gemm(shards, B, Ag, C, flags, rank=rank, b_layout=lay,
                                                           producer="cu", k_chunks=kc, arrival_seed=7000 + i,
                                                           trace=tr, **link),
                            sgt.trace_words(W, M, K, N, k_chunks=kc), (M // 256) * (-(-N // 256)), torch,
                            local_flags=sgt.ag_flag_count(W, M, K, k_chunks=kc) // W)
        out = {"cu_producer": {"step_ms": over_ms, "overlap_efficiency_step": a_ms / over_ms, **rel},
               "gemm_alone_ms": a_ms}
        out.update(bench_engines(ctx, shards, B, Ag, C, flags, rank, lay, kc, link, a_ms, flops, (W, M, K, N), args,
                                 torch, sgt))
        print(json.dumps(out), flush=True)
        ctx.close()
        return
    # board power and engine clocks while the overlapped call runs back to back
    power = power_under_load(lambda i, ev: ag("cu", arrival_seed=5000 + i, **link)(i, ev), torch, ctx)
    # the same consumer with data resident and flags preset, on all CUs and on the grid the overlapped
    # run leaves it (all CUs but the producer's); the better of the two is "the GEMM alone"
    alone_all = timed(ag("preset"), args.steps, args.warmup, torch, ctx)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    prod_wgs = max(8, n_cu // 8)
    alone_part = timed(ag("preset", consumer_cus=n_cu - prod_wgs), args.steps, args.warmup, torch, ctx)
    best = min((alone_all, n_cu), (alone_part, n_cu - prod_wgs), key=lambda x: x[0][0])
    (alone_ms, alone_kern_ms, _), alone_grid = best
    # Overlap efficiency from interleaved pairs: overlapped call, then the same consumer alone on the same grid.
    ov_list, al_list = pairs(lambda i, ev: ag("cu", arrival_seed=1000 + i, **link)(i, ev),
                             ag("preset", consumer_cus=alone_grid), args.steps, torch, ctx)
    ov_k, al_k = statistics.median(ov_list), statistics.median(al_list)
    serial_ms, _, _ = timed(lambda i, ev: ag("serial", arrival_seed=i + 1, **link)(i, ev), max(3, args.steps // 4),
                            2, torch, ctx)
    unthr_ms, _, _ = timed(ag("cu"), max(3, args.steps // 4), 2, torch, ctx)
    # the same overlapped call with whole-row signal tiles (flag_rows rows x all K), for comparison
    whole_ms = None
    if kc:
        flags_w = torch.zeros(sgt.ag_flag_count(W, M, K), dtype=torch.int32, device=dev)
        whole_ms, _, _ = timed(lambda i, ev: ctx.ag_gemm(shards, B, Ag, C, flags_w, rank=rank, b_layout=lay,
                                                         producer="cu", consumer_events=ev, arrival_seed=i + 1,
                                                         **link), args.steps, args.warmup, torch, ctx)
        del flags_w
    # correctness spot check of the last overlapped result against the gathered bits
    assert torch.equal(Ag.view(torch.int16), torch.cat(shards).view(torch.int16)), "gathered buffer mismatch"
    # when the last signal tile is released, from the call's in-kernel stamps (a few traced calls)
    rel = release_times(ctx, lambda i, tr: ctx.ag_gemm(shards, B, Ag, C, flags, rank=rank, b_layout=lay,
                                                       producer="cu", k_chunks=kc, arrival_seed=7000 + i,
                                                       trace=tr, **link),
                        sgt.trace_words(W, M, K, N, k_chunks=kc), (M // 256) * (-(-N // 256)), torch,
                        local_flags=sgt.ag_flag_count(W, M, K, k_chunks=kc) // W)
    # the engine clock of the same GEMM with the data resident (flags preset), on the grid it was timed on
    alone_clock = trace_clock(lambda i, tr: ctx.ag_gemm(shards, B, Ag, C, flags, rank=rank, b_layout=lay,
                                                        producer="preset", k_chunks=kc, consumer_cus=alone_grid,
                                                        trace=tr),
                              sgt.trace_words(W, M, K, N, k_chunks=kc), (M // 256) * (-(-N // 256)), torch, ctx)

    shard_bytes = (M // W) * K * 2
    link_floor_us = shard_bytes / (w.peer_gbps * 1e9) * 1e6
    tflops = flops / (over_ms * 1e-3) / 1e12
    kern_tflops = flops / (over_kern_ms * 1e-3) / 1e12
    # the engine clock over the instrumented block: each call's clock weighted by its kernel time
    pairs_ck = [(c, k) for c, k in zip(over_clock, over_list) if c]
    block_clock = sum(c * k for c, k in pairs_ck) / sum(k for _, k in pairs_ck) if pairs_ck else None
    n_tiles = (M // 256) * (-(-N // 256))

    def e_max(floor_us):
        # ceiling on E: the last panel's data cannot land before its link delivers it (the link floor; jitter
        # only delays releases), and then its tiles (side by side) still compute what depends on the last
        # signal tile: one tile time = T_alone * grid / tiles, or one K chunk of it with K-chunked tiles
        t_alone = al_k * 1e3
        t_tile = t_alone * alone_grid / n_tiles / (kc if kc else 1)
        return t_alone / max(t_alone, floor_us + t_tile)

    # the arrival sweep: unthrottled, the xGMI link rate and 50 GB/s, jitter up to one signal tile's link time
    sweep = []
    sweep_n = max(4, args.steps // 2)
    for gbps in (0.0, 153.6, 50.0):
        jit = (256 * K * 2) / (gbps * 1e9) * 1e6 if gbps else 0.0
        kw = dict(peer_gbps=gbps, jitter_us=jit)
        o_l, a_l = pairs(lambda i, ev: ag("cu", arrival_seed=3000 + i, **kw)(i, ev),
                         ag("preset", consumer_cus=alone_grid), sweep_n, torch, ctx)
        floor = shard_bytes / (gbps * 1e9) * 1e6 if gbps else 0.0
        sweep.append({"peer_gbps": gbps or None, "jitter_us": jit, "link_floor_us": floor,
                      "overlapped_kernel_ms": spread(o_l), "alone_kernel_ms": spread(a_l),
                      "tflops_median": flops / (statistics.median(o_l) * 1e-3) / 1e12,
                      "overlap_efficiency": statistics.median(a_l) / statistics.median(o_l),
                      "overlap_efficiency_max": e_max(floor)})
    engines = bench_engines(ctx, shards, B, Ag, C, flags, rank, lay, kc, link, alone_ms, flops, (W, M, K, N), args,
                            torch, sgt)
    # MALL-flushed (a 512 MiB scrub buffer written before each call) against warm back-to-back calls
    scrub = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    fl_n = max(4, args.steps // 2)
    cold = flushed(lambda i, ev: ag("cu", arrival_seed=4000 + i, **link)(i, ev), fl_n, torch, ctx, scrub)
    cold_alone = flushed(ag("preset", consumer_cus=alone_grid), fl_n, torch, ctx, scrub)
    del scrub
    clocks = device_clocks()
    B_kn = B.t().contiguous() if lay == "nk" else B
    micro = microbench(torch, Ag, B_kn, max(3, args.steps // 4))
    del B_kn

    # the step-level overlap efficiency (block-timed GEMM alone over the block-timed overlapped step) and its
    # ceiling from the measured last release: after it, the tiles of the last signal tile still run one chunk
    t_tail_ms = al_k * alone_grid / n_tiles / (kc if kc else 1)
    e_step = alone_ms / over_ms
    e_step_max = alone_ms / max(alone_ms, rel["last_release_us"] * 1e-3 + t_tail_ms)
    detail = {
        "overlap_efficiency_step": e_step,
        "overlap_efficiency_step_max": e_step_max,
        "release_trace": rel,
        "overlapped_ms": over_ms,
        "overlapped_kernel_ms": spread(over_list),
        "overlapped_host_call_ms": over_host,
        "overlapped_clock_mhz": block_clock,
        "power_under_load": power,
        "overlapped_clock_mhz_per_call": spread([c for c in over_clock if c]) if any(over_clock) else None,
        "traced_overlapped_clock_mhz": rel.get("clock_mhz"),
        "gemm_alone_clock_mhz": alone_clock,
        "clock_note": "engine clock from traced calls: each tile's s_memtime cycles over its 100 MHz duration "
                      "(median over tiles, then over 3 calls); it moves with the board's power state from call "
                      "to call and box to box",
        "overlapped_host_call_max_ms": over_host_max,
        "gemm_alone_ms": alone_ms,
        "gemm_alone_tflops": flops / (alone_ms * 1e-3) / 1e12,
        "gemm_alone_kernel_ms": alone_kern_ms,
        "gemm_alone_pct_peak": 100.0 * flops / (alone_kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "gemm_alone_grid": alone_grid,
        "gemm_alone_all_cus_ms": alone_all[0],
        "gemm_alone_consumer_grid_ms": alone_part[0],
        "serial_ms": serial_ms,
        "producer_only_ms_est": serial_ms - alone_all[0],
        "producer_only_note": "serial call (paced producer, then the consumer on all CUs) minus the GEMM alone on "
                              "all CUs",
        "unthrottled_producer_ms": unthr_ms,
        "overlapped_whole_row_signal_tiles_ms": whole_ms,
        "overlapped_whole_row_signal_tiles_tflops": flops / (whole_ms * 1e-3) / 1e12 if whole_ms else None,
        "overlap_efficiency_pairs": al_k / ov_k,
        "overlap_efficiency_pairs_max_nominal": e_max(link_floor_us),
        "overlap_efficiency_note": "step: block-timed GEMM alone (best grid) over the block-timed overlapped step, "
                                   "its maximum from the measured last release plus one chunk of a tile; pairs: "
                                   "median consumer-kernel times of %d interleaved pairs, its maximum from the "
                                   "nominal link floor" % args.steps,
        "pairs_overlapped_kernel_ms": spread(ov_list),
        "pairs_alone_kernel_ms": spread(al_list),
        "speedup_vs_serial": serial_ms / over_ms,
        "link_floor_us": link_floor_us,
        "peer_gbps": w.peer_gbps,
        "jitter_us": w.jitter_us,
        "pct_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "arrival_sweep": sweep,
        "copy_engine_producer": engines,
        "copy_engine_note": "SGT_PROD_SDMA: copy-engine copies of whole 256-row panels gated on the call's stream "
                            "position, a releaser workgroup publishing each K chunk's flag once its panel has "
                            "landed and its link time has come; the CU producer's last release is in "
                            "release_trace",
        "mall_flushed_call_ms": spread(cold),
        "mall_flushed_alone_call_ms": spread(cold_alone),
        "mall_flushed_tflops_median": flops / (statistics.median(cold) * 1e-3) / 1e12,
        "mall_flushed_overlap_efficiency": statistics.median(cold_alone) / statistics.median(cold),
        "mall_flushed_note": "whole call (producer fork to join) timed alone after writing a 512 MiB buffer",
        "rocm_smi_clocks": clocks,
        "microbench": micro,
    }

    if not args.no_rs:
        detail["gemm_rs"] = bench_gemm_rs(ctx, up, args, torch, sgt, I, lay, rank)

    detail["ag_other_workloads"] = bench_ag_other(ctx, up, args, torch, sgt, I, lay)
    if not args.no_ll:
        detail["ll_allgather"] = bench_ll(ctx, up, args, torch, sgt, I)
    if not args.no_ring:
        detail["ring_allreduce"] = bench_ring(ctx, up, args, torch, sgt, I)

    if not args.no_moe:
        detail["moe_ag_grouped"], tables = bench_moe(ctx, up, args, torch, sgt, I, lay)
        detail["moe_gemm_rs"] = bench_moe_rs(ctx, up, args, torch, sgt, I, lay, tables)
        if not args.no_a2a:
            detail["a2a"] = bench_a2a(ctx, up, args, torch, sgt, I, tables)
        del tables

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shards_h, B_h, M, N, K, args.cpu_seconds, b_layout=lay)
        cpu.pop("seconds", None)
        detail["cpu_oracle_host"] = cpu_host_details(I)

    # the full detail goes to a file and to earlier lines; the last line stays short (under 2 KB)
    detail_path = os.path.join(ROOT, "gpurun_out", "bench_detail.json")
    try:
        os.makedirs(os.path.dirname(detail_path), exist_ok=True)
        with open(detail_path, "w") as fh:
            json.dump(detail, fh, indent=1)
    except OSError:
        detail_path = None
    for k, v in detail.items():
        print(json.dumps({"detail": k, "value": v}), flush=True)
    rs = detail.get("gemm_rs") or {}
    moe = detail.get("moe_ag_grouped") or {}
    line = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": WARM_S,
        "ms_per_step": over_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "W": W, "M": M, "K": K, "N": N, "rank": rank, "b_layout": lay,
                   "k_chunks": kc, "peer_gbps": w.peer_gbps, "jitter_us": w.jitter_us, "out": "fp32"},
        "roofline": {"bound": "mfma", "kernel": "ag_consumer_bf16", "achieved": round(kern_tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(), "algorithmic_bytes": (M * K + K * N) * 2 + M * N * 4,
                     # the engine clock of traced overlapped calls (per-tile cycle counts over durations) and the
                     # fraction of the peak the chip has at that clock (256 CUs x 4096 flop per cycle)
                     "clock_mhz": round(block_clock) if block_clock else None,
                     "frac_at_clock": round(kern_tflops / (256 * 4096 * block_clock / 1e6), 4)
                     if block_clock else None,
                     # amd-smi under the same load: the package's power limit is what sets that clock
                     "board_power_w": power.get("socket_power_w") if power else None},
        "overlap": {"efficiency": round(e_step, 4), "efficiency_max": round(e_step_max, 4),
                    "last_release_us": round(rel["last_release_us"], 1), "link_floor_us": round(link_floor_us, 1),
                    "gemm_alone_ms": round(alone_ms, 4), "gemm_alone_tflops": round(flops / alone_ms / 1e9, 1)},
        "reduction": {"workload": rs.get("workload"), "gbs": round(rs["reduction_window_gbs"], 1) if rs else None,
                      "hbm_frac": round(rs["reduction_window_gbs"] / PEAK_HBM_GBS, 4) if rs else None,
                      "window_us": round(rs["reduction_window_us"], 1) if rs else None,
                      "step_ms": round(rs["step_ms"], 4) if rs else None},
        "moe_ag_grouped": {"step_ms": round(moe["step_ms"], 4),
                           "consumer_ms_resident": round(moe["preset_consumer_kernel_ms"], 4),
                           "mfma_frac_resident": round(moe["resident_consumer_mfma_frac"], 4)} if moe else None,
        "ll_allgather": {"ll_faster_up_to_tokens_per_rank":
                         detail.get("ll_allgather", {}).get("crossover", {}).get("ll_faster_up_to_tokens_per_rank")},
        "cpu_baseline": cpu,
        "detail_file": os.path.relpath(detail_path, ROOT) if detail_path else None,
    }
    ctx.close()
    text = json.dumps(line)
    for k in ("ll_allgather", "moe_ag_grouped", "reduction"):  # keep the line under 2 KB whatever it holds
        if len(text) < 2048:
            break
        line.pop(k, None)
        text = json.dumps(line)
    print(text, flush=True)


if __name__ == "__main__":
    main()
