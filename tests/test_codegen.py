"""Checks on the built gfx950 code object (CPU only; reads the AMD assembly of this library's own build).

A tile kernel whose matrix-core loop the compiler has dropped (for instance
after undefined behaviour in a compile-time schedule) still links and runs,
but computes nothing; counting the MFMAs of each tile kernel catches that
without a GPU.  The same pass checks that no kernel writes through the scalar
data cache.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

import signal_gated_tiled_amd as sgt

OBJDUMP = shutil.which("llvm-objdump") or "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(sgt.LIB_PATH):
        pytest.skip("libsgt.so is not built")
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not found")
    d = tmp_path_factory.mktemp("codeobj")
    lib = str(d / "libsgt.so")
    shutil.copy(sgt.LIB_PATH, lib)
    subprocess.run([OBJDUMP, "--offloading", lib], cwd=str(d), check=True, capture_output=True)
    objs = [str(d / f) for f in os.listdir(d) if f.endswith("gfx950")]
    assert objs, "no gfx950 code object in libsgt.so"
    funcs = {}
    for o in objs:
        txt = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn", o], check=True, capture_output=True,
                             text=True).stdout
        name = None
        for line in txt.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
            if m:
                name = m.group(1)
                funcs.setdefault(name, [])
            elif name is not None and line.strip():
                funcs[name].append(line.strip())
    return funcs


def _tile_shape(name):
    """(waves, rows) of a tile kernel from its mangled template arguments, or None."""
    m = re.search(r"(ag_consumer_bf16|gemm_rs_kernel)ILi(\d)E", name)
    if m:
        return int(m.group(2)), 256
    m = re.search(r"moe_consumer_bf16ILi(\d)ELi(\d+)E", name)
    if m:
        return int(m.group(1)), int(m.group(2))
    if re.search(r"moe_rs_kernelILb", name):
        return 8, 256
    return None


def test_every_tile_kernel_keeps_its_mfma_loop(kernels):
    seen = 0
    for name, body in kernels.items():
        shape = _tile_shape(name)
        if shape is None:
            continue
        kw, kr = shape
        mi = kr // (kw // 2) // 32
        n = sum(1 for ln in body if ln.startswith("v_mfma_f32_32x32x16_bf16"))
        # the K loop is unrolled over the two LDS stages: 2 x 4 substeps x (MI x 4) MFMAs, or over five steps
        # on the five-slot ring (the 8-wave tiles with both operands stored k-contiguous in the AllGather and
        # MoE consumers); the AllGather consumer's ring tile holds two K loops (a whole panel at once, or K
        # chunk by K chunk); the MoE consumer with 256-row tiles holds a 256-row and a 128-row loop (the
        # short tail of a group)
        ring = "ag_consumer_bf16ILi8ELb1E" in name or re.search(r"moe_consumer_bf16ILi8ELi\d+ELb1E", name)
        steps = 5 if ring else 2
        want = (2 if "ag_consumer" in name and ring else 1) * steps * 4 * mi * 4
        if "moe_consumer_bf16" in name and kr == 256:
            want += steps * 4 * (128 // (kw // 2) // 32) * 4
        assert n == want, "%s: %d MFMAs, expected %d" % (name, n, want)
        seen += 1
    # 8 AllGather, 16 MoE, 4 GEMM+RS and 4 MoE combine (B layout x Y dtype) instantiations
    assert seen == 32, seen


def test_no_scalar_cache_writes(kernels):
    bad = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")
    for name, body in kernels.items():
        hits = [ln for ln in body if bad.match(ln)]
        assert not hits, "%s: %s" % (name, hits[:3])


def test_copy_loops_keep_their_loads_in_flight(kernels):
    # A copy is latency-bound: each pass must issue all of its 16-byte loads
    # before its first store.  (Left to itself the scheduler pairs every store
    # with its load, which halves a producer workgroup's bandwidth.)
    want = {"ag_producer_kernel": 32, "ag_allgather_kernel": 32, "ll_allgather_kernel": 8}
    found = set()
    for name, body in kernels.items():
        key = next((k for k in want if k in name), None)
        if key is None:
            continue
        found.add(key)
        run = best = 0
        for ln in body:
            if ln.startswith("buffer_load_dwordx4"):
                run += 1
            elif ln.startswith("buffer_store_dwordx4"):
                best = max(best, run)
                run = 0
        assert best >= want[key], "%s: at most %d loads before a store" % (name, best)
    assert found == set(want), found
