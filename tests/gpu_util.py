"""Helpers for the GPU tests: host <-> device copies and the parity checks.

Tolerances (bf16 inputs, fp32 accumulation and output) are the ones the
workload definition fixes: every element within 1e-2 * (|ref| + 1) of the
fp64 oracle, and the relative Frobenius error at most 2e-3.  fp32 inputs use
1e-4 * (|ref| + 1) and 1e-5 (fp32 accumulation over K <= a few thousand terms
of O(1) values stays near 1e-6 relative).  bf16 outputs add the rounding of
the result, at most 2^-9 relative per element: 2^-8 |ref| + 1e-5 per element,
2.5e-3 relative Frobenius.
"""
from __future__ import annotations

import numpy as np
import torch

from signal_gated_tiled_amd import inputs as I

TOL_BF16 = dict(max_coef=1e-2, rel_fro=2e-3)
TOL_F32 = dict(max_coef=1e-4, rel_fro=1e-5)


def dev(a: np.ndarray, device="cuda:0") -> torch.Tensor:
    """numpy fp32 or bf16-bits array -> contiguous GPU tensor of the same bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> numpy (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def values(a: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def assert_close(gpu: np.ndarray, ref: np.ndarray, max_coef: float, rel_fro: float, what: str = ""):
    g = values(gpu)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), "%s: non-finite values" % what
    d = np.abs(g - ref)
    bound = max_coef * (np.abs(ref) + 1.0)
    bad = d > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements over the bound, first at %s: gpu %r ref %r" %
                             (what, int(bad.sum()), tuple(i), g[tuple(i)], ref[tuple(i)]))
    nref = np.linalg.norm(ref)
    rf = np.linalg.norm(g - ref) / (nref if nref > 0 else 1.0)
    assert rf <= rel_fro, "%s: relative Frobenius error %.3e > %.1e" % (what, rf, rel_fro)
    return rf


def assert_close_bf16_out(gpu_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    g = values(gpu_bits)
    assert np.isfinite(g).all(), what
    d = np.abs(g - ref)
    assert (d <= 2.0 ** -8 * np.abs(ref) + 1e-5).all(), "%s: bf16 output off by more than its rounding" % what
    rf = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rf <= 2.5e-3, "%s: relative Frobenius %.3e" % (what, rf)


def poison_like(t: torch.Tensor) -> torch.Tensor:
    """Fill with quiet-NaN bit patterns (so an early read shows as NaN)."""
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(0x7FC0)
    else:
        t.view(torch.int32).fill_(0x7FC00000)
    return t


def sample_rows(M: int, W: int, per_shard: int = 4, seed: int = 0):
    """A few rows of every shard: first, last, and random ones."""
    rng = np.random.default_rng(seed)
    R = M // W
    rows = []
    for p in range(W):
        rows += [p * R, p * R + R - 1]
        rows += list(p * R + rng.integers(0, R, size=max(0, per_shard - 2)))
    return np.array(sorted(set(int(r) for r in rows)), dtype=np.int64)
