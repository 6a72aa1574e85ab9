"""Shared helpers for the GPU tests: host <-> device copies and the workloads.

The workload shapes are those of the pages' examples (MSLK Kernel Library --
Complete Reference, Quick start: a causal [2, 2048, 32, 128] bf16 forward and a
2-way split of a [1, 1024, 16, 128] K/V with 128 queries) plus the decode and
packed-sequence cases built on the same API.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from transformer_attention_02_amd import synth

TOL_BF16_OUT = 2e-2   # max |out - oracle| for bf16 outputs
TOL_LSE = 1e-3        # max |lse - oracle| for the fp32 LSE of bf16 inputs
TOL_F32 = 1e-5        # max error of every output of the fp32 path
# bf16 gradients: a per-element worst-case bound derived from the kernels' arithmetic
# (tests/bwd_bound.py)
# fp32 gradients: fp32 throughout, so the sums' rounding only (bounded by the largest terms)
TOL_BWD_F32 = 1e-5    # max |grad - oracle| <= TOL_BWD_F32 * (1 + max|oracle|)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload generated host data (uint16 bf16 bits or float32) unchanged."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def maxerr(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d))) if d.size else 0.0


def varlen_workload(seed=5, n=8, lo=256, hi=4096, G=8, Hg=4, D=128):
    """Packed causal prefill: lengths ~ U[lo, hi], q [1,M,G,Hg,D], base k/v [1,M,G,1,D] (bf16 bits)."""
    lens = synth.varlen_lengths(seed, n, lo, hi)
    ss = synth.seqstarts(lens)
    M = int(ss[-1])
    q = synth.normal(seed, synth.TAG_Q, (1, M, G, Hg, D), "bf16")
    kb = synth.normal(seed, synth.TAG_K, (1, M, G, 1, D), "bf16")
    vb = synth.normal(seed, synth.TAG_V, (1, M, G, 1, D), "bf16")
    return lens, ss, q, kb, vb


def f64_threads(x: np.ndarray, dtype: str = "bf16", workers: int = 16) -> np.ndarray:
    """synth.to_f64 of a large array, split over threads along its first axis of extent > 1
    (numpy's conversions release the GIL); exact, like synth.to_f64 itself."""
    from concurrent.futures import ThreadPoolExecutor

    x = np.asarray(x)
    out = np.empty(x.shape, dtype=np.float64)
    ax = next((i for i, n in enumerate(x.shape) if n > 1), 0)
    n = x.shape[ax] if x.ndim else 1
    parts = max(1, min(workers, n))
    bounds = [(n * i // parts, n * (i + 1) // parts) for i in range(parts)]

    def one(ab):
        sl = (slice(None),) * ax + (slice(*ab),)
        out[sl] = synth.to_f64(x[sl], dtype)

    with ThreadPoolExecutor(parts) as ex:
        list(ex.map(one, bounds))
    return out
