"""Helpers shared by the GPU parity tests (plumbing only: no attention math)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

TOL_F32 = 1e-4   # max-abs error for fp32 inputs
TOL_BF16 = 2e-2  # max-abs error for bf16 inputs with fp32 accumulation


def tol_bf16_scaled(ref) -> float:
    """Bound for bf16-input outputs whose reference exceeds 1 in magnitude: 2e-2 times that
    magnitude (equal absolute and relative tolerance, the convention of the RL-Kernel linear
    logp runbook's bf16 gate against an fp32-accumulation reference, "Reading Output").
    The kernels round P and dS to bf16 before their fp32-accumulating products, so their
    error grows with the output's own scale; for outputs within [-1, 1] this is TOL_BF16."""
    return TOL_BF16 * max(1.0, float(np.abs(np.asarray(ref)).max()))


def per_head(fn, heads, workers: int | None = None):
    """[fn(h) for h in heads], run in a thread pool with one BLAS thread per call: numpy
    releases the interpreter lock in its array loops, so independent heads of the fp64
    oracle run in parallel on the host's cores."""
    from threadpoolctl import threadpool_limits
    n = workers or min(16, len(os.sched_getaffinity(0)), len(heads))
    with threadpool_limits(1), ThreadPoolExecutor(max(1, n)) as ex:
        return list(ex.map(fn, heads))


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().double().numpy()


def gather(x: torch.Tensor, positions, dev="cuda") -> torch.Tensor:
    """Local shard of a global [B,H,T,D] tensor: rows at ``positions``, contiguous, on the GPU."""
    idx = torch.as_tensor(list(positions), dtype=torch.long)
    return x.index_select(2, idx).contiguous().to(dev)


def max_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    if (np.isneginf(got) != np.isneginf(ref)).any():
        return float("inf")
    d = np.abs(np.where(both_inf, 0.0, got) - np.where(both_inf, 0.0, ref))
    return float(d.max()) if d.size else 0.0
