"""Helpers shared by the GPU parity tests (plumbing only: no attention math)."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL_F32 = 1e-4   # max-abs error for fp32 inputs
TOL_BF16 = 2e-2  # max-abs error for bf16 inputs with fp32 accumulation


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
