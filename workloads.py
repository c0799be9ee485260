"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module only names shapes and draws random numbers. It holds none of the
attention arithmetic, so both the HIP path and the fp64 oracle can take their
inputs from it without sharing any of the method.

Workloads (global token order, all inputs i.i.d. N(0, 1)):

  tiny      B=1 H=4  D=64  T=256   ring degree 2, fp32 inputs
  gpt2s     B=4 H=12 D=64  T=4096  ring degree 4, bf16 inputs (GPT-2-small heads)
  win16k    B=1 H=32 D=128 T=16384 ring degree 2, bf16 inputs
  win32k    B=1 H=16 D=128 T=32768 ring degree 2, bf16 inputs, rotary theta 10000
  bwd16k    B=1 H=32 D=128 T=16384 ring degree 2, bf16 inputs, upstream dO drawn too
  gqa16k    the 16k window with 8 KV heads shared by groups of 4 query heads
            (grouped-query attention, the next row after the hot path), dO drawn

Seeds are 1234 + k for the k-th workload in that order; 1234 is the init seed
used throughout the BluScriptCP development log (entry of 2026-06-05 on the
named-weight init files).

bf16 inputs are drawn in fp32 and rounded to bf16 with round-to-nearest-even
(torch's cast). Every consumer -- kernel and oracle alike -- receives the
rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    D: int
    T: int
    ring: int
    dtype: str  # "f32" or "bf16"
    rope_theta: float = 0.0
    backward: bool = False
    note: str = ""
    H_kv: int = 0  # KV heads (0: one per query head)

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def seed(self) -> int:
        return 1234 + self.index

    @property
    def chunk(self) -> int:
        """Tokens per chunk when the sequence is cut into 2 * ring chunks."""
        return self.T // (2 * self.ring)

    @property
    def local_len(self) -> int:
        """Tokens each rank holds (two chunks)."""
        return 2 * self.chunk

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = [
    Workload("tiny", 0, B=1, H=4, D=64, T=256, ring=2, dtype="f32",
             note="4 chunks of 64 tokens; both ranks' shares"),
    Workload("gpt2s", 1, B=4, H=12, D=64, T=4096, ring=4, dtype="bf16",
             note="GPT-2-small heads; 8 chunks of 512; rank 0's share"),
    Workload("win16k", 2, B=1, H=32, D=128, T=16384, ring=2, dtype="bf16",
             note="16k window; 4 chunks of 4096; rank 0's share"),
    Workload("win32k", 3, B=1, H=16, D=128, T=32768, ring=2, dtype="bf16", rope_theta=10000.0,
             note="32k window with rotary at global positions; one head share of 32"),
    Workload("bwd16k", 4, B=1, H=32, D=128, T=16384, ring=2, dtype="bf16", backward=True,
             note="16k window forward + backward; all ranks' shares"),
    Workload("gqa16k", 5, B=1, H=32, D=128, T=16384, ring=2, dtype="bf16", backward=True, H_kv=8,
             note="16k window, grouped-query attention with 8 KV heads (groups of 4)"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def draw(w: Workload, heads: slice | None = None, seed: int | None = None):
    """Draw (q, k, v[, do]) for workload ``w`` as CPU tensors [B, H, T, D].

    The tensors are drawn in fp32 from ``torch.Generator`` seeded with
    ``w.seed`` (or ``seed``) in the order q, k, v, do, then rounded to the
    workload dtype; k and v have ``w.kv_heads`` heads. ``heads`` selects a
    head range after drawing, so a subset has exactly the values of the full
    draw.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    names = ["q", "k", "v"] + (["do"] if w.backward else [])
    out = {}
    for n in names:
        shape = (w.B, w.kv_heads if n in ("k", "v") else w.H, w.T, w.D)
        t = torch.randn(shape, dtype=torch.float32, generator=g)
        t = t.to(w.torch_dtype)
        if heads is not None:
            t = t[:, heads].contiguous()
        out[n] = t
    return out


def draw_shape(B: int, H: int, T: int, D: int, dtype=torch.float32, seed: int = 0,
               n: int = 3, scale: float = 1.0):
    """Draw ``n`` i.i.d. N(0, scale^2) tensors of shape [B, H, T, D] (test cases of any size)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return [(torch.randn((B, H, T, D), dtype=torch.float32, generator=g) * scale).to(dtype)
            for _ in range(n)]
