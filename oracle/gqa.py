"""Grouped-query attention (GQA / MQA) in fp64: KV heads shared by groups of
query heads.

Source: BluScriptCP development log, entries of 2026-06-29 (keep the
GQA-grouped KV in the ring), 2026-07-01 (GQA/MQA with nkv < nq; the dK/dV
group reduce is an explicit sum over the query heads of a group) and
2026-07-06 (query head hq uses KV head hq / G, G = nq / nkv; dQ is per query
head and needs no reduce).

With H query heads and H_kv KV heads (G = H / H_kv), query head h attends with
KV head h // G. The forward is plain attention against the KV head of its
group. The gradient of a shared K or V head is the sum, over the G query heads
of its group, of the per-head gradients.
"""
from __future__ import annotations

import numpy as np

from . import attention


def group_size(H: int, H_kv: int) -> int:
    if H_kv <= 0 or H % H_kv:
        raise ValueError("H must be a positive multiple of H_kv")
    return H // H_kv


def expand_kv(x, H: int):
    """[B, H_kv, T, D] -> [B, H, T, D]: KV head j serves query heads j*G .. j*G+G-1."""
    x = np.asarray(x, dtype=np.float64)
    return np.repeat(x, group_size(H, x.shape[1]), axis=1)


def reduce_groups(g, H_kv: int):
    """[B, H, T, D] per-query-head gradients -> [B, H_kv, T, D] sums over each group."""
    g = np.asarray(g, dtype=np.float64)
    B, H, T, D = g.shape
    G = group_size(H, H_kv)
    return g.reshape(B, H_kv, G, T, D).sum(axis=2)


def block_attention_fwd(q, k, v, qpos, kpos, causal=True, scale=None):
    H = np.asarray(q).shape[1]
    return attention.block_attention_fwd(q, expand_kv(k, H), expand_kv(v, H), qpos, kpos, causal=causal, scale=scale)


def block_attention_bwd(q, k, v, do, o, lse, qpos, kpos, causal=True, scale=None):
    """(dq, dk, dv) of one block for the final (o, lse); dk and dv per KV head."""
    H, H_kv = np.asarray(q).shape[1], np.asarray(k).shape[1]
    dq, dk, dv = attention.block_attention_bwd(q, expand_kv(k, H), expand_kv(v, H), do, o, lse, qpos, kpos,
                                               causal=causal, scale=scale)
    return dq, reduce_groups(dk, H_kv), reduce_groups(dv, H_kv)


def causal_attention_bwd(q, k, v, do, scale=None):
    """Full-sequence GQA gradients (global order): dq per query head, dk / dv per KV head."""
    H, H_kv = np.asarray(q).shape[1], np.asarray(k).shape[1]
    dq, dk, dv, o, lse = attention.causal_attention_bwd(q, expand_kv(k, H), expand_kv(v, H), do, scale=scale)
    return dq, reduce_groups(dk, H_kv), reduce_groups(dv, H_kv), o, lse
