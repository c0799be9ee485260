"""The ring schedule of context-parallel attention, assembled in fp64.

Source: BluScriptCP development log, entry of 2026-03-20 (ring rotator,
per-step SDPA, merger, forward and backward) and the 2026-03-21 / 2026-05-07
entries on the backward (dQ stays local, dK/dV accumulate as their block
travels, an accumulator must never be cleared between steps).

Each rank holds the query rows of its shard. At ring step s it holds the KV
block of rank src(s); it computes block attention at global positions and
folds the partial result into its running (O, LSE) with the log-sum-exp merge.
The backward recomputes each block with the final LSE and D (see
``attention.block_attention_bwd``) and accumulates dQ per rank and dK/dV per
block owner.

These functions take an arbitrary assignment of global positions to ranks and
an arbitrary block order, so the invariant tests can check that every chunk
partition and every ring order reproduces unsharded attention.
"""
from __future__ import annotations

import numpy as np

from .attention import block_attention_bwd, block_attention_fwd
from .merge import lse_merge


def ring_forward(q, k, v, assignment, rank, order=None, scale=None):
    """Rank ``rank``'s share: O, LSE for its rows (global tensors [..., T, D]).

    ``assignment[r]`` lists the global positions rank r holds, in local order.
    ``order`` lists the owners of the KV blocks in the order they are seen
    (default: the ring, rank, rank-1, ...).
    """
    n = len(assignment)
    order = [(rank - s) % n for s in range(n)] if order is None else order
    qpos = np.asarray(assignment[rank])
    ql = np.take(np.asarray(q, np.float64), qpos, axis=-2)
    o = lse = None
    for src in order:
        kpos = np.asarray(assignment[src])
        kl = np.take(np.asarray(k, np.float64), kpos, axis=-2)
        vl = np.take(np.asarray(v, np.float64), kpos, axis=-2)
        ob, lb = block_attention_fwd(ql, kl, vl, qpos, kpos, causal=True, scale=scale)
        if o is None:
            o, lse = ob, lb
        else:
            o, lse = lse_merge(o, lse, ob, lb)
    return o, lse


def ring_backward(q, k, v, do, assignment, scale=None):
    """All ranks' shares of the backward; returns global-order dq, dk, dv.

    Runs the forward for every rank first (final O, LSE), then for each rank
    and each ring step adds the block gradients into dq (the rank's rows) and
    into dk, dv of the block owner's rows.
    """
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    n = len(assignment)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for r in range(n):
        qpos = np.asarray(assignment[r])
        o, lse = ring_forward(q, k, v, assignment, r, scale=scale)
        ql, dol = np.take(q, qpos, axis=-2), np.take(do, qpos, axis=-2)
        for s in range(n):
            src = (r - s) % n
            kpos = np.asarray(assignment[src])
            kl, vl = np.take(k, kpos, axis=-2), np.take(v, kpos, axis=-2)
            gq, gk, gv = block_attention_bwd(ql, kl, vl, dol, o, lse, qpos, kpos,
                                             causal=True, scale=scale)
            dq[..., qpos, :] += gq
            dk[..., kpos, :] += gk
            dv[..., kpos, :] += gv
    return dq, dk, dv
