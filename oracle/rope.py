"""Rotary position embedding at global positions, in fp64.

Source: BluScriptCP development log, entries of 2026-06-29 (the rotary table
must follow each token's global position under load balancing; keys carry
their positions around the ring) and 2026-07-02 (Llama-style fused rotary),
and the 2026-06-05 entries on global positions per rank. Reading: the
half-split form, where dimension i is paired with i + D/2 for i < D/2, with
frequency theta^(-2i/D); no YaRN scaling (scale 1).

    (x_i, x_{i+D/2}) -> (x_i cos a - x_{i+D/2} sin a,  x_{i+D/2} cos a + x_i sin a)
    a = pos * theta^(-2i/D)

Backward through the rotary (the next step after the rotated forward: gradients
of q and k come back through the transposed rotation, R(p)^T): each pair
rotation is orthogonal, so its transpose is the rotation by -a:

    (g_i, g_{i+D/2}) -> (g_i cos a + g_{i+D/2} sin a,  g_{i+D/2} cos a - g_i sin a)
"""
from __future__ import annotations

import numpy as np

from . import attention


def rope_angles(pos, D: int, theta: float):
    pos = np.asarray(pos, dtype=np.float64)
    i = np.arange(D // 2, dtype=np.float64)
    inv = np.power(float(theta), -2.0 * i / D)
    return pos[:, None] * inv[None, :]


def rope_apply(x, pos, theta: float):
    """Rotate ``x`` [..., T, D] whose rows sit at global positions ``pos`` [T]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    a = rope_angles(pos, D, theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_apply_transpose(g, pos, theta: float):
    """R(pos)^T applied to ``g`` [..., T, D]: the gradient with respect to the
    unrotated rows, given the gradient ``g`` with respect to the rotated rows."""
    g = np.asarray(g, dtype=np.float64)
    D = g.shape[-1]
    a = rope_angles(pos, D, theta)
    c, s = np.cos(a), np.sin(a)
    g1, g2 = g[..., : D // 2], g[..., D // 2:]
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)


def rope_attention_bwd(q, k, v, do, theta: float, scale=None):
    """Gradients of causal attention over rotated queries and keys (all tokens in
    global order, position = index): attention backward on R q and R k, then the
    q and k gradients taken back through R^T."""
    pos = np.arange(np.asarray(q).shape[-2])
    qr, kr = rope_apply(q, pos, theta), rope_apply(k, pos, theta)
    dqr, dkr, dv, _, _ = attention.causal_attention_bwd(qr, kr, v, do, scale=scale)
    return rope_apply_transpose(dqr, pos, theta), rope_apply_transpose(dkr, pos, theta), dv
