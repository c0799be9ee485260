"""Rotary position embedding at global positions, in fp64.

Source: BluScriptCP development log, entries of 2026-06-29 (the rotary table
must follow each token's global position under load balancing; keys carry
their positions around the ring) and 2026-07-02 (Llama-style fused rotary),
and the 2026-06-05 entries on global positions per rank. Reading: the
half-split form, where dimension i is paired with i + D/2 for i < D/2, with
frequency theta^(-2i/D); no YaRN scaling (scale 1).

    (x_i, x_{i+D/2}) -> (x_i cos a - x_{i+D/2} sin a,  x_{i+D/2} cos a + x_i sin a)
    a = pos * theta^(-2i/D)
"""
from __future__ import annotations

import numpy as np


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
