"""Pure-Python loop versions for tiny inputs (T <= 16, D <= 8).

These restate the same definitions with scalar loops, ``math.exp`` and
``math.fsum`` -- no numpy -- so that the vectorised oracle can be checked
against an implementation that shares none of its code paths. Inputs are
nested lists [T][D] of floats (one head).
"""
from __future__ import annotations

import math


def attention(q, k, v, qpos, kpos, causal=True, scale=None):
    D = len(q[0])
    sig = 1.0 / math.sqrt(D) if scale is None else scale
    O, L = [], []
    for p in range(len(q)):
        vis = [j for j in range(len(k)) if (not causal) or kpos[j] <= qpos[p]]
        if not vis:
            O.append([0.0] * len(v[0]))
            L.append(-math.inf)
            continue
        s = {j: sig * math.fsum(q[p][d] * k[j][d] for d in range(D)) for j in vis}
        m = max(s.values())
        lse = m + math.log(math.fsum(math.exp(s[j] - m) for j in vis))
        w = {j: math.exp(s[j] - lse) for j in vis}
        O.append([math.fsum(w[j] * v[j][d] for j in vis) for d in range(len(v[0]))])
        L.append(lse)
    return O, L


def merge(oa, la, ob, lb):
    O, L = [], []
    for p in range(len(oa)):
        if la[p] == -math.inf and lb[p] == -math.inf:
            O.append([0.0] * len(oa[p]))
            L.append(-math.inf)
            continue
        m = max(la[p], lb[p])
        lse = m + math.log(math.exp(la[p] - m) + math.exp(lb[p] - m))
        wa, wb = math.exp(la[p] - lse), math.exp(lb[p] - lse)
        O.append([wa * oa[p][d] + wb * ob[p][d] for d in range(len(oa[p]))])
        L.append(lse)
    return O, L


def rope(x, pos, theta):
    D = len(x[0])
    h = D // 2
    out = []
    for t, row in enumerate(x):
        r = list(row)
        for i in range(h):
            a = pos[t] * theta ** (-2.0 * i / D)
            c, s = math.cos(a), math.sin(a)
            r[i] = row[i] * c - row[i + h] * s
            r[i + h] = row[i + h] * c + row[i] * s
        out.append(r)
    return out
