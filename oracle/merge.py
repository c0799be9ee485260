"""Log-sum-exp merge of two partial attention results, in fp64.

Source: BluScriptCP development log, entry of 2026-03-20 (SDPAMerger, part of
the first context-parallel implementation) and entry of 2026-05-20 (partial
merge of a row range). The formula is not printed on the pages; it is the
standard log-sum-exp combination, the same combination the RL-Kernel linear
logp runbook uses when its forward merges a global log-sum-exp across shards
(runbook introduction).

For partial results (O_a, L_a) and (O_b, L_b) over disjoint key sets:

    L = log(exp(L_a) + exp(L_b))
    O = exp(L_a - L) O_a + exp(L_b - L) O_b

A side with L = -inf (no visible key) is the identity; if both are -inf the
result is (0, -inf).
"""
from __future__ import annotations

import numpy as np


def lse_merge(o_a, lse_a, o_b, lse_b):
    o_a, lse_a = np.asarray(o_a, np.float64), np.asarray(lse_a, np.float64)
    o_b, lse_b = np.asarray(o_b, np.float64), np.asarray(lse_b, np.float64)
    m = np.maximum(lse_a, lse_b)
    dead = ~np.isfinite(m)
    ms = np.where(dead, 0.0, m)
    ea = np.exp(lse_a - ms)
    eb = np.exp(lse_b - ms)
    tot = ea + eb
    with np.errstate(divide="ignore"):
        lse = np.where(dead, -np.inf, ms + np.log(np.where(dead, 1.0, tot)))
    wa = np.where(dead, 0.0, ea / np.where(dead, 1.0, tot))
    wb = np.where(dead, 0.0, eb / np.where(dead, 1.0, tot))
    o = wa[..., None] * o_a + wb[..., None] * o_b
    return o, lse
