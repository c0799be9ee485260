"""Causal softmax attention in fp64: forward (O, LSE) and analytic backward.

Written from the definition of scaled dot-product attention with a causal mask
expressed in GLOBAL token positions, which is what each ring step of context
parallel attention computes (BluScriptCP development log, entry of 2026-04-20
on the CP-aware attention kernels with separate query/key lengths and offsets,
and entry of 2026-06-29 listing the dual-offset global-causal mask and the
log-sum-exp as an output among the kernel requirements).

Conventions (readings where the pages are silent):
  * scale sigma = 1/sqrt(D) unless given; no dropout, bias or window;
  * key j is visible from query p iff pos_k[j] <= pos_q[p] (self included; the
    log's 2026-06-05 entries note that position 0 attends only to itself);
  * LSE is the natural-log log-sum-exp of the scaled scores of visible keys;
  * a row with no visible key yields O = 0 and LSE = -inf.

All arithmetic is float64 numpy: one matmul for the scores, exp, one matmul
for the weighted sum. Work is blocked over query rows only so that long
sequences fit in memory; nothing else is reordered.
"""
from __future__ import annotations

import math

import numpy as np

_ROWS = 512  # query rows per block (memory only)


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _scale(D, scale):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def block_attention_fwd(q, k, v, qpos, kpos, causal=True, scale=None):
    """Attention of queries ``q`` [..., Tq, D] over keys/values ``k``, ``v`` [..., Tk, D].

    ``qpos`` [Tq] and ``kpos`` [Tk] are global positions. Returns
    (O [..., Tq, D], LSE [..., Tq]) in float64.

        s_pj  = sigma * q_p . k_j            for visible j
        LSE_p = log sum_j exp(s_pj)
        O_p   = sum_j exp(s_pj - LSE_p) v_j
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    lead = q.shape[:-2]
    Tq, D = q.shape[-2:]
    Tk = k.shape[-2]
    sig = _scale(D, scale)
    qf = q.reshape(-1, Tq, D)
    kf = k.reshape(-1, Tk, D)
    vf = v.reshape(-1, Tk, v.shape[-1])
    O = np.zeros((qf.shape[0], Tq, vf.shape[-1]), dtype=np.float64)
    L = np.full((qf.shape[0], Tq), -np.inf, dtype=np.float64)
    for n in range(qf.shape[0]):
        for r0 in range(0, Tq, _ROWS):
            r1 = min(Tq, r0 + _ROWS)
            s = sig * (qf[n, r0:r1] @ kf[n].T)
            if causal:
                s[kpos[None, :] > qpos[r0:r1, None]] = -np.inf
            m = s.max(axis=1)
            live = np.isfinite(m)
            if not live.any():
                continue
            sl = s[live]
            ml = m[live]
            e = np.exp(sl - ml[:, None])
            lse = ml + np.log(e.sum(axis=1))
            p = np.exp(sl - lse[:, None])
            idx = np.nonzero(live)[0] + r0
            L[n, idx] = lse
            O[n, idx] = p @ vf[n]
    return O.reshape(lead + (Tq, vf.shape[-1])), L.reshape(lead + (Tq,))


def causal_attention_fwd(q, k, v, rows=None, scale=None):
    """Full-sequence causal attention of the global sequence, for query ``rows``.

    ``q``, ``k``, ``v`` are [..., T, D] in global token order; ``rows`` lists
    the global query positions wanted (default: all). Returns O, LSE for those
    rows in the order given.
    """
    T = q.shape[-2]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    return block_attention_fwd(np.take(_as64(q), rows, axis=-2), k, v, rows, np.arange(T),
                               causal=True, scale=scale)


def block_attention_bwd(q, k, v, do, o, lse, qpos, kpos, causal=True, scale=None):
    """Analytic gradients of one query block against one key block.

    ``o`` and ``lse`` are the FINAL (fully merged) output and log-sum-exp of
    the query rows, so that P below are the global softmax probabilities
    restricted to this key block:

        P_pj  = exp(s_pj - LSE_p)            (0 for hidden keys)
        D_p   = sum_d dO_pd O_pd
        dV_j  = sum_p P_pj dO_p
        dP_pj = dO_p . v_j
        dS_pj = P_pj (dP_pj - D_p)
        dQ_p  = sigma sum_j dS_pj k_j
        dK_j  = sigma sum_p dS_pj q_p

    Returns (dq, dk, dv) in float64; summing them over all key blocks (dq) and
    all query blocks (dk, dv) gives the gradients of the unsharded attention.
    """
    q, k, v, do, o, lse = map(_as64, (q, k, v, do, o, lse))
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    lead = q.shape[:-2]
    Tq, D = q.shape[-2:]
    Tk = k.shape[-2]
    sig = _scale(D, scale)
    qf, kf, vf = q.reshape(-1, Tq, D), k.reshape(-1, Tk, D), v.reshape(-1, Tk, D)
    dof, of, lf = do.reshape(-1, Tq, D), o.reshape(-1, Tq, D), lse.reshape(-1, Tq)
    dq = np.zeros_like(qf)
    dk = np.zeros_like(kf)
    dv = np.zeros_like(vf)
    for n in range(qf.shape[0]):
        for r0 in range(0, Tq, _ROWS):
            r1 = min(Tq, r0 + _ROWS)
            s = sig * (qf[n, r0:r1] @ kf[n].T)
            lrow = lf[n, r0:r1]
            with np.errstate(invalid="ignore"):
                p = np.exp(s - lrow[:, None])
            if causal:
                p[kpos[None, :] > qpos[r0:r1, None]] = 0.0
            p[~np.isfinite(lrow)] = 0.0
            dlt = (dof[n, r0:r1] * of[n, r0:r1]).sum(axis=1)
            dv[n] += p.T @ dof[n, r0:r1]
            dp = dof[n, r0:r1] @ vf[n].T
            ds = p * (dp - dlt[:, None])
            dq[n, r0:r1] += sig * (ds @ kf[n])
            dk[n] += sig * (ds.T @ qf[n, r0:r1])
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)


def causal_attention_bwd(q, k, v, do, scale=None):
    """Gradients of the full-sequence causal attention for upstream ``do``.

    Returns (dq, dk, dv, o, lse) in global token order.
    """
    T = q.shape[-2]
    pos = np.arange(T)
    o, lse = block_attention_fwd(q, k, v, pos, pos, causal=True, scale=scale)
    dq, dk, dv = block_attention_bwd(q, k, v, do, o, lse, pos, pos, causal=True, scale=scale)
    return dq, dk, dv, o, lse


def delta(do, o):
    """D_p = sum_d dO_pd O_pd (the softmax-backward row term)."""
    return (_as64(do) * _as64(o)).sum(axis=-1)
