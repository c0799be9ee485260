"""GPU parity of the block backward with dS staged in HBM (cpattn_block_bwd_staged, and
cpattn_ring_bwd given a workspace large enough to stage): against the fp64 oracle, and bit
for bit against the recomputing form (cpattn_block_bwd / _gqa), which contracts the same bf16
dS values in the same order. The staging area starts filled with NaN, so a block read before
it was written would show in the results."""
import numpy as np
import pytest
import torch

import context_causal_attention_cpattn_amd as cp
from oracle import attention as oa
from workloads import draw_shape

from _util import f64, gather, log, max_err, tol_bf16_scaled

pytestmark = pytest.mark.gpu
DEV = "cuda"


def positions(m):
    L, split, d0, d1 = m
    return np.array([i + (d0 if i < split else d1) for i in range(L)])


def nan_area(nbytes):
    return torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=DEV)


def both_forms(q, k, v, do, lse, delta, qm, km, causal, acc, fill=None):
    """(recompute, staged) results [dq, dk, dv]; accumulators start from ``fill`` (or zeros)."""
    B, H, Tq, D = q.shape
    Hk, Tk = k.shape[1], k.shape[2]
    out = []
    for staged in (False, True):
        g = [torch.zeros(B, H, Tq, D, device=DEV), torch.zeros(B, Hk, Tk, D, device=DEV),
             torch.zeros(B, Hk, Tk, D, device=DEV)]
        if fill is not None:
            for x, f in zip(g, fill):
                x.copy_(f)
        if staged:
            ws = nan_area(cp.cpattn_block_bwd_staged_workspace_bytes(B, H, Tq, Tk, D))
            cp.cpattn_block_bwd_staged(q, k, v, do, lse, delta, *g, qm, km, ws, causal=causal, accumulate=acc)
        else:
            cp.cpattn_block_bwd_gqa(q, k, v, do, lse, delta, *g, qm, km, causal=causal, accumulate=acc)
        out.append(g)
    torch.cuda.synchronize()
    return out


# (B, H, H_kv, Tq, Tk, causal, maps): head-tail shards of T = 600 (rank 0 against its own block
# and against rank 1's), ragged non-causal blocks, single rows and keys, a grouped-query block
CASES = [
    (1, 2, 2, 300, 300, True, "ht600_own"),
    (1, 2, 2, 300, 300, True, "ht600_other"),
    (2, 3, 3, 150, 230, False, "plain"),
    (1, 2, 2, 33, 1, True, "plain"),
    (1, 2, 2, 1, 77, False, "plain"),
    (2, 1, 1, 2, 129, True, "plain"),
    (1, 3, 3, 97, 161, True, "plain"),
    (1, 4, 2, 260, 260, True, "ht520_own"),
    (1, 4, 1, 200, 333, False, "plain"),
]


def case_maps(Tq, Tk, kind):
    if kind == "plain":
        return (Tq, Tq, 0, 0), (Tk, Tk, 0, 0)
    T = int(kind[2:5])
    own = kind.endswith("own")
    qm, _ = cp.cpattn_headtail_shard(T, 2, 0)
    km, _ = cp.cpattn_headtail_shard(T, 2, 0 if own else 1)
    return qm, km


@pytest.mark.parametrize("case", CASES, ids=[f"{c[3]}x{c[4]}_H{c[1]}_{c[2]}_{'c' if c[5] else 'nc'}_{c[6]}"
                                            for c in CASES])
def test_block_bwd_staged_against_oracle_and_recompute(case):
    B, H, Hk, Tq, Tk, causal, kind = case
    D = 128
    log(f"block_bwd_staged B={B} H={H} H_kv={Hk} Tq={Tq} Tk={Tk} causal={causal} {kind}")
    qm, km = case_maps(Tq, Tk, kind)
    qp, kp = positions(qm), positions(km)
    q, do = draw_shape(B, H, Tq, D, torch.bfloat16, seed=500 + Tq, n=2)
    k, v = draw_shape(B, Hk, Tk, D, torch.bfloat16, seed=501 + Tk, n=2)
    G = H // Hk
    ke, ve = (np.repeat(f64(x), G, axis=1) for x in (k, v))  # query head h reads KV head h // G
    O, L = oa.block_attention_fwd(f64(q), ke, ve, qp, kp, causal=causal)
    o = torch.tensor(O, dtype=torch.float32, device=DEV)
    lse = torch.tensor(L, dtype=torch.float32, device=DEV)
    delta = torch.empty(B, H, Tq, device=DEV)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    cp.cpattn_bwd_preprocess(dod, o, delta)
    gq, gk, gv = oa.block_attention_bwd(f64(q), ke, ve, f64(do), O, L, qp, kp, causal=causal)
    gk = gk.reshape(B, Hk, G, Tk, D).sum(axis=2)  # a KV head's gradient sums its query heads'
    gv = gv.reshape(B, Hk, G, Tk, D).sum(axis=2)
    rec, stg = both_forms(qd, kd, vd, dod, lse, delta, qm, km, causal, acc=True)
    for t, r, name in zip(stg, (gq, gk, gv), ("dq", "dk", "dv")):
        e = max_err(f64(t), r)
        log(f"  {name} max err {e:.3g}")
        assert e <= tol_bf16_scaled(r), (name, e)
    for a_, b_ in zip(rec, stg):
        assert torch.equal(a_, b_)
    # adding into filled accumulators and overwriting NaN-filled ones: still the same bits
    g = torch.Generator(device="cpu").manual_seed(Tq + Tk)
    fill = [torch.randn(x.shape, generator=g).to(DEV) for x in rec]
    rec2, stg2 = both_forms(qd, kd, vd, dod, lse, delta, qm, km, causal, acc=True, fill=fill)
    for a_, b_ in zip(rec2, stg2):
        assert torch.equal(a_, b_)
    nan = [torch.full_like(x, float("nan")) for x in rec]
    rec3, stg3 = both_forms(qd, kd, vd, dod, lse, delta, qm, km, causal, acc=False, fill=nan)
    for a_, b_, c_ in zip(rec3, stg3, rec):
        assert torch.equal(a_, b_) and torch.equal(b_, c_)


def test_block_bwd_staged_64_wide_heads_need_no_workspace():
    log("block_bwd_staged D=64")
    B, H, Tq, Tk, D = 1, 2, 190, 190, 64
    assert cp.cpattn_block_bwd_staged_workspace_bytes(B, H, Tq, Tk, D) == 0
    q, do = draw_shape(B, H, Tq, D, torch.bfloat16, seed=61, n=2)
    k, v = draw_shape(B, H, Tk, D, torch.bfloat16, seed=62, n=2)
    qm = km = (Tq, Tq, 0, 0)
    O, L = oa.block_attention_fwd(f64(q), f64(k), f64(v), positions(qm), positions(km), causal=True)
    o = torch.tensor(O, dtype=torch.float32, device=DEV)
    lse = torch.tensor(L, dtype=torch.float32, device=DEV)
    delta = torch.empty(B, H, Tq, device=DEV)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    cp.cpattn_bwd_preprocess(dod, o, delta)
    a = [torch.zeros(B, H, Tq, D, device=DEV) for _ in range(3)]
    b = [torch.zeros_like(x) for x in a]
    cp.cpattn_block_bwd(qd, kd, vd, dod, lse, delta, *a, qm, km)
    cp.cpattn_block_bwd_staged(qd, kd, vd, dod, lse, delta, *b, qm, km, None)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("T,N", [(600, 2), (900, 3), (1036, 2)])
def test_ring_bwd_staged_workspace_bitwise(T, N):
    """cpattn_ring_bwd with room to stage dS gives the bits of the one without, on every rank."""
    B, H, D = 1, 2, 128
    log(f"ring_bwd staged T={T} N={N}")
    q, k, v, do = draw_shape(B, H, T, D, torch.bfloat16, seed=T + N, n=4)
    maps, pos = zip(*[cp.cpattn_headtail_shard(T, N, r) for r in range(N)])
    Tl = T // N
    kb = [gather(k, p) for p in pos]
    vb = [gather(v, p) for p in pos]
    fws = torch.empty(cp.cpattn_ring_fwd_workspace_bytes(B, H, Tl, D), dtype=torch.uint8, device=DEV)
    small = cp.cpattn_ring_bwd_workspace_bytes(B, H, Tl)
    big = cp.cpattn_ring_bwd_staged_workspace_bytes(B, H, Tl, Tl, D)
    assert big > small
    for r in range(N):
        qr, dor = gather(q, pos[r]), gather(do, pos[r])
        o = torch.empty(B, H, Tl, D, device=DEV)
        lse = torch.empty(B, H, Tl, device=DEV)
        cp.cpattn_ring_fwd(qr, kb, vb, maps, r, maps[r], o, lse, fws)
        res = []
        for nbytes in (small, big):
            dq = torch.zeros(B, H, Tl, D, device=DEV)
            dk = [torch.zeros(B, H, Tl, D, device=DEV) for _ in range(N)]
            dv = [torch.zeros(B, H, Tl, D, device=DEV) for _ in range(N)]
            cp.cpattn_ring_bwd(qr, kb, vb, maps, r, maps[r], dor, o, lse, dq, dk, dv, nan_area(nbytes),
                               accumulate=False)
            res.append([dq] + dk + dv)
        torch.cuda.synchronize()
        for x, y in zip(*res):
            assert torch.equal(x, y), r


def test_block_bwd_staged_strided_views():
    """Inputs and accumulators that are views into larger allocations (head and row strides
    beyond their shapes): the staged form still equals the recomputing one bit for bit."""
    B, H, Tq, Tk, D = 2, 3, 180, 200, 128
    log("block_bwd_staged strided")
    g = torch.Generator(device="cpu").manual_seed(77)

    def view(shape, pad_h=1, pad_t=24, dtype=torch.bfloat16):
        Bb, Hh, T, Dd = shape
        big = (torch.randn(Bb, Hh + pad_h, T + pad_t, Dd + 64, generator=g) * 0.7).to(dtype).to(DEV)
        return big[:, :Hh, :T, :Dd]

    q, do = view((B, H, Tq, D)), view((B, H, Tq, D))
    k, v = view((B, H, Tk, D)), view((B, H, Tk, D))
    qm, km = (Tq, Tq, 0, 0), (Tk, Tk, 0, 0)
    O, L = oa.block_attention_fwd(f64(q), f64(k), f64(v), positions(qm), positions(km), causal=True)
    o = torch.tensor(O, dtype=torch.float32, device=DEV)
    lse = torch.tensor(L, dtype=torch.float32, device=DEV)
    delta = torch.empty(B, H, Tq, device=DEV)
    cp.cpattn_bwd_preprocess(do, o, delta)
    outs = []
    for staged in (False, True):
        acc = [view((B, H, Tq, D), dtype=torch.float32), view((B, H, Tk, D), dtype=torch.float32),
               view((B, H, Tk, D), dtype=torch.float32)]
        for x in acc:
            x.zero_()
        if staged:
            ws = nan_area(cp.cpattn_block_bwd_staged_workspace_bytes(B, H, Tq, Tk, D))
            cp.cpattn_block_bwd_staged(q, k, v, do, lse, delta, *acc, qm, km, ws)
        else:
            cp.cpattn_block_bwd(q, k, v, do, lse, delta, *acc, qm, km)
        outs.append(acc)
    torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert torch.equal(x, y)
    gq, gk, gv = oa.block_attention_bwd(f64(q), f64(k), f64(v), f64(do), O, L, positions(qm), positions(km))
    for t_, r in zip(outs[1], (gq, gk, gv)):
        assert max_err(f64(t_), r) <= tol_bf16_scaled(r)
