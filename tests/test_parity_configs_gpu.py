"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (the ring driver, then the backward preprocess and one block
backward per ring step), against the fp64 oracle.

The kernels always run on every head. The forward of every workload is
compared on every head; the 16k backward on four heads spread over the grid
(first, last and two between), both ranks, every row and key of those heads,
and on every head through sums the softmax fixes (sum of dK zero, sum of dV
the sum of dO, sum q.dQ equal to sum k.dK). The oracle runs one head per host
thread.
"""
import numpy as np
import pytest
import torch

import context_causal_attention_cpattn_amd as cp
from oracle import attention as oa
from oracle import rope as orope
from workloads import BY_NAME, draw

from _util import TOL_BF16, TOL_F32, f64, gather, log, max_err, per_head

pytestmark = pytest.mark.gpu
DEV = "cuda"


class Share:
    """One rank's share of the ring on the GPU (all KV blocks resident)."""

    def __init__(self, w, t, rank, rope=False):
        self.w, self.rank = w, rank
        N = w.ring
        self.maps, self.pos = zip(*[cp.cpattn_headtail_shard(w.T, N, r) for r in range(N)])
        self.kb = [gather(t["k"], p) for p in self.pos]
        self.vb = [gather(t["v"], p) for p in self.pos]
        self.q = gather(t["q"], self.pos[rank])
        self.do = gather(t["do"], self.pos[rank]) if "do" in t else None
        Tl = w.local_len
        self.tab = None
        if rope:
            self.tab = torch.empty(w.T, w.D, device=DEV)
            cp.cpattn_rope_table(w.rope_theta, w.T, w.D, self.tab)
        self.ws = torch.empty(cp.cpattn_ring_fwd_workspace_bytes(w.B, w.H, Tl, w.D, rope=rope), dtype=torch.uint8,
                              device=DEV)
        self.o = torch.empty(w.B, w.H, Tl, w.D, device=DEV)
        self.lse = torch.empty(w.B, w.H, Tl, device=DEV)

    def forward(self):
        cp.cpattn_ring_fwd(self.q, self.kb, self.vb, self.maps, self.rank, self.maps[self.rank], self.o, self.lse,
                           self.ws, rope_table=self.tab)

    def backward(self, dk, dv, dq=None, staged=False):
        """Per-step block backward calls; ``staged``: the form that stages dS in HBM."""
        w, N, r = self.w, self.w.ring, self.rank
        self.delta = torch.empty(w.B, w.H, w.local_len, device=DEV)
        cp.cpattn_bwd_preprocess(self.do, self.o, self.delta)
        self.dq = torch.zeros_like(self.o) if dq is None else dq
        ws = None
        if staged:
            n = cp.cpattn_block_bwd_staged_workspace_bytes(w.B, w.H, w.local_len, w.local_len, w.D)
            ws = torch.full((max(n, 1),), 0xFF, dtype=torch.uint8, device=DEV)  # NaN where never written
        for s in range(N):
            src = (r - s) % N
            args = (self.q, self.kb[src], self.vb[src], self.do, self.lse, self.delta, self.dq, dk[src], dv[src],
                    self.maps[r], self.maps[src])
            if staged:
                cp.cpattn_block_bwd_staged(*args, ws)
            else:
                cp.cpattn_block_bwd(*args)


def oracle_fwd(t, rows, heads, rope_theta=0.0):
    """fp64 O [B, len(heads), rows, D] and LSE of the global causal attention for the given
    query rows, one head per host thread (rotary applied at every global position first)."""
    def one(h):
        q, k, v = (f64(t[n][:, h:h + 1]) for n in ("q", "k", "v"))
        if rope_theta:
            allpos = np.arange(q.shape[2])
            q, k = orope.rope_apply(q, allpos, rope_theta), orope.rope_apply(k, allpos, rope_theta)
        return oa.causal_attention_fwd(q, k, v, rows=rows)
    res = per_head(one, list(heads))
    return np.concatenate([r[0] for r in res], axis=1), np.concatenate([r[1] for r in res], axis=1)


def check_fwd(share, t, heads, tol, rope_theta=0.0, ref=None):
    rows = list(share.pos[share.rank])
    O, L = ref if ref is not None else oracle_fwd(t, rows, heads, rope_theta)
    eo = max_err(f64(share.o[:, heads]), O)
    el = max_err(f64(share.lse[:, heads]), L)
    log(f"  rank {share.rank}: max err O {eo:.3g} LSE {el:.3g} ({len(heads)} heads)")
    assert eo <= tol and el <= tol
    return O, L


def test_tiny_fp32_both_ranks():
    w = BY_NAME["tiny"]
    log(f"workload {w.name}")
    t = draw(w)
    for r in range(w.ring):
        s = Share(w, t, r)
        s.forward()
        torch.cuda.synchronize()
        check_fwd(s, t, list(range(w.H)), TOL_F32)


def test_gpt2s_rank0_forward_and_backward():
    w = BY_NAME["gpt2s"]
    log(f"workload {w.name}")
    g = torch.Generator().manual_seed(w.seed + 1000)
    t = draw(w)
    t["do"] = torch.randn(w.B, w.H, w.T, w.D, generator=g).to(torch.bfloat16)
    t64 = {n: f64(x) for n, x in t.items()}
    s = Share(w, t, 0)
    dk = [torch.zeros(w.B, w.H, w.local_len, w.D, device=DEV) for _ in range(w.ring)]
    dv = [torch.zeros_like(x) for x in dk]
    s.forward()
    s.backward(dk, dv)
    torch.cuda.synchronize()
    O, L = check_fwd(s, t, list(range(w.H)), TOL_BF16)
    rows = list(s.pos[0])
    gq, gk, gv = oa.block_attention_bwd(t64["q"][:, :, rows], t64["k"], t64["v"], t64["do"][:, :, rows], O, L, rows,
                                        np.arange(w.T))
    e = [max_err(f64(s.dq), gq)]
    for src in range(w.ring):
        p = list(s.pos[src])
        e += [max_err(f64(dk[src]), gk[:, :, p]), max_err(f64(dv[src]), gv[:, :, p])]
    log(f"  rank-0 backward share: max err dq {e[0]:.3g} dk/dv {max(e[1:]):.3g}")
    assert max(e) <= TOL_BF16


def test_win16k_rank0_forward():
    w = BY_NAME["win16k"]
    log(f"workload {w.name}")
    t = draw(w)
    s = Share(w, t, 0)
    s.forward()
    torch.cuda.synchronize()
    check_fwd(s, t, list(range(w.H)), TOL_BF16)


_WIN32K = {}


def _win32k_reference():
    """Inputs and the rank-0 fp64 reference (every head) of the 32k window with rotary."""
    if not _WIN32K:
        w = BY_NAME["win32k"]
        t = draw(w)
        _, pos = cp.cpattn_headtail_shard(w.T, w.ring, 0)
        _WIN32K.update(t=t, ref=oracle_fwd(t, list(pos), range(w.H), w.rope_theta))
    return _WIN32K["t"], _WIN32K["ref"]


def test_win32k_rope_rank0_forward():
    """The ring driver's rotary form: Q and each K block rotated once, then the block kernels
    (the form the benchmark times)."""
    w = BY_NAME["win32k"]
    log(f"workload {w.name}")
    t, ref = _win32k_reference()
    s = Share(w, t, 0, rope=True)
    s.forward()
    torch.cuda.synchronize()
    check_fwd(s, t, list(range(w.H)), TOL_BF16, ref=ref)


def test_win32k_fused_rotary_block_fwd_rank0():
    """cpattn_block_fwd with the rotary table (the per-tile fused rotation) at the 32k window's
    full size: step 0 on the own block, step 1 on the other block's visible rows into a second
    pair, then cpattn_lse_merge; every head against the same reference."""
    w = BY_NAME["win32k"]
    log(f"workload {w.name}, fused rotary block forward")
    t, ref = _win32k_reference()
    s = Share(w, t, 0, rope=True)
    Tl = w.local_len
    cp.cpattn_block_fwd(s.q, s.kb[0], s.vb[0], s.maps[0], s.maps[0], s.o, s.lse, rope_table=s.tab)
    src = (0 - 1) % w.ring
    rb, _ = cp.cpattn_step_rows(s.maps[0], s.maps[src])
    ob = torch.empty_like(s.o)
    lb = torch.empty_like(s.lse)
    cp.cpattn_block_fwd(s.q, s.kb[src], s.vb[src], s.maps[0], s.maps[src], ob, lb, rope_table=s.tab,
                        row_begin=rb, row_end=Tl)
    cp.cpattn_lse_merge(s.o, s.lse, ob, lb, rb, Tl)
    torch.cuda.synchronize()
    check_fwd(s, t, list(range(w.H)), TOL_BF16, ref=ref)


def test_bwd16k_all_ranks():
    w = BY_NAME["bwd16k"]
    log(f"workload {w.name}")
    t = draw(w)
    dk = [torch.zeros(w.B, w.H, w.local_len, w.D, device=DEV) for _ in range(w.ring)]
    dv = [torch.zeros_like(x) for x in dk]
    shares = []
    for r in range(w.ring):
        s = Share(w, t, r)
        s.forward()
        s.backward(dk, dv)
        shares.append(s)
    # the form with dS staged in HBM gives the same bits on every head of both ranks
    dk2 = [torch.zeros_like(x) for x in dk]
    dv2 = [torch.zeros_like(x) for x in dk]
    for s in shares:
        dq1 = s.dq
        s.backward(dk2, dv2, staged=True)
        torch.cuda.synchronize()
        assert torch.equal(dq1, s.dq), s.rank
    for r in range(w.ring):
        assert torch.equal(dk[r], dk2[r]) and torch.equal(dv[r], dv2[r]), r
    log("  staged dS: every head of both ranks bitwise equal to the recomputing form")
    torch.cuda.synchronize()
    heads = [0, 11, 20, 31]
    res = per_head(lambda h: oa.causal_attention_bwd(*(f64(t[n][:, h:h + 1]) for n in ("q", "k", "v", "do"))),
                   heads)
    dQ, dK, dV, O, L = (np.concatenate([r[i] for r in res], axis=1) for i in range(5))
    for s in shares:
        rows = list(s.pos[s.rank])
        eo = max_err(f64(s.o[:, heads]), O[:, :, rows])
        el = max_err(f64(s.lse[:, heads]), L[:, :, rows])
        eq = max_err(f64(s.dq[:, heads]), dQ[:, :, rows])
        ek = max_err(f64(dk[s.rank][:, heads]), dK[:, :, rows])
        ev = max_err(f64(dv[s.rank][:, heads]), dV[:, :, rows])
        log(f"  rank {s.rank}, heads {heads}: O {eo:.3g} LSE {el:.3g} dq {eq:.3g} dk {ek:.3g} dv {ev:.3g}")
        assert max(eo, el, eq, ek, ev) <= TOL_BF16
    _bwd_sum_invariants(w, t, shares, dk, dv)


def _bwd_sum_invariants(w, t, shares, dk, dv):
    """Every head, every row and key of the sequence: each row of P sums to one and each row
    of dS to zero, so sum_j dV_j = sum_p dO_p and sum_j dK_j = 0; and S depends on q and k
    only through q.k, so scaling q by a and k by 1/a changes nothing: sum_p q_p.dQ_p =
    sum_j k_j.dK_j (both sides contract the same dS values, so this one holds to fp32
    accumulation)."""
    g = lambda x: torch.empty(w.B, w.H, w.T, w.D, dtype=torch.float64, device=DEV)
    dqg, dkg, dvg = g(0), g(0), g(0)
    for s in shares:
        dqg[:, :, list(s.pos[s.rank])] = s.dq.double()
    for r in range(w.ring):
        idx = list(shares[0].pos[r])
        dkg[:, :, idx] = dk[r].double()
        dvg[:, :, idx] = dv[r].double()
    qg, kg, dog = (t[n].to(DEV).double() for n in ("q", "k", "do"))
    rk = float((dkg.sum(2).abs() / dkg.abs().sum(2)).max())
    rv = float(((dvg.sum(2) - dog.sum(2)).abs() / dvg.abs().sum(2)).max())
    qd, kd = qg * dqg, kg * dkg
    rs = float(((qd.sum((2, 3)) - kd.sum((2, 3))).abs() / (qd.abs().sum((2, 3)) + kd.abs().sum((2, 3)))).max())
    log(f"  every head: |sum dK| / sum|dK| {rk:.3g}, |sum dV - sum dO| / sum|dV| {rv:.3g}, "
        f"|sum q.dQ - sum k.dK| / sum|.| {rs:.3g}")
    assert rk <= 1e-3 and rv <= 1e-3 and rs <= 1e-6


def test_win32k_rope_backward_all_ranks_sampled():
    """Backward through the rotary at the 32k window's full size (both ranks, all heads):
    block backward on the rotated Q and K blocks, dQ and each dK block taken back through
    R^T after the last step. The oracle checks sampled rows one by one: dQ of rows spread
    over the sequence, dK and dV of the last keys (every query that sees them is in the last
    rows); for every key, sum_j R(j) dK_j = 0 and sum_j dV_j = sum_p dO_p per head."""
    w = BY_NAME["win32k"]
    log(f"workload {w.name} backward through rotary")
    g = torch.Generator().manual_seed(w.seed + 1000)
    t = draw(w)
    t["do"] = torch.randn(w.B, w.H, w.T, w.D, generator=g).to(torch.bfloat16)
    N, Tl = w.ring, w.local_len
    dk = [torch.zeros(w.B, w.H, Tl, w.D, device=DEV) for _ in range(N)]
    dv = [torch.zeros_like(x) for x in dk]
    shares = [Share(w, t, r, rope=True) for r in range(N)]
    tab = shares[0].tab
    kr = [cp.cpattn_rope_rotate(shares[0].kb[i], shares[0].maps[i], tab, torch.empty_like(shares[0].kb[i]))
          for i in range(N)]
    dq = []
    for s in shares:
        s.forward()
        qrot = cp.cpattn_rope_rotate(s.q, s.maps[s.rank], tab, torch.empty_like(s.q))
        delta = torch.empty(w.B, w.H, Tl, device=DEV)
        cp.cpattn_bwd_preprocess(s.do, s.o, delta)
        d = torch.zeros_like(s.o)
        for st in range(N):
            src = (s.rank - st) % N
            cp.cpattn_block_bwd(qrot, kr[src], s.vb[src], s.do, s.lse, delta, d, dk[src], dv[src], s.maps[s.rank],
                                s.maps[src])
        cp.cpattn_rope_rotate_grad(d, s.maps[s.rank], tab)
        dq.append(d)
    for i in range(N):
        cp.cpattn_rope_rotate_grad(dk[i], shares[0].maps[i], tab)
    torch.cuda.synchronize()
    T = w.T
    where = {}
    for r, s in enumerate(shares):
        for li, gp in enumerate(s.pos[r]):
            where[gp] = (r, li)
    allpos = np.arange(T)
    head = 9
    q64, k64, v64, do64 = (f64(t[n][:, head:head + 1]) for n in ("q", "k", "v", "do"))
    qr, krot = orope.rope_apply(q64, allpos, w.rope_theta), orope.rope_apply(k64, allpos, w.rope_theta)
    # dQ of sampled rows
    P = [0, 1, 777, T // 2 - 1, T // 2, 30000, T - 1]
    O, L = oa.block_attention_fwd(qr[:, :, P], krot, v64, P, allpos)
    gq, _, _ = oa.block_attention_bwd(qr[:, :, P], krot, v64, do64[:, :, P], O, L, P, allpos)
    gq = orope.rope_apply_transpose(gq, P, w.rope_theta)
    got = np.stack([f64(dq[where[p][0]][:, head:head + 1, where[p][1]]) for p in P], axis=2)
    eq = max_err(got, gq)
    # dK, dV of the last keys from the rows that can see them
    J = [T - 68, T - 7, T - 1]
    R = list(range(J[0], T))
    O, L = oa.block_attention_fwd(qr[:, :, R], krot, v64, R, allpos)
    _, gk, gv = oa.block_attention_bwd(qr[:, :, R], krot[:, :, J], v64[:, :, J], do64[:, :, R], O, L, R, J)
    gk = orope.rope_apply_transpose(gk, J, w.rope_theta)
    gotk = np.stack([f64(dk[where[j][0]][:, head:head + 1, where[j][1]]) for j in J], axis=2)
    gotv = np.stack([f64(dv[where[j][0]][:, head:head + 1, where[j][1]]) for j in J], axis=2)
    ek, ev = max_err(gotk, gk), max_err(gotv, gv)
    log(f"  sampled rows, head {head}: dq {eq:.3g} dk {ek:.3g} dv {ev:.3g}")
    assert max(eq, ek, ev) <= TOL_BF16
    # sums over every key of the sequence, all heads
    kglob = np.zeros((w.B, w.H, T, w.D))
    vglob = np.zeros_like(kglob)
    for i in range(N):
        kglob[:, :, list(shares[0].pos[i])] = f64(dk[i])
        vglob[:, :, list(shares[0].pos[i])] = f64(dv[i])
    ksum = orope.rope_apply(kglob, allpos, w.rope_theta).sum(axis=2)
    kabs = np.abs(kglob).sum(axis=2)
    vsum, dosum = vglob.sum(axis=2), f64(t["do"]).sum(axis=2)
    rk = float((np.abs(ksum) / kabs).max())
    rv = float((np.abs(vsum - dosum) / np.abs(vglob).sum(axis=2)).max())
    log(f"  invariants: |sum R dK| / sum|dK| {rk:.3g}, |sum dV - sum dO| / sum|dV| {rv:.3g}")
    assert rk <= 1e-3 and rv <= 1e-3


def _ring_bwd(s, dq, dk, dv, accumulate, staged=False):
    w = s.w
    n = (cp.cpattn_ring_bwd_staged_workspace_bytes(w.B, w.H, w.local_len, w.local_len, w.D) if staged
         else cp.cpattn_ring_bwd_workspace_bytes(w.B, w.H, w.local_len))
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)
    cp.cpattn_ring_bwd(s.q, s.kb, s.vb, s.maps, s.rank, s.maps[s.rank], s.do, s.o, s.lse, dq, dk, dv, ws,
                       accumulate=accumulate)


@pytest.mark.parametrize("name,rank", [("gpt2s", 1), ("bwd16k", 1)])
def test_ring_bwd_equals_step_driven_backward(name, rank):
    """The one-call ring backward launches the same kernels as the per-step calls: overwriting
    NaN-filled accumulators gives exactly the per-step result into zeros, and adding into filled
    accumulators gives exactly the per-step result from the same fill."""
    w = BY_NAME[name]
    log(f"workload {w.name} rank {rank}")
    t = draw(w)
    if "do" not in t:
        g = torch.Generator().manual_seed(w.seed + 1000)
        t["do"] = torch.randn(w.B, w.H, w.T, w.D, generator=g).to(torch.bfloat16)
    s = Share(w, t, rank)
    s.forward()
    shape = (w.B, w.H, w.local_len, w.D)
    dk_ref = [torch.zeros(shape, device=DEV) for _ in range(w.ring)]
    dv_ref = [torch.zeros(shape, device=DEV) for _ in range(w.ring)]
    s.backward(dk_ref, dv_ref)
    nan = lambda: torch.full(shape, float("nan"), device=DEV)
    for staged in (False, True):  # with room to stage dS: the same bits
        dq, dk, dv = nan(), [nan() for _ in range(w.ring)], [nan() for _ in range(w.ring)]
        _ring_bwd(s, dq, dk, dv, accumulate=False, staged=staged)
        torch.cuda.synchronize()
        assert torch.equal(dq, s.dq), staged
        for i in range(w.ring):
            assert torch.equal(dk[i], dk_ref[i]) and torch.equal(dv[i], dv_ref[i]), (i, staged)
    # accumulate: both forms start from the same fill
    g = torch.Generator(device="cpu").manual_seed(7)
    fill = [torch.randn(shape, generator=g).to(DEV) for _ in range(1 + 2 * w.ring)]
    dq2, dk2, dv2 = fill[0].clone(), [x.clone() for x in fill[1:1 + w.ring]], [x.clone() for x in fill[1 + w.ring:]]
    _ring_bwd(s, dq2, dk2, dv2, accumulate=True)
    dk_ref2, dv_ref2 = [x.clone() for x in fill[1:1 + w.ring]], [x.clone() for x in fill[1 + w.ring:]]
    s.backward(dk_ref2, dv_ref2, dq=fill[0].clone())
    torch.cuda.synchronize()
    assert torch.equal(dq2, s.dq)
    for i in range(w.ring):
        assert torch.equal(dk2[i], dk_ref2[i]) and torch.equal(dv2[i], dv_ref2[i]), i
    log(f"  ring backward equals the per-step calls ({w.ring} steps)")


def test_ring_bwd_contiguous_shards_with_invisible_blocks():
    """Contiguous sharding (rank r holds [r L, (r+1) L)): every later rank's block lies in the future
    of all local rows. Overwriting writes zeros for those blocks, adding leaves them untouched,
    and the visible blocks match the oracle."""
    from workloads import Workload
    w = Workload("contig", 11, B=1, H=2, D=64, T=1024, ring=4, dtype="bf16", backward=True)
    t = draw(w)
    t64 = {n: f64(x) for n, x in t.items()}
    L = w.T // w.ring
    maps = [cp.cpattn_posmap(L, L, r * L, r * L) for r in range(w.ring)]
    pos = [list(range(r * L, (r + 1) * L)) for r in range(w.ring)]
    kb = [gather(t["k"], p) for p in pos]
    vb = [gather(t["v"], p) for p in pos]
    shape = (w.B, w.H, L, w.D)
    for rank in (0, 2):
        log(f"  contiguous rank {rank}")
        q, do = gather(t["q"], pos[rank]), gather(t["do"], pos[rank])
        o = torch.empty(shape, device=DEV)
        lse = torch.empty(w.B, w.H, L, device=DEV)
        wsf = torch.empty(cp.cpattn_ring_fwd_workspace_bytes(w.B, w.H, L, w.D), dtype=torch.uint8, device=DEV)
        cp.cpattn_ring_fwd(q, kb, vb, maps, rank, maps[rank], o, lse, wsf)
        ws = torch.empty(cp.cpattn_ring_bwd_workspace_bytes(w.B, w.H, L), dtype=torch.uint8, device=DEV)
        nan = lambda: torch.full(shape, float("nan"), device=DEV)
        dq, dk, dv = nan(), [nan() for _ in range(w.ring)], [nan() for _ in range(w.ring)]
        cp.cpattn_ring_bwd(q, kb, vb, maps, rank, maps[rank], do, o, lse, dq, dk, dv, ws, accumulate=False)
        fill = [torch.full(shape, 3.0, device=DEV) for _ in range(2 * w.ring)]
        dk2, dv2 = fill[:w.ring], fill[w.ring:]
        dq2 = torch.zeros(shape, device=DEV)
        cp.cpattn_ring_bwd(q, kb, vb, maps, rank, maps[rank], do, o, lse, dq2, dk2, dv2, ws, accumulate=True)
        torch.cuda.synchronize()
        rows = pos[rank]
        O, Lr = oa.causal_attention_fwd(t64["q"], t64["k"], t64["v"], rows=rows)
        gq, gk, gv = oa.block_attention_bwd(t64["q"][:, :, rows], t64["k"], t64["v"], t64["do"][:, :, rows], O, Lr,
                                            rows, np.arange(w.T))
        errs = [max_err(f64(dq), gq), max_err(f64(dq2), gq)]
        for src in range(w.ring):
            p = pos[src]
            if src > rank:  # invisible: zeros when overwriting, untouched when adding
                assert torch.count_nonzero(dk[src]) == 0 and torch.count_nonzero(dv[src]) == 0
                assert bool((dk2[src] == 3.0).all()) and bool((dv2[src] == 3.0).all())
            errs += [max_err(f64(dk[src]), gk[:, :, p]), max_err(f64(dv[src]), gv[:, :, p]),
                     max_err(f64(dk2[src]) - 3.0, gk[:, :, p]), max_err(f64(dv2[src]) - 3.0, gv[:, :, p])]
        log(f"  rank {rank}: max err {max(errs):.3g}")
        assert max(errs) <= TOL_BF16


def test_gqa16k_staged_backward_bitwise_both_ranks():
    """The grouped-query 16k workload (32 query heads over 8 KV heads) at full size: the staged
    block backward gives the bits of the recomputing one for every step of both ranks (dQ per
    query head, dK/dV summed over each group), with the staging area filled with NaN."""
    w = BY_NAME["gqa16k"]
    log(f"workload {w.name}")
    t = draw(w)
    N, Tl, Hk = w.ring, w.local_len, w.kv_heads
    maps, pos = zip(*[cp.cpattn_headtail_shard(w.T, N, r) for r in range(N)])
    kb = [gather(t["k"], p) for p in pos]
    vb = [gather(t["v"], p) for p in pos]
    n = cp.cpattn_block_bwd_staged_workspace_bytes(w.B, w.H, Tl, Tl, w.D)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)
    for r in range(N):
        q, do = gather(t["q"], pos[r]), gather(t["do"], pos[r])
        o = torch.empty(w.B, w.H, Tl, w.D, device=DEV)
        lse = torch.empty(w.B, w.H, Tl, device=DEV)
        cp.cpattn_block_fwd_gqa(q, kb[r], vb[r], maps[r], maps[r], o, lse)
        for s in range(1, N):
            src = (r - s) % N
            rb, _ = cp.cpattn_step_rows(maps[r], maps[src])
            if rb < Tl:
                cp.cpattn_block_fwd_merge(q, kb[src], vb[src], maps[r], maps[src], o, lse, row_begin=rb)
        delta = torch.empty(w.B, w.H, Tl, device=DEV)
        cp.cpattn_bwd_preprocess(do, o, delta)
        res = []
        for staged in (False, True):
            dq = torch.zeros(w.B, w.H, Tl, w.D, device=DEV)
            dk = [torch.zeros(w.B, Hk, Tl, w.D, device=DEV) for _ in range(N)]
            dv = [torch.zeros_like(x) for x in dk]
            for s in range(N):
                src = (r - s) % N
                args = (q, kb[src], vb[src], do, lse, delta, dq, dk[src], dv[src], maps[r], maps[src])
                if staged:
                    cp.cpattn_block_bwd_staged(*args, ws, accumulate=s > 0)
                else:
                    cp.cpattn_block_bwd_gqa(*args, accumulate=s > 0)
            res.append([dq] + dk + dv)
        torch.cuda.synchronize()
        for x, y in zip(*res):
            assert torch.equal(x, y), r
            assert bool(torch.isfinite(y).all()), r
        log(f"  rank {r}: staged equals recomputing on dQ and every block's dK, dV")
        _local_sum_invariants(q, do, res[1][0], kb, res[1][1:1 + N], res[1][1 + N:], w.H // Hk)


def _local_sum_invariants(q, do, dq, kbs, dks, dvs, G):
    """One rank's rows against every key block, per KV head (grouped-query: G query heads
    share it): the identities of the full-size backward above, restricted to the rows this
    rank holds (each row's P and dS rows run over all keys of all blocks)."""
    B, H, _, D = q.shape
    qd = (q.double() * dq.double()).reshape(B, H // G, G, -1, D)
    dog = do.double().reshape(B, H // G, G, -1, D).sum((2, 3))
    dk = torch.cat([x.double() for x in dks], dim=2)
    dv = torch.cat([x.double() for x in dvs], dim=2)
    kd = torch.cat([x.double() for x in kbs], dim=2) * dk
    rk = float((dk.sum(2).abs() / dk.abs().sum(2)).max())
    rv = float(((dv.sum(2) - dog).abs() / dv.abs().sum(2)).max())
    rs = float(((qd.sum((2, 3, 4)) - kd.sum((2, 3))).abs() / (qd.abs().sum((2, 3, 4)) + kd.abs().sum((2, 3)))).max())
    log(f"  every KV head: |sum dK| / sum|dK| {rk:.3g}, |sum dV - sum dO| / sum|dV| {rv:.3g}, "
        f"|sum q.dQ - sum k.dK| / sum|.| {rs:.3g}")
    assert rk <= 1e-3 and rv <= 1e-3 and rs <= 1e-6
