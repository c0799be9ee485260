"""The ring forward and backward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay gives the bits of the same calls run eagerly. The library issues no memset and
no allocation inside its calls, so a captured step holds only its kernels; the replays are
interleaved with eager work of the same program and checked one by one."""
import pytest
import torch

import context_causal_attention_cpattn_amd as cp
from workloads import draw_shape

from _util import log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _share(T, N, rank, B, H, D, seed):
    maps, pos = zip(*[cp.cpattn_headtail_shard(T, N, r) for r in range(N)])
    Tl = T // N
    q, do = (x.to(DEV) for x in draw_shape(B, H, Tl, D, torch.bfloat16, seed=seed, n=2))
    kb = [x.to(DEV) for x in draw_shape(B, H, Tl, D, torch.bfloat16, seed=seed + 1, n=N)]
    vb = [x.to(DEV) for x in draw_shape(B, H, Tl, D, torch.bfloat16, seed=seed + 2, n=N)]
    return maps, q, do, kb, vb


@pytest.mark.parametrize("D,rope,bwd", [(128, False, "ring"), (128, True, None), (64, False, "ring"),
                                        (128, False, "noalloc")])
def test_ring_step_graph_replays_bitwise(D, rope, bwd):
    """bwd: the one-call ring backward with a staging workspace, or the one that allocates
    nothing (its device scratch array set up by the eager call before the capture)."""
    T, N, rank, B, H = 2048, 2, 0, 1, 4
    log(f"graph replay D={D} rope={rope} backward={bwd} T={T} ring={N}")
    maps, q, do, kb, vb = _share(T, N, rank, B, H, D, seed=1200 + D)
    Tl = T // N
    tab = None
    if rope:
        tab = torch.empty(T, D, device=DEV)
        cp.cpattn_rope_table(10000.0, T, D, tab)
    fws = torch.empty(cp.cpattn_ring_fwd_workspace_bytes(B, H, Tl, D, rope=rope), dtype=torch.uint8, device=DEV)
    bws = torch.empty(cp.cpattn_ring_bwd_staged_workspace_bytes(B, H, Tl, Tl, D), dtype=torch.uint8, device=DEV)

    def buffers():
        o = torch.empty(B, H, Tl, D, device=DEV)
        lse = torch.empty(B, H, Tl, device=DEV)
        dq = torch.empty(B, H, Tl, D, device=DEV)
        dk = [torch.empty(B, H, Tl, D, device=DEV) for _ in range(N)]
        dv = [torch.empty(B, H, Tl, D, device=DEV) for _ in range(N)]
        return o, lse, dq, dk, dv

    def step(bufs):
        o, lse, dq, dk, dv = bufs
        cp.cpattn_ring_fwd(q, kb, vb, maps, rank, maps[rank], o, lse, fws, rope_table=tab)
        if bwd == "ring":
            cp.cpattn_ring_bwd(q, kb, vb, maps, rank, maps[rank], do, o, lse, dq, dk, dv, bws, accumulate=False)
        elif bwd == "noalloc":
            cp.cpattn_ring_bwd_noalloc(q, kb, vb, maps, rank, maps[rank], do, o, lse, dq, dk, dv, accumulate=False)

    def flat(bufs):
        o, lse, dq, dk, dv = bufs
        return [o, lse] + ([dq] + dk + dv if bwd else [])

    ref = buffers()
    step(ref)
    torch.cuda.synchronize()
    got = buffers()
    for x in flat(got):
        x.fill_(float("nan"))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(got)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(got)
    torch.cuda.synchronize()
    other = buffers()
    for i in range(3):
        for x in flat(got):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(flat(ref), flat(got)):
            assert torch.equal(x, y), i
        step(other)  # eager work of the same program between the replays
        torch.cuda.synchronize()
        for x, y in zip(flat(ref), flat(other)):
            assert torch.equal(x, y), i
    log(f"  3 replays bitwise equal to the eager step ({len(flat(ref))} outputs)")
