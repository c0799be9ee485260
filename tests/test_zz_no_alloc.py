"""cpattn_ring_bwd_noalloc, the ring backward that allocates nothing (its fp32 delta lives in
the library's static device array), against cpattn_ring_bwd with a caller workspace.

Both run the same kernels in the same order, so the results must be equal bit for bit. Two
cases in a row on the same GPU, the second smaller than the first, so the second call finds
the first call's contents in the shared array; each case both overwrites NaN-filled
accumulators and adds into filled ones.
"""
import pytest
import torch

import context_causal_attention_cpattn_amd as cp
from workloads import draw_shape

from _util import gather, log

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (B, H, T, D, ring, rank): the first fills 2*8*2048 = 32768 rows of the array, the second 512
CASES = [(2, 8, 4096, 128, 2, 1), (1, 2, 1024, 64, 4, 2)]


def _setup(B, H, T, D, N, rank, seed):
    q, k, v, do = draw_shape(B, H, T, D, torch.bfloat16, seed=seed, n=4)
    maps, pos = zip(*[cp.cpattn_headtail_shard(T, N, r) for r in range(N)])
    kb = [gather(k, p) for p in pos]
    vb = [gather(v, p) for p in pos]
    qr, dor = gather(q, pos[rank]), gather(do, pos[rank])
    Tl = T // N
    o = torch.empty(B, H, Tl, D, device=DEV)
    lse = torch.empty(B, H, Tl, device=DEV)
    cp.cpattn_ring_fwd(qr, kb, vb, maps, rank, maps[rank], o, lse, None)
    return qr, kb, vb, maps, dor, o, lse


def _grads(shape, N, fill, seed):
    if fill is None:
        mk = lambda: torch.full(shape, float("nan"), device=DEV)
        return mk(), [mk() for _ in range(N)], [mk() for _ in range(N)]
    g = torch.Generator().manual_seed(seed)
    mk = lambda: torch.randn(shape, generator=g).to(DEV)
    return mk(), [mk() for _ in range(N)], [mk() for _ in range(N)]


def test_noalloc_equals_ring_bwd_on_two_calls_second_smaller():
    assert cp.NOALLOC_MAX_ROWS == 1 << 20
    for i, (B, H, T, D, N, rank) in enumerate(CASES):
        log(f"noalloc case B={B} H={H} T={T} D={D} ring={N} rank={rank}")
        assert B * H * (T // N) <= cp.NOALLOC_MAX_ROWS
        qr, kb, vb, maps, dor, o, lse = _setup(B, H, T, D, N, rank, seed=700 + i)
        shape = (B, H, T // N, D)
        ws = torch.empty(cp.cpattn_ring_bwd_workspace_bytes(B, H, T // N), dtype=torch.uint8, device=DEV)
        for accumulate in (False, True):
            fill = None if not accumulate else 1
            dq_r, dk_r, dv_r = _grads(shape, N, fill, 800 + i)
            cp.cpattn_ring_bwd(qr, kb, vb, maps, rank, maps[rank], dor, o, lse, dq_r, dk_r, dv_r, ws,
                               accumulate=accumulate)
            dq_n, dk_n, dv_n = _grads(shape, N, fill, 800 + i)
            cp.cpattn_ring_bwd_noalloc(qr, kb, vb, maps, rank, maps[rank], dor, o, lse, dq_n, dk_n, dv_n,
                                       accumulate=accumulate)
            torch.cuda.synchronize()
            assert not torch.isnan(dq_n).any()
            assert torch.equal(dq_n, dq_r), (i, accumulate, "dq")
            for j in range(N):
                assert torch.equal(dk_n[j], dk_r[j]) and torch.equal(dv_n[j], dv_r[j]), (i, accumulate, j)
        log(f"  equal bit for bit (overwrite and accumulate)")
