"""Pins for the fp64 oracle: each check ties an oracle function to something
other than itself -- a worked example printed on the pages, a closed form, an
invariant, an independent library routine, brute force, or finite differences.

The ``mutant`` tests at the end plant plausible mistakes IN THE ORACLE (on the
CPU) and show that at least one pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, brute, gqa, merge, ring, rope, shard

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------- shard map

def test_shard_worked_example_from_log():
    g = json.load(open(os.path.join(GOLDEN, "headtail_worked_example.json")))
    assert shard.headtail_positions(g["T"], g["ring"], g["rank"]) == g["positions"]


@pytest.mark.parametrize("ring", [1, 2, 3, 4, 8])
def test_shard_chunk_pairs_and_permutation(ring):
    T = 2 * ring * 5
    c = T // (2 * ring)
    allpos = []
    for r in range(ring):
        pos = shard.headtail_positions(T, ring, r)
        assert pos[:c] == list(range(r * c, (r + 1) * c))
        last = 2 * ring - 1 - r
        assert pos[c:] == list(range(last * c, (last + 1) * c))
        L, split, d0, d1 = shard.headtail_deltas(T, ring, r)
        assert (L, split) == (2 * c, c)
        assert shard.positions_from_deltas(L, split, d0, d1) == pos
        assert d1 >= d0  # positions increase with the local index
        allpos += pos
    assert sorted(allpos) == list(range(T))


def test_shard_tiny_workload_chunks():
    # 4 chunks of 64 tokens; rank r holds chunks r and 3 - r.
    for r in range(2):
        pos = shard.headtail_positions(256, 2, r)
        assert pos == list(range(64 * r, 64 * r + 64)) + list(range(64 * (3 - r), 64 * (4 - r)))


@pytest.mark.parametrize("T,ring", [(256, 2), (4096, 4), (16384, 2), (48, 3)])
def test_shard_balance_exact(T, ring):
    # Every rank sees exactly T(T+1)/(2N) visible (q, k) pairs over the whole ring.
    tot = 0
    for r in range(ring):
        pairs = sum(p + 1 for p in shard.headtail_positions(T, ring, r))
        assert pairs * 2 * ring == T * (T + 1)
        tot += pairs
    assert 2 * tot == T * (T + 1)


@pytest.mark.parametrize("ring", [2, 3, 4])
def test_step_shapes(ring):
    # Dev log 2026-06-17: under zigzag/HeadTail a ring step is either the causal
    # diagonal (own block), all rows against the head half of the keys, or the
    # tail half of the rows against all keys.
    T = 2 * ring * 6
    c = T // (2 * ring)
    for r in range(ring):
        qp = np.array(shard.headtail_positions(T, ring, r))
        for src in range(ring):
            kp = np.array(shard.headtail_positions(T, ring, src))
            vis = kp[None, :] <= qp[:, None]
            if src == r:
                assert vis.sum() == c * (c + 1) // 2 + c * c + c * (c + 1) // 2
            elif src < r:
                assert vis[:, :c].all() and not vis[:, c:].any()
            else:
                assert vis[c:, :].all() and not vis[:c, :].any()


def test_ring_source_schedule():
    for n in (1, 2, 4, 5):
        for r in range(n):
            srcs = [shard.ring_source(r, s, n) for s in range(n)]
            assert srcs[0] == r and sorted(srcs) == list(range(n))


def test_shard_rejects_bad_sizes():
    with pytest.raises(ValueError):
        shard.headtail_positions(10, 2, 0)
    with pytest.raises(ValueError):
        shard.headtail_positions(8, 2, 2)


# --------------------------------------------------------------------------- forward

def _tolist(x):
    return [list(map(float, r)) for r in x]


@pytest.mark.parametrize("seed", range(4))
def test_fwd_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    Tq, Tk, D = 7, 9, 4
    q, k, v = rng.standard_normal((Tq, D)), rng.standard_normal((Tk, D)), rng.standard_normal((Tk, D))
    qpos = rng.permutation(20)[:Tq]
    kpos = rng.permutation(20)[:Tk]
    for causal in (True, False):
        O, L = attention.block_attention_fwd(q, k, v, qpos, kpos, causal=causal)
        Ob, Lb = brute.attention(_tolist(q), _tolist(k), _tolist(v), list(qpos), list(kpos), causal)
        np.testing.assert_allclose(O, np.array(Ob), atol=1e-13)
        Lb = np.array(Lb)
        assert np.array_equal(np.isinf(L), np.isinf(Lb))
        np.testing.assert_allclose(L[np.isfinite(L)], Lb[np.isfinite(Lb)], atol=1e-13)


def test_fwd_full_sequence_brute_force_T16():
    q, k, v = rnd(3, 16, 8, seed=1), rnd(3, 16, 8, seed=2), rnd(3, 16, 8, seed=3)
    O, L = attention.causal_attention_fwd(q, k, v)
    for h in range(3):
        Ob, Lb = brute.attention(_tolist(q[h]), _tolist(k[h]), _tolist(v[h]), list(range(16)), list(range(16)))
        np.testing.assert_allclose(O[h], Ob, atol=1e-13)
        np.testing.assert_allclose(L[h], Lb, atol=1e-13)


def test_fwd_matches_torch_sdpa_float64():
    # Independent library routine: torch's math SDPA in float64 with is_causal.
    q, k, v = (torch.from_numpy(rnd(2, 3, 40, 16, seed=s)) for s in (4, 5, 6))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    O, L = attention.causal_attention_fwd(q.numpy(), k.numpy(), v.numpy())
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)
    s = (q @ k.transpose(-1, -2)) / 4.0
    s = s.masked_fill(torch.ones(40, 40, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


def test_fwd_row0_closed_form():
    # Position 0 attends only to itself (dev log 2026-06-05): O_0 = v_0, LSE_0 = sigma q_0.k_0.
    q, k, v = rnd(2, 33, 8, seed=7), rnd(2, 33, 8, seed=8), rnd(2, 33, 8, seed=9)
    O, L = attention.causal_attention_fwd(q, k, v)
    np.testing.assert_allclose(O[:, 0], v[:, 0], atol=1e-14)
    np.testing.assert_allclose(L[:, 0], (q[:, 0] * k[:, 0]).sum(-1) / math.sqrt(8), atol=1e-14)


def test_fwd_zero_queries_closed_form():
    # q = 0: uniform weights over visible keys -> O_p = mean(v_0..v_p), LSE_p = ln(p+1).
    T = 50
    k, v = rnd(T, 8, seed=10), rnd(T, 8, seed=11)
    O, L = attention.causal_attention_fwd(np.zeros((T, 8)), k, v)
    np.testing.assert_allclose(O, np.cumsum(v, 0) / np.arange(1, T + 1)[:, None], atol=1e-13)
    np.testing.assert_allclose(L, np.log(np.arange(1, T + 1)), atol=1e-13)


def test_fwd_key_shift_invariance():
    # k -> k + 1 u^T leaves O unchanged and shifts LSE_p by sigma q_p.u.
    T, D = 40, 16
    q, k, v = rnd(T, D, seed=12), rnd(T, D, seed=13), rnd(T, D, seed=14)
    u = rnd(D, seed=15)
    O, L = attention.causal_attention_fwd(q, k, v)
    O2, L2 = attention.causal_attention_fwd(q, k + u[None, :], v)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2 - L, q @ u / math.sqrt(D), atol=1e-12)


def test_fwd_single_token_and_dead_rows():
    O, L = attention.causal_attention_fwd(rnd(1, 4, seed=16), rnd(1, 4, seed=17), rnd(1, 4, seed=18))
    assert O.shape == (1, 4) and np.isfinite(L).all()
    # all keys in the future: O = 0, LSE = -inf
    O, L = attention.block_attention_fwd(rnd(3, 4), rnd(5, 4), rnd(5, 4), [0, 1, 2], [5, 6, 7, 8, 9])
    assert (O == 0).all() and np.isneginf(L).all()


def test_fwd_rows_subset_matches_full():
    q, k, v = rnd(2, 64, 8, seed=19), rnd(2, 64, 8, seed=20), rnd(2, 64, 8, seed=21)
    rows = shard.headtail_positions(64, 2, 1)
    O, L = attention.causal_attention_fwd(q, k, v)
    Os, Ls = attention.causal_attention_fwd(q, k, v, rows=rows)
    np.testing.assert_array_equal(Os, O[:, rows])
    np.testing.assert_array_equal(Ls, L[:, rows])


# --------------------------------------------------------------------------- merge

def test_merge_matches_brute_and_identities():
    oa, ob, oc = rnd(6, 5, seed=22), rnd(6, 5, seed=23), rnd(6, 5, seed=24)
    la, lb, lc = rnd(6, seed=25), rnd(6, seed=26), rnd(6, seed=27)
    la[1] = -np.inf
    lb[2] = -np.inf
    la[3] = lb[3] = -np.inf
    o, l = merge.lse_merge(oa, la, ob, lb)
    obr, lbr = brute.merge(_tolist(oa), list(la), _tolist(ob), list(lb))
    np.testing.assert_allclose(o, obr, atol=1e-14)
    np.testing.assert_allclose(l, lbr, atol=1e-14)
    assert (o[3] == 0).all() and np.isneginf(l[3]) and not np.isnan(o).any()
    # identity
    o1, l1 = merge.lse_merge(oa, la, np.zeros_like(oa), np.full(6, -np.inf))
    np.testing.assert_array_equal(l1, la)
    np.testing.assert_allclose(o1[np.isfinite(la)], oa[np.isfinite(la)], atol=0)
    # commutative, associative
    o2, l2 = merge.lse_merge(ob, lb, oa, la)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_allclose(l2, l, atol=1e-14)
    x = merge.lse_merge(*merge.lse_merge(oa, la, ob, lb), oc, lc)
    y = merge.lse_merge(oa, la, *merge.lse_merge(ob, lb, oc, lc))
    np.testing.assert_allclose(x[0], y[0], atol=1e-14)
    np.testing.assert_allclose(x[1], y[1], atol=1e-14)


def test_merge_of_split_keys_equals_whole():
    # Splitting the keys of one softmax into two parts and merging recovers it.
    q, k, v = rnd(10, 8, seed=28), rnd(30, 8, seed=29), rnd(30, 8, seed=30)
    qpos, kpos = np.arange(20, 30), np.arange(30)
    O, L = attention.block_attention_fwd(q, k, v, qpos, kpos)
    a = attention.block_attention_fwd(q, k[:13], v[:13], qpos, kpos[:13])
    b = attention.block_attention_fwd(q, k[13:], v[13:], qpos, kpos[13:])
    o, l = merge.lse_merge(*a, *b)
    np.testing.assert_allclose(o, O, atol=1e-13)
    np.testing.assert_allclose(l, L, atol=1e-13)


@pytest.mark.parametrize("ring_n", [2, 3, 4])
def test_invariant_headtail_ring_equals_unsharded(ring_n):
    T = 2 * ring_n * 8
    q, k, v = rnd(2, 2, T, 8, seed=31), rnd(2, 2, T, 8, seed=32), rnd(2, 2, T, 8, seed=33)
    O, L = attention.causal_attention_fwd(q, k, v)
    assign = [shard.headtail_positions(T, ring_n, r) for r in range(ring_n)]
    for r in range(ring_n):
        o, l = ring.ring_forward(q, k, v, assign, r)
        np.testing.assert_allclose(o, O[..., assign[r], :], atol=1e-12)
        np.testing.assert_allclose(l, L[..., assign[r]], atol=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_invariant_any_partition_any_order(seed):
    # Any chunk partition of the sequence and any block order reproduce unsharded attention.
    rng = np.random.default_rng(200 + seed)
    T, n = 36, int(rng.integers(2, 6))
    perm = rng.permutation(T)
    cuts = np.sort(rng.choice(np.arange(1, T), n - 1, replace=False))
    assign = [list(map(int, p)) for p in np.split(perm, cuts)]
    q, k, v = rnd(1, 2, T, 4, seed=40 + seed), rnd(1, 2, T, 4, seed=50 + seed), rnd(1, 2, T, 4, seed=60 + seed)
    O, L = attention.causal_attention_fwd(q, k, v)
    for r in range(n):
        order = list(rng.permutation(n))
        o, l = ring.ring_forward(q, k, v, assign, r, order=order)
        np.testing.assert_allclose(o, O[..., assign[r], :], atol=1e-12)
        np.testing.assert_allclose(l, L[..., assign[r]], atol=1e-12)


# --------------------------------------------------------------------------- rope

def test_rope_identity_norm_and_textbook_rotation():
    x = rnd(5, 8, seed=70)
    np.testing.assert_allclose(rope.rope_apply(x, np.zeros(5), 10000.0), x, atol=0)
    y = rope.rope_apply(x, np.arange(5) * 1000, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)
    # D = 2: a plain 2-D rotation by pos radians (theta irrelevant: i = 0)
    x2 = rnd(4, 2, seed=71)
    pos = np.array([0.0, 1.0, 2.5, 37.0])
    for t in range(4):
        a = pos[t]
        R = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
        np.testing.assert_allclose(rope.rope_apply(x2[t:t + 1], pos[t:t + 1], 10000.0)[0], R @ x2[t], atol=1e-14)


def test_rope_matches_brute_and_complex_form():
    x = rnd(6, 8, seed=72)
    pos = [0, 3, 17, 100, 4095, 32767]
    y = rope.rope_apply(x, pos, 10000.0)
    np.testing.assert_allclose(y, brute.rope(_tolist(x), pos, 10000.0), atol=1e-12)
    z = (x[:, :4] + 1j * x[:, 4:]) * np.exp(1j * np.outer(pos, 10000.0 ** (-np.arange(4) / 4.0)))
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], 1), atol=1e-12)


def test_rope_relative_position_property():
    # Shifting every position by the same amount leaves causal attention unchanged.
    T, D = 24, 8
    q, k, v = rnd(T, D, seed=73), rnd(T, D, seed=74), rnd(T, D, seed=75)
    pos = np.arange(T)
    a = attention.block_attention_fwd(rope.rope_apply(q, pos, 10000.0), rope.rope_apply(k, pos, 10000.0), v, pos, pos)
    b = attention.block_attention_fwd(rope.rope_apply(q, pos + 777, 10000.0),
                                      rope.rope_apply(k, pos + 777, 10000.0), v, pos, pos)
    np.testing.assert_allclose(a[0], b[0], atol=1e-11)
    np.testing.assert_allclose(a[1], b[1], atol=1e-11)


# --------------------------------------------------------------------------- backward

def _loss(q, k, v, do):
    O, _ = attention.causal_attention_fwd(q, k, v)
    return float((O * do).sum())


def test_bwd_finite_differences():
    T, D = 6, 4
    q, k, v, do = rnd(T, D, seed=80), rnd(T, D, seed=81), rnd(T, D, seed=82), rnd(T, D, seed=83)
    dq, dk, dv, _, _ = attention.causal_attention_bwd(q, k, v, do)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for i in range(T):
            for d in range(D):
                xp, xm = x.copy(), x.copy()
                xp[i, d] += h
                xm[i, d] -= h
                args = {"q": q, "k": k, "v": v}
                ap, am = dict(args), dict(args)
                ap[name], am[name] = xp, xm
                num[i, d] = (_loss(ap["q"], ap["k"], ap["v"], do) - _loss(am["q"], am["k"], am["v"], do)) / (2 * h)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(g).max()), name


def _rope_loss(q, k, v, do, theta):
    pos = np.arange(q.shape[-2])
    O, _ = attention.causal_attention_fwd(rope.rope_apply(q, pos, theta), rope.rope_apply(k, pos, theta), v)
    return float((O * do).sum())


def test_rope_bwd_finite_differences():
    """Backward through the rotary: central differences of sum(dO * O(Rq, Rk, v)) with
    respect to the UNROTATED q, k, v (positions far apart so that every angle matters)."""
    T, D, theta = 6, 8, 10.0
    q, k, v, do = (rnd(T, D, seed=s) for s in (120, 121, 122, 123))
    dq, dk, dv = rope.rope_attention_bwd(q, k, v, do, theta)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for i in range(T):
            for d in range(D):
                xp, xm = x.copy(), x.copy()
                xp[i, d] += h
                xm[i, d] -= h
                args = {"q": q, "k": k, "v": v}
                ap, am = dict(args), dict(args)
                ap[name], am[name] = xp, xm
                num[i, d] = (_rope_loss(ap["q"], ap["k"], ap["v"], do, theta) -
                             _rope_loss(am["q"], am["k"], am["v"], do, theta)) / (2 * h)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(g).max()), name


def test_rope_transpose_is_the_inverse_rotation():
    x = rnd(2, 7, 16, seed=124)
    pos = np.array([0, 3, 17, 100, 4095, 9000, 32767])
    y = rope.rope_apply(x, pos, 10000.0)
    np.testing.assert_allclose(rope.rope_apply_transpose(y, pos, 10000.0), x, atol=1e-13)
    # the transpose of a rotation by a is the rotation by -a
    np.testing.assert_allclose(rope.rope_apply_transpose(x, pos, 10000.0), rope.rope_apply(x, -pos, 10000.0),
                               atol=1e-13)
    # and it preserves norms row by row
    np.testing.assert_allclose(np.linalg.norm(rope.rope_apply_transpose(x, pos, 10000.0), axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_mutant_rope_bwd_without_transpose_is_caught():
    # planted: the q gradient rotated forward by R instead of back by R^T
    T, D, theta = 6, 8, 10.0
    q, k, v, do = (rnd(T, D, seed=s) for s in (125, 126, 127, 128))
    pos = np.arange(T)
    dqr, _, _, _, _ = attention.causal_attention_bwd(rope.rope_apply(q, pos, theta), rope.rope_apply(k, pos, theta),
                                                     v, do)
    bad = rope.rope_apply(dqr, pos, theta)
    good, _, _ = rope.rope_attention_bwd(q, k, v, do, theta)
    assert np.abs(bad - good).max() > 1e-3


def _gqa_loss(q, k, v, do):
    T = q.shape[-2]
    O, _ = gqa.block_attention_fwd(q, k, v, np.arange(T), np.arange(T))
    return float((O * do).sum())


@pytest.mark.parametrize("H,H_kv", [(4, 2), (3, 1)])
def test_gqa_bwd_finite_differences(H, H_kv):
    """GQA / MQA: central differences of sum(dO * O) with respect to the SHARED K and V
    heads (each feeds several query heads) and to Q."""
    T, D = 5, 4
    q, do = rnd(1, H, T, D, seed=130), rnd(1, H, T, D, seed=131)
    k, v = rnd(1, H_kv, T, D, seed=132), rnd(1, H_kv, T, D, seed=133)
    pos = np.arange(T)
    o, lse = gqa.block_attention_fwd(q, k, v, pos, pos)
    dq, dk, dv = gqa.block_attention_bwd(q, k, v, do, o, lse, pos, pos)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            ap, am = dict(args), dict(args)
            ap[name], am[name] = xp, xm
            num[idx] = (_gqa_loss(ap["q"], ap["k"], ap["v"], do) - _gqa_loss(am["q"], am["k"], am["v"], do)) / (2 * h)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(g).max()), name


def test_gqa_groups_are_consecutive_heads_and_g1_is_mha():
    q, k, v = rnd(1, 6, 9, 8, seed=134), rnd(1, 2, 9, 8, seed=135), rnd(1, 2, 9, 8, seed=136)
    pos = np.arange(9)
    o, _ = gqa.block_attention_fwd(q, k, v, pos, pos)
    # query heads 0..2 use KV head 0, heads 3..5 KV head 1 (brute force per head)
    for h in range(6):
        ob, _ = brute.attention(_tolist(q[0, h]), _tolist(k[0, h // 3]), _tolist(v[0, h // 3]), list(pos), list(pos))
        np.testing.assert_allclose(o[0, h], np.array(ob), atol=1e-12)
    k6, v6 = rnd(1, 6, 9, 8, seed=137), rnd(1, 6, 9, 8, seed=138)
    o1, l1 = gqa.block_attention_fwd(q, k6, v6, pos, pos)
    o2, l2 = attention.block_attention_fwd(q, k6, v6, pos, pos)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_mutant_gqa_strided_grouping_is_caught():
    # planted: query head h paired with KV head h % H_kv instead of h // G
    q, k, v = rnd(1, 4, 7, 8, seed=139), rnd(1, 2, 7, 8, seed=140), rnd(1, 2, 7, 8, seed=141)
    pos = np.arange(7)
    good, _ = gqa.block_attention_fwd(q, k, v, pos, pos)
    bad, _ = attention.block_attention_fwd(q, np.tile(k, (1, 2, 1, 1)), np.tile(v, (1, 2, 1, 1)), pos, pos)
    assert np.abs(good - bad).max() > 1e-3


@pytest.mark.parametrize("H,H_kv", [(4, 2), (4, 1)])
def test_gqa_causal_bwd_matches_torch_autograd(H, H_kv):
    """gqa.causal_attention_bwd against torch float64 autograd of SDPA over K / V heads
    gathered per query head (the gather's backward sums each KV head's group: an independent
    library route to the group reduce of the log's 2026-07-01 entry)."""
    T, D = 33, 8
    q, do = (torch.from_numpy(rnd(2, H, T, D, seed=s)) for s in (170, 171))
    k, v = (torch.from_numpy(rnd(2, H_kv, T, D, seed=s)) for s in (172, 173))
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    idx = torch.arange(H) // (H // H_kv)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt[:, idx], vt[:, idx], is_causal=True)
    out.backward(do)
    dq, dk, dv, o, lse = gqa.causal_attention_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy())
    np.testing.assert_allclose(o, out.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-12)


def test_gqa_causal_bwd_finite_differences_shared_kv():
    """gqa.causal_attention_bwd on the full sequence: central differences with respect to
    the shared K and V heads (MQA, G = 3) and to q."""
    H, H_kv, T, D = 3, 1, 5, 4
    q, do = rnd(1, H, T, D, seed=174), rnd(1, H, T, D, seed=175)
    k, v = rnd(1, H_kv, T, D, seed=176), rnd(1, H_kv, T, D, seed=177)
    dq, dk, dv, _, _ = gqa.causal_attention_bwd(q, k, v, do)

    def loss(qq, kk, vv):
        # per query head, brute force against the KV head of its group
        tot = []
        for hq in range(H):
            O, _ = brute.attention(_tolist(qq[0, hq]), _tolist(kk[0, hq * H_kv // H]),
                                   _tolist(vv[0, hq * H_kv // H]), list(range(T)), list(range(T)))
            tot += [o * g for orow, grow in zip(O, _tolist(do[0, hq])) for o, g in zip(orow, grow)]
        return math.fsum(tot)

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            ap, am = dict(args), dict(args)
            ap[name], am[name] = xp, xm
            num[idx] = (loss(ap["q"], ap["k"], ap["v"]) - loss(am["q"], am["k"], am["v"])) / (2 * h)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(g).max()), name


def test_mutant_gqa_group_mean_is_caught():
    # planted: the group reduce takes the mean over a group's query heads instead of the
    # sum; the torch-autograd pin above rejects it
    H, H_kv, T, D = 4, 2, 9, 4
    q, do = (torch.from_numpy(rnd(1, H, T, D, seed=s)) for s in (178, 179))
    k, v = (torch.from_numpy(rnd(1, H_kv, T, D, seed=s)) for s in (180, 181))
    kt, vt = (x.clone().requires_grad_(True) for x in (k, v))
    idx = torch.arange(H) // (H // H_kv)
    torch.nn.functional.scaled_dot_product_attention(q, kt[:, idx], vt[:, idx], is_causal=True).backward(do)
    _, dk_h, dv_h, _, _ = attention.causal_attention_bwd(q.numpy(), gqa.expand_kv(k.numpy(), H),
                                                         gqa.expand_kv(v.numpy(), H), do.numpy())
    bad_dv = dv_h.reshape(1, H_kv, H // H_kv, T, D).mean(axis=2)
    assert np.abs(bad_dv - vt.grad.numpy()).max() > 1e-3


def test_bwd_matches_torch_autograd_float64():
    q, k, v, do = (torch.from_numpy(rnd(1, 2, 30, 8, seed=s)) for s in (84, 85, 86, 87))
    qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    out.backward(do)
    dq, dk, dv, _, _ = attention.causal_attention_bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy())
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-12)


def test_bwd_sum_identities():
    # sum_j dS_pj = 0 for every row  =>  sum_j dK_j = 0 ; sum_j dV_j = sum_p dO_p
    q, k, v, do = rnd(2, 40, 8, seed=88), rnd(2, 40, 8, seed=89), rnd(2, 40, 8, seed=90), rnd(2, 40, 8, seed=91)
    dq, dk, dv, _, _ = attention.causal_attention_bwd(q, k, v, do)
    np.testing.assert_allclose(dk.sum(axis=-2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=-2), do.sum(axis=-2), atol=1e-12)


def test_bwd_scale_symmetry():
    # S depends on q and k only through q.k: the output is unchanged under q -> a q, k -> k / a,
    # so d/da at a = 1 gives sum_p q_p.dQ_p = sum_j k_j.dK_j (per head, causal or not)
    q, k, v, do = rnd(2, 40, 8, seed=96), rnd(2, 40, 8, seed=97), rnd(2, 40, 8, seed=98), rnd(2, 40, 8, seed=99)
    dq, dk, _, _, _ = attention.causal_attention_bwd(q, k, v, do)
    lhs, rhs = (q * dq).sum(axis=(-2, -1)), (k * dk).sum(axis=(-2, -1))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    # the GPU tests check this at full size on every head: a dQ off by 1 % on one row breaks it
    bad = dq.copy()
    bad[1, 17] *= 1.01
    assert np.abs((q * bad).sum(axis=(-2, -1)) - rhs).max() > 1e-6 * np.abs(q * dq).sum()


@pytest.mark.parametrize("ring_n", [2, 3])
def test_bwd_ring_accumulated_equals_unsharded(ring_n):
    # dev log 2026-06-05: the two-rank ring gradient equals the single-pass gradient.
    T = 2 * ring_n * 6
    q, k, v, do = (rnd(1, 2, T, 8, seed=s) for s in (92, 93, 94, 95))
    dq, dk, dv, _, _ = attention.causal_attention_bwd(q, k, v, do)
    assign = [shard.headtail_positions(T, ring_n, r) for r in range(ring_n)]
    rq, rk, rv = ring.ring_backward(q, k, v, do, assign)
    np.testing.assert_allclose(rq, dq, atol=1e-12)
    np.testing.assert_allclose(rk, dk, atol=1e-12)
    np.testing.assert_allclose(rv, dv, atol=1e-12)


def _dq_from_row_term(q, k, v, do, row_term):
    """dQ of full-sequence causal attention (one head) with the softmax-backward row term
    supplied by ``row_term(do, o)``; everything else from the oracle's forward."""
    T, D = q.shape
    sig = 1.0 / math.sqrt(D)
    O, L = attention.causal_attention_fwd(q, k, v)
    P = np.exp(sig * (q @ k.T) - L[:, None]) * np.tri(T)
    dS = P * ((do @ v.T) - row_term(do, O)[:, None])
    return sig * (dS @ k)


def _fd_grad_q(q, k, v, do, h=1e-6):
    """Central differences of sum(dO * O) with respect to q (O from brute force)."""
    T, D = q.shape
    pos = list(range(T))

    def loss(qq):
        O, _ = brute.attention(_tolist(qq), _tolist(k), _tolist(v), pos, pos)
        return math.fsum(o * g for orow, grow in zip(O, _tolist(do)) for o, g in zip(orow, grow))

    num = np.zeros_like(q)
    for i in range(T):
        for d in range(D):
            qp, qm = q.copy(), q.copy()
            qp[i, d] += h
            qm[i, d] -= h
            num[i, d] = (loss(qp) - loss(qm)) / (2 * h)
    return num


def test_delta_pinned_by_finite_differences():
    # The row term D_p of the softmax backward (the log's 2026-03-24 "Di correction"): with
    # attention.delta as the row term, dQ matches central differences of sum(dO * O) taken
    # through the brute-force forward.
    T, D = 7, 4
    q, k, v, do = (rnd(T, D, seed=s) for s in (150, 151, 152, 153))
    got = _dq_from_row_term(q, k, v, do, attention.delta)
    num = _fd_grad_q(q, k, v, do)
    assert np.abs(got - num).max() <= 1e-6 * max(1.0, np.abs(num).max())


def test_delta_equals_probability_weighted_dp():
    # D_p = sum_j P_pj (dO_p . v_j): the expectation of dP under the row's softmax, with
    # P from pure-Python brute force (no numpy), for causal rows at global positions.
    rng = np.random.default_rng(154)
    Tq, Tk, D = 6, 9, 4
    q, k, v, do = (rng.standard_normal((n, D)) for n in (Tq, Tk, Tk, Tq))
    qpos, kpos = [3, 4, 5, 12, 13, 14], list(range(9))
    O, L = brute.attention(_tolist(q), _tolist(k), _tolist(v), qpos, kpos)
    sig = 1.0 / math.sqrt(D)
    want = []
    for p in range(Tq):
        terms = []
        for j in range(Tk):
            if kpos[j] > qpos[p]:
                continue
            s = sig * math.fsum(q[p, d] * k[j, d] for d in range(D))
            terms.append(math.exp(s - L[p]) * math.fsum(do[p, d] * v[j, d] for d in range(D)))
        want.append(math.fsum(terms))
    np.testing.assert_allclose(attention.delta(do, np.array(O)), want, atol=1e-13)


def test_mutant_delta_from_block_output_is_caught():
    # planted: the row term taken from the output of the first key block only instead of
    # the final merged output -- the mistake the log's 2026-03-24 entry corrects
    T, D = 7, 4
    q, k, v, do = (rnd(T, D, seed=s) for s in (155, 156, 157, 158))
    split = 3
    pos = np.arange(T)
    O_blk, _ = attention.block_attention_fwd(q, k[:split], v[:split], pos, pos[:split])
    bad = _dq_from_row_term(q, k, v, do, lambda d, o: attention.delta(d, O_blk))
    num = _fd_grad_q(q, k, v, do)
    assert np.abs(bad - num).max() > 1e-3


def test_mutant_delta_summed_over_rows_is_caught():
    # planted: the product summed over the rows (axis -2) and broadcast back
    T, D = 7, 7
    q, k, v, do = (rnd(T, D, seed=s) for s in (159, 160, 161, 162))
    bad = _dq_from_row_term(q, k, v, do, lambda d, o: (d * o).sum(axis=-2))
    num = _fd_grad_q(q, k, v, do)
    assert np.abs(bad - num).max() > 1e-3


# --------------------------------------------------------------------------- planted mistakes

def _mut_fwd_strict_mask(q, k, v, qpos, kpos, causal=True, scale=None):
    # planted: a key at the same position is hidden (strict < instead of <=)
    return attention.block_attention_fwd(q, k, v, np.asarray(qpos) - 1, kpos, causal, scale)


def _mut_fwd_no_scale(q, k, v, qpos, kpos, causal=True, scale=None):
    return attention.block_attention_fwd(q, k, v, qpos, kpos, causal, 1.0)


def _mut_fwd_transposed(q, k, v, qpos, kpos, causal=True, scale=None):
    # planted: values taken from the keys
    return attention.block_attention_fwd(q, k, k, qpos, kpos, causal, scale)


@pytest.mark.parametrize("mutant", [_mut_fwd_strict_mask, _mut_fwd_no_scale, _mut_fwd_transposed])
def test_mutant_forward_is_caught(mutant):
    rng = np.random.default_rng(300)
    q, k, v = rng.standard_normal((7, 4)), rng.standard_normal((9, 4)), rng.standard_normal((9, 4))
    qpos, kpos = np.arange(7) + 2, np.arange(9)
    O, L = mutant(q, k, v, qpos, kpos)
    Ob, Lb = brute.attention(_tolist(q), _tolist(k), _tolist(v), list(qpos), list(kpos))
    assert not np.allclose(O, np.array(Ob), atol=1e-6)


def test_mutant_merge_sign_is_caught():
    oa, ob = rnd(4, 3, seed=98), rnd(4, 3, seed=99)
    la, lb = rnd(4, seed=100), rnd(4, seed=101)
    # planted: weights exp(L - L_x) instead of exp(L_x - L)
    m = np.maximum(la, lb)
    lse = m + np.log(np.exp(la - m) + np.exp(lb - m))
    bad = np.exp(lse - la)[:, None] * oa + np.exp(lse - lb)[:, None] * ob
    good, _ = brute.merge(_tolist(oa), list(la), _tolist(ob), list(lb))
    assert not np.allclose(bad, good, atol=1e-6)


def test_mutant_rope_pairing_is_caught():
    # planted: adjacent pairs (2i, 2i+1) instead of (i, i + D/2)
    x = rnd(3, 8, seed=102)
    pos = [0, 5, 9]
    a = rope.rope_angles(pos, 8, 10000.0)
    x1, x2 = x[:, 0::2], x[:, 1::2]
    y = np.empty_like(x)
    y[:, 0::2] = x1 * np.cos(a) - x2 * np.sin(a)
    y[:, 1::2] = x2 * np.cos(a) + x1 * np.sin(a)
    assert not np.allclose(y, np.array(brute.rope(_tolist(x), pos, 10000.0)), atol=1e-6)


def test_mutant_bwd_missing_delta_is_caught():
    # planted: dS = P dP (the D_p term dropped) -> dK no longer sums to zero
    T, D = 12, 4
    q, k, v, do = (rnd(T, D, seed=s) for s in (103, 104, 105, 106))
    O, L = attention.causal_attention_fwd(q, k, v)
    s = (q @ k.T) / 2.0
    p = np.exp(s - L[:, None]) * np.tri(T)
    ds = p * (do @ v.T)
    dk_bad = (ds.T @ q) / 2.0
    assert np.abs(dk_bad.sum(0)).max() > 1e-3
