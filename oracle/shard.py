"""HeadTail (load-balanced) shard map, written from its definition.

Source: BluScriptCP development log.
  * entry of 2026-05-16 on the HeadTail kernel: the permutation works on whole
    chunks, replacing the token-level interleave of the 2026-03-23 entry;
  * entry of 2026-06-29 on fused-RoPE load balancing: Megatron's per-rank
    rotary slice takes chunks r and 2*cp-1-r;
  * entry of 2026-06-29 on RopeDeltas.h: the worked example with two ranks and
    eight tokens, where rank 0 holds global positions 0, 1, 6 and 7;
  * entry of 2026-07-10 (fused-RoPE Phase 3): a local index i sits at global
    position i + d1 when i is in the second half of the shard, else i + d0.

NeMo Automodel PR #2931 (squashed commit log, CPSharder commit) pairs chunks
the same way (round-robin head/tail pairs of 2*cp chunks).
"""
from __future__ import annotations


def chunk_size(T: int, ring: int) -> int:
    if ring < 1 or T % (2 * ring) != 0:
        raise ValueError("T must be a positive multiple of 2 * ring")
    return T // (2 * ring)


def headtail_chunks(ring: int, rank: int) -> tuple[int, int]:
    """The two chunk indices rank ``rank`` holds, head chunk first."""
    if not 0 <= rank < ring:
        raise ValueError("rank out of range")
    return rank, 2 * ring - 1 - rank


def headtail_positions(T: int, ring: int, rank: int) -> list[int]:
    """Global token positions of rank ``rank``'s shard, in local order."""
    c = chunk_size(T, ring)
    a, b = headtail_chunks(ring, rank)
    return list(range(a * c, (a + 1) * c)) + list(range(b * c, (b + 1) * c))


def headtail_deltas(T: int, ring: int, rank: int) -> tuple[int, int, int, int]:
    """(len, split, d0, d1) with position(i) = i + (d0 if i < split else d1)."""
    c = chunk_size(T, ring)
    a, b = headtail_chunks(ring, rank)
    # head chunk: local i in [0, c) sits at a*c + i ; tail: local i in [c, 2c) at b*c + (i - c)
    return 2 * c, c, a * c, b * c - c


def positions_from_deltas(length: int, split: int, d0: int, d1: int) -> list[int]:
    return [i + (d0 if i < split else d1) for i in range(length)]


def ring_source(rank: int, step: int, ring: int) -> int:
    """Owner of the KV block rank ``rank`` holds at ring step ``step``.

    Reading: blocks travel to the next rank each step (send to r+1, receive
    from r-1), so at step s rank r holds the block that started on r-s.
    The exact result does not depend on this order; only rounding does.
    """
    return (rank - step) % ring
