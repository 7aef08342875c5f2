"""Batch-aware sequence-parallel groups: which GPUs form a group and which
tokens each GPU holds.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

BASP page, Section IV-A/B (Algorithms 1 and 2, Figure 4): with N GPUs and a
micro-batch of B sequences of length L, the GPUs are cut into B groups of
K = N / B consecutive ranks (ranks gK .. gK + K - 1 form group g); group g
takes sequence g and its rank at local position l holds tokens
[l L/K, (l+1) L/K).  Each group then runs its own K-way all-to-all.

Readings where the page is silent:
  * K must be a whole number and L a multiple of K (the page assumes both);
  * B > N falls back to data parallelism: each rank then takes B/N whole
    sequences, rank r holding sequences [r B/N, (r+1) B/N) (B a multiple
    of N).
"""
from __future__ import annotations


def group_size(world: int, batch: int) -> int:
    """K, the ranks per group (1 under the data-parallel fallback)."""
    if world <= 0 or batch <= 0:
        raise ValueError("world and batch must be positive")
    if batch > world:
        if batch % world:
            raise ValueError("batch must be a multiple of world when batch > world")
        return 1
    if world % batch:
        raise ValueError("world must be a multiple of batch")
    return world // batch


def groups(world: int, batch: int) -> list:
    """The rank lists of the groups, consecutive ranks per group."""
    K = group_size(world, batch)
    return [list(range(g * K, (g + 1) * K)) for g in range(world // K)]


def shard(rank: int, world: int, batch: int, seq_len: int):
    """(seq_begin, seq_end, tok_begin, tok_end) held by ``rank``."""
    if not 0 <= rank < world:
        raise ValueError("rank out of range")
    if seq_len < 0:
        raise ValueError("seq_len must be >= 0")
    K = group_size(world, batch)
    if batch > world:
        per = batch // world
        return rank * per, (rank + 1) * per, 0, seq_len
    if seq_len % K:
        raise ValueError("seq_len must be a multiple of the group size")
    g, l = rank // K, rank % K
    chunk = seq_len // K
    return g, g + 1, l * chunk, (l + 1) * chunk
