"""Pins of the oracle's GQA-aware Ulysses packs and of the batch-aware groups.

The kv-head split is pinned end to end: P emulated ranks pack their token
shards, exchange chunks as an all-to-all would, run ordinary attention on the
heads they received and send the results back; that must reproduce global
GQA attention (and its gradients) of the whole sequence.  The bf16 rounding of
the gradient sum is pinned against torch's own float -> bfloat16 conversion.
"""
import numpy as np
import pytest
import torch

from oracle.attention import attn_fwd, attn_bwd
from oracle.permute import (seq2head, head2seq, rank_kv_heads, kv_seq2head, kv_head2seq_sum,
                            round_to_bf16, qkv_seq2head, qkv_head2seq)
from oracle import sp_groups


def _exchange(sent, P):
    """sent[s][p] is what rank s sends to rank p; returns what each rank receives, stacked
    over sources along the token axis."""
    return [np.concatenate([sent[s][p] for s in range(P)], axis=0) for p in range(P)]


SPLITS = [  # (P, Hq, Hkv)
    (2, 4, 4), (4, 8, 2), (8, 32, 4), (8, 16, 8), (4, 8, 8), (8, 8, 1), (2, 8, 1), (4, 16, 16),
]


@pytest.mark.parametrize("P,Hq,Hkv", SPLITS)
def test_rank_kv_heads_cover_every_kv_head(P, Hq, Hkv):
    heads = [rank_kv_heads(p, P, Hq, Hkv) for p in range(P)]
    # each rank's query heads read only the kv heads it holds
    hq = Hq // P
    for p in range(P):
        for h in range(p * hq, (p + 1) * hq):
            assert h * Hkv // Hq in heads[p]
    # every kv head is held somewhere, and by P/Hkv ranks when Hkv < P
    count = np.zeros(Hkv, dtype=int)
    for hs in heads:
        for g in hs:
            count[g] += 1
    assert (count == max(1, P // Hkv)).all()


def test_kv_pack_of_mha_is_the_plain_pack(rng):
    x = rng.standard_normal((9, 8, 4))
    assert np.array_equal(kv_seq2head(x, 4, 8), seq2head(x, 4))
    y = rng.standard_normal((4, 9, 2, 4))
    assert np.array_equal(kv_head2seq_sum(y, 8, 8), head2seq(y))


@pytest.mark.parametrize("P,Hq,Hkv", SPLITS)
@pytest.mark.parametrize("causal", [True, False])
def test_ulysses_emulation_reproduces_global_gqa_attention(rng, P, Hq, Hkv, causal):
    n, d = 5, 8
    N = P * n
    cu = np.array([0, 3, N - 4, N])            # documents cross the rank boundaries
    q = rng.standard_normal((N, Hq, d))
    k = rng.standard_normal((N, Hkv, d))
    v = rng.standard_normal((N, Hkv, d))
    do = rng.standard_normal((N, Hq, d))
    o_ref, lse_ref = attn_fwd(q, k, v, cu, cu, causal)
    dq_ref, dk_ref, dv_ref = attn_bwd(q, k, v, do, cu, cu, causal)

    rows = [slice(s * n, (s + 1) * n) for s in range(P)]
    packs = [qkv_seq2head(q[r], k[r], v[r], P) for r in rows]
    qp = _exchange([pk[0] for pk in packs], P)
    kp = _exchange([pk[1] for pk in packs], P)
    vp = _exchange([pk[2] for pk in packs], P)
    dop = _exchange([seq2head(do[r], P) for r in rows], P)
    # rank p: ordinary attention over its heads of the whole sequence
    res = [attn_bwd(qp[p], kp[p], vp[p], dop[p], cu, cu, causal, return_fwd=True)
           for p in range(P)]
    o_back = [head2seq(np.stack([res[p][3][rows[s]] for p in range(P)])) for s in range(P)]
    lse_back = np.concatenate([res[p][4] for p in range(P)], axis=0)       # heads in rank order
    assert np.allclose(np.concatenate(o_back), o_ref, atol=1e-12)
    assert np.allclose(lse_back, lse_ref, atol=1e-12)
    # gradients go back through the inverse exchange, kv gradients summed over replicas
    for s in range(P):
        dq_s, dk_s, dv_s = qkv_head2seq(np.stack([res[p][0][rows[s]] for p in range(P)]),
                                        np.stack([res[p][1][rows[s]] for p in range(P)]),
                                        np.stack([res[p][2][rows[s]] for p in range(P)]), Hkv)
        assert np.allclose(dq_s, dq_ref[rows[s]], atol=1e-11)
        assert np.allclose(dk_s, dk_ref[rows[s]], atol=1e-11)
        assert np.allclose(dv_s, dv_ref[rows[s]], atol=1e-11)


@pytest.mark.parametrize("P,Hq,Hkv", SPLITS)
def test_kv_unpack_is_the_adjoint_of_the_pack(rng, P, Hq, Hkv):
    x = rng.standard_normal((6, Hkv, 3))
    y = rng.standard_normal((P, 6, max(1, Hkv // P), 3))
    lhs = np.sum(kv_seq2head(x, P, Hq) * y)
    rhs = np.sum(x * kv_head2seq_sum(y, Hq, Hkv))
    assert abs(lhs - rhs) < 1e-12 * (1 + abs(lhs))


def _bf16_values(rng, shape):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(
        torch.bfloat16).float().numpy()


def test_round_to_bf16_matches_torch(rng):
    a = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(
        -20, 20, 4000), np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                                  3.0e38, 1e-40], dtype=np.float32)]).astype(np.float32)
    mine = round_to_bf16(a)
    lib = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    assert np.array_equal(mine.view(np.uint32), lib.view(np.uint32))


@pytest.mark.parametrize("P,Hq,Hkv", [(8, 32, 4), (8, 8, 1), (8, 32, 2), (4, 8, 8)])
def test_kv_round_trip_sums_replicas_exactly(rng, P, Hq, Hkv):
    # a kv head held by r ranks comes back as r * x; in float32 that sum is
    # exact for bf16 x, so only the final rounding to bf16 remains
    r = max(1, P // Hkv)
    x = _bf16_values(rng, (7, Hkv, 16))
    back = kv_head2seq_sum(kv_seq2head(x, P, Hq), Hq, Hkv, round_bf16=True)
    want = torch.from_numpy(r * x.astype(np.float64)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(back.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("P,Hq,Hkv", [(4, 6, 3), (3, 6, 2), (8, 12, 3), (4, 2, 2), (0, 4, 4)])
def test_bad_head_splits_are_rejected(rng, P, Hq, Hkv):
    with pytest.raises(ValueError):
        kv_seq2head(rng.standard_normal((2, Hkv, 2)), P, Hq)


# ------------------------------------------------------------ batch-aware groups
def test_basp_figure4_groups():
    # N = 4 GPUs, B = 2 sequences: two groups of K = 2 consecutive ranks
    assert sp_groups.groups(4, 2) == [[0, 1], [2, 3]]
    L = 16
    assert [sp_groups.shard(r, 4, 2, L) for r in range(4)] == [
        (0, 1, 0, 8), (0, 1, 8, 16), (1, 2, 0, 8), (1, 2, 8, 16)]


@pytest.mark.parametrize("N,B", [(1, 1), (8, 1), (8, 2), (8, 4), (8, 8), (6, 3), (4, 8), (2, 6),
                                 (16, 4)])
def test_basp_shards_partition_the_batch(N, B):
    L = 24
    held = {}
    K = sp_groups.group_size(N, B)
    for r in range(N):
        s0, s1, t0, t1 = sp_groups.shard(r, N, B, L)
        for s in range(s0, s1):
            for t in range(t0, t1):
                assert (s, t) not in held
                held[(s, t)] = r
        # the per-GPU footprint is B L / N tokens, as with an N-way split of all sequences
        assert (s1 - s0) * (t1 - t0) == B * L // N
    assert len(held) == B * L
    for g, ranks in enumerate(sp_groups.groups(N, B)):
        assert len(ranks) == K and ranks == list(range(ranks[0], ranks[0] + K))
        seqs = {sp_groups.shard(r, N, B, L)[:2] for r in ranks}
        assert len(seqs) == 1                      # a group shares its sequence(s)
        starts = [sp_groups.shard(r, N, B, L)[2] for r in ranks]
        assert starts == sorted(starts)            # local rank order follows token order


@pytest.mark.parametrize("args", [(4, 3, 12), (3, 2, 12), (8, 2, 10), (4, 6, 8), (0, 1, 4)])
def test_basp_rejects_non_divisible(args):
    N, B, L = args
    with pytest.raises(ValueError):
        for r in range(max(N, 1)):
            sp_groups.shard(r, N, B, L)
