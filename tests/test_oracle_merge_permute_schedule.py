"""Pins of the oracle's merge, permute and scheduler."""
import os

import numpy as np
import pytest

from oracle.attention import attn_fwd
from oracle.merge import lse_merge
from oracle.permute import seq2head, head2seq
from oracle import schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- merge
def test_merge_single_partial_is_identity(rng):
    o = rng.standard_normal((10, 3, 4))
    lse = rng.standard_normal((3, 10))
    om, lm = lse_merge([o], [lse])
    assert np.allclose(om, o, atol=1e-15) and np.allclose(lm, lse, atol=1e-15)


def test_merge_with_empty_partial_changes_nothing(rng):
    o1, o2 = rng.standard_normal((2, 8, 2, 4))
    l1, l2 = rng.standard_normal((2, 2, 8))
    ref = lse_merge([o1, o2], [l1, l2])
    junk = rng.standard_normal((8, 2, 4)) * 1e3
    got = lse_merge([o1, junk, o2], [l1, np.full((2, 8), -np.inf), l2])
    assert np.allclose(got[0], ref[0], atol=1e-14) and np.allclose(got[1], ref[1], atol=1e-14)


def test_merge_all_empty_gives_zero_and_neg_inf(rng):
    o = rng.standard_normal((4, 1, 2))
    om, lm = lse_merge([o, o], [np.full((1, 4), -np.inf)] * 2)
    assert np.all(om == 0) and np.all(np.isneginf(lm))


def test_merge_order_invariant(rng):
    parts = [rng.standard_normal((6, 2, 3)) for _ in range(5)]
    lses = [rng.standard_normal((2, 6)) * 4 for _ in range(5)]
    a = lse_merge(parts, lses)
    perm = rng.permutation(5)
    b = lse_merge([parts[i] for i in perm], [lses[i] for i in perm])
    assert np.allclose(a[0], b[0], atol=1e-13) and np.allclose(a[1], b[1], atol=1e-13)


def test_merge_of_ring_partials_equals_full_attention(rng):
    # 4 chunks of 16; query chunk 3; chunks 0..2 unmasked, chunk 3 causal
    n, c, h, d = 4, 16, 2, 8
    L = n * c
    q = rng.standard_normal((L, h, d))
    k = rng.standard_normal((L, h, d))
    v = rng.standard_normal((L, h, d))
    full_o, full_l = attn_fwd(q, k, v, [0, L], [0, L])
    qc = q[3 * c:]
    os_, ls_ = [], []
    for j in range(n):
        o_p, l_p = attn_fwd(qc, k[j * c:(j + 1) * c], v[j * c:(j + 1) * c], [0, c], [0, c],
                            causal=(j == 3))
        os_.append(o_p)
        ls_.append(l_p)
    om, lm = lse_merge(os_, ls_)
    assert np.allclose(om, full_o[3 * c:], atol=1e-12) and np.allclose(lm, full_l[:, 3 * c:], atol=1e-12)


# ---------------------------------------------------------------- permute
@pytest.mark.parametrize("P,H", [(1, 4), (2, 4), (4, 8), (8, 32), (3, 6)])
def test_permute_inverse(rng, P, H):
    x = rng.standard_normal((11, H, 5))
    y = seq2head(x, P)
    assert y.shape == (P, 11, H // P, 5)
    assert np.array_equal(head2seq(y), x)


def test_permute_rejects_bad_degree(rng):
    with pytest.raises(ValueError):
        seq2head(rng.standard_normal((3, 6, 2)), 4)


@pytest.mark.parametrize("P", [2, 4, 8])
def test_permute_all_to_all_emulation(rng, P):
    # IntraSP: P ranks each hold n tokens x H heads; after the all-to-all rank g
    # holds all N = P n tokens for heads [g h, (g+1) h), h = H / P.
    n, H, d = 7, 16, 3
    N, h = P * n, 16 // P
    X = rng.standard_normal((N, H, d))
    shards = [X[r * n:(r + 1) * n] for r in range(P)]
    sent = [seq2head(s, P) for s in shards]               # rank r's P outgoing chunks
    for g in range(P):
        recv = np.concatenate([sent[r][g] for r in range(P)], axis=0)   # [N, h, d]
        assert np.array_equal(recv, X[:, g * h:(g + 1) * h, :])
    # and back: rank g returns chunk r (its rows of source rank r) to rank r
    outs = [X[:, g * h:(g + 1) * h, :] for g in range(P)]
    for r in range(P):
        back = np.stack([outs[g][r * n:(r + 1) * n] for g in range(P)])  # [P, n, h, d]
        assert np.array_equal(head2seq(back), shards[r])
    # bytes held per rank are unchanged by the exchange
    assert sum(s.nbytes for s in sent) == X.nbytes


# ---------------------------------------------------------------- schedule
def _brute_cover(cu_q, cu_k, causal, bq, bk, items, col):
    docs = schedule.doc_table(cu_q, cu_k)
    cover = {}
    for it in items:
        b = int(it[0])
        _, lq, _, lk = docs[b]
        if col == "fwd":
            t = int(it[1])
            tiles = [(t, j) for j in range(int(it[2]), int(it[2]) + int(it[3]))]
        else:
            j = int(it[1])
            tiles = [(t, j) for t in range(int(it[2]), int(it[2]) + int(it[3]))]
        for t, j in tiles:
            any_vis = False
            for i in range(t * bq, min(lq, (t + 1) * bq)):
                for kk in range(j * bk, min(lk, (j + 1) * bk)):
                    if (not causal) or kk <= i + lk - lq:
                        cover[(b, i, kk)] = cover.get((b, i, kk), 0) + 1
                        any_vis = True
            assert any_vis, "an issued tile holds no visible pair"
    expect = set()
    for b, (_, lq, _, lk) in enumerate(docs):
        for i in range(lq):
            for kk in range(lk):
                if (not causal) or kk <= i + lk - lq:
                    expect.add((b, i, kk))
    assert set(cover) == expect
    assert all(c == 1 for c in cover.values())


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("bq,bk", [(4, 4), (8, 4), (4, 8), (16, 16)])
def test_schedule_covers_each_visible_pair_once(rng, causal, bq, bk):
    for _ in range(4):
        lq = rng.integers(0, 40, size=5)
        lk = lq.copy() if rng.random() < 0.5 else rng.integers(0, 40, size=5)
        cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        f = schedule.fwd_items(cq, ck, causal, bq, bk)
        bw = schedule.bwd_items(cq, ck, causal, bq, bk)
        _brute_cover(cq, ck, causal, bq, bk, [x for x in f if x[3] > 0], "fwd")
        _brute_cover(cq, ck, causal, bq, bk, [x for x in bw if x[3] > 0], "bwd")
        # every query tile of every doc is listed (so empty rows are written)
        assert len(f) == sum(-(-int(x) // bq) for x in lq)
        assert len(bw) == sum(-(-int(x) // bk) for x in lk)
        # longest first, ties by (doc, tile)
        keys = [(-int(x[3]), int(x[0]), int(x[1])) for x in f]
        assert keys == sorted(keys)


def _brute_issued_area(items, bq, bk, col):
    """Cells of the issued tiles, enumerated one by one (tile cells past a
    document's end included: the area the kernels compute)."""
    n = 0
    for it in items:
        if col == "fwd":
            tiles = [(int(it[1]), j) for j in range(int(it[2]), int(it[2]) + int(it[3]))]
        else:
            tiles = [(t, int(it[1])) for t in range(int(it[2]), int(it[2]) + int(it[3]))]
        for t, j in tiles:
            for _i in range(t * bq, (t + 1) * bq):
                for _kk in range(j * bk, (j + 1) * bk):
                    n += 1
    return n


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("bq,bk", [(4, 8), (8, 4), (3, 5)])
def test_issued_pairs_equals_enumerated_tile_area(rng, causal, bq, bk):
    for _ in range(4):
        lq = rng.integers(0, 30, size=4)
        lk = lq.copy() if rng.random() < 0.5 else rng.integers(0, 30, size=4)
        cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        f = schedule.fwd_items(cq, ck, causal, bq, bk)
        bw = schedule.bwd_items(cq, ck, causal, bq, bk)
        assert schedule.issued_pairs(f, bq, bk) == _brute_issued_area(f, bq, bk, "fwd")
        assert schedule.issued_pairs(bw, bq, bk) == _brute_issued_area(bw, bq, bk, "bwd")
        # the issued area covers every visible pair
        assert schedule.issued_pairs(f, bq, bk) >= schedule.visible_pairs(cq, ck, causal)


def test_issued_pairs_tiny_batch_by_hand():
    # documents [17, 64, 128, 47], causal.  Forward tiles of 128 query rows x
    # 64 keys: one query tile per document; the 128-token document needs two
    # key tiles, the others one -> 5 tiles of 8192 cells.  dK/dV tiles of 32
    # query rows x 128 keys: one key tile per document with 1, 2, 4 and 2
    # query tiles -> 9 tiles of 4096 cells.
    cu = np.array([0, 17, 81, 209, 256], dtype=np.int32)
    f = schedule.fwd_items(cu, cu, True, 128, 64)
    bw = schedule.bwd_items(cu, cu, True, 32, 128)
    assert schedule.issued_pairs(f, 128, 64) == 5 * 128 * 64 == 40960
    assert schedule.issued_pairs(bw, 32, 128) == 9 * 32 * 128 == 36864
    assert round(schedule.visible_pairs(cu, cu, True) / 40960, 3) == 0.284


def test_visible_pairs_closed_form():
    lengths = [17, 64, 128, 47]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    assert schedule.visible_pairs(cu, cu, True) == sum(L * (L + 1) // 2 for L in lengths) == 11617
    assert schedule.visible_pairs(cu, cu, False) == sum(L * L for L in lengths)


def test_useful_flops_tiny():
    cu = np.array([0, 17, 81, 209, 256], dtype=np.int32)
    assert schedule.useful_flops(cu, cu, True, 4, 64, bwd=False) == 4 * 64 * 11617 * 4
    assert schedule.useful_flops(cu, cu, True, 4, 64) == 14 * 64 * 11617 * 4


@pytest.mark.parametrize("bad", [[1, 5], [0, 5, 3], [0, -1], [], [0, 2**31]])
def test_validate_cu_rejects(bad):
    with pytest.raises(ValueError):
        schedule.validate_cu(np.array(bad, dtype=np.int64))


def test_validate_cu_total():
    with pytest.raises(ValueError):
        schedule.validate_cu(np.array([0, 4, 9]), total=10)
    schedule.validate_cu(np.array([0, 4, 4, 10]), total=10)


def _read_golden(name):
    lines = [ln.strip() for ln in open(os.path.join(GOLDEN, name)) if ln.strip() and not ln.startswith("#")]
    cu = [int(x) for x in lines[0].split()[1:]]
    chunk = int(lines[1].split()[1])
    grid = [ln.split() for ln in lines[2:]]
    return cu, chunk, grid


def test_block_patterns_reproduce_hsap_fig3():
    cu, chunk, grid = _read_golden("hsap_fig3_step1.txt")
    assert schedule.block_patterns(np.array(cu), chunk) == grid


def test_block_patterns_single_document_is_lower_triangle():
    g = schedule.block_patterns(np.array([0, 32]), 8)
    for r in range(4):
        assert g[r] == ["A2"] * r + ["A1"] + ["N"] * (3 - r)
