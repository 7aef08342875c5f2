"""Pins of the fp64 attention oracle against things other than itself.

Brute-force loops, torch's fp64 scaled_dot_product_attention and autograd with
an explicit document mask, finite differences, closed-form special cases and
invariants.  All CPU, all small.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attn_fwd, attn_bwd, attn_fwd_rows, attn_bwd_dq_rows, attn_bwd_dkv_rows
from oracle.merge import lse_merge


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _rand(rng, lengths_q, lengths_k, hq, hkv, d, scale=1.0):
    tq, tk = int(sum(lengths_q)), int(sum(lengths_k))
    q = rng.standard_normal((tq, hq, d)) * scale
    k = rng.standard_normal((tk, hkv, d))
    v = rng.standard_normal((tk, hkv, d))
    do = rng.standard_normal((tq, hq, d))
    return q, k, v, do


def brute_fwd(q, k, v, cu_q, cu_k, causal, scale):
    """Pure-Python loops over every (doc, head, query, key)."""
    tq, hq, d = len(q), len(q[0]), len(q[0][0])
    hkv = len(k[0])
    o = [[[0.0] * d for _ in range(hq)] for _ in range(tq)]
    lse = [[-math.inf] * tq for _ in range(hq)]
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        lq, lk = qe - qs, ke - ks
        for h in range(hq):
            g = h * hkv // hq
            for i in range(lq):
                scores = []
                for j in range(lk):
                    if causal and j > i + lk - lq:
                        continue
                    s = 0.0
                    for c in range(d):
                        s += q[qs + i][h][c] * k[ks + j][g][c]
                    scores.append((j, s * scale))
                if not scores:
                    continue
                m = max(s for _, s in scores)
                z = sum(math.exp(s - m) for _, s in scores)
                lse[h][qs + i] = m + math.log(z)
                for j, s in scores:
                    p = math.exp(s - m) / z
                    for c in range(d):
                        o[qs + i][h][c] += p * v[ks + j][g][c]
    return np.array(o), np.array(lse)


def _doc_mask(lengths, causal):
    """Block-diagonal (optionally causal) boolean mask [T, T] for Lq == Lk."""
    t = int(sum(lengths))
    m = torch.zeros(t, t, dtype=torch.bool)
    s = 0
    for L in lengths:
        blk = torch.ones(L, L, dtype=torch.bool)
        if causal:
            blk = torch.tril(blk)
        m[s:s + L, s:s + L] = blk
        s += L
    return m


def _torch_sdpa(q, k, v, lengths, causal, scale):
    """torch fp64 SDPA over the packed batch as one sequence with the document mask."""
    hq, hkv = q.shape[1], k.shape[1]
    tq = torch.tensor(q).permute(1, 0, 2).unsqueeze(0)
    tk = torch.tensor(k).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2).unsqueeze(0)
    tv = torch.tensor(v).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2).unsqueeze(0)
    return tq, tk, tv, _doc_mask(lengths, causal)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_fwd_brute_force(rng, causal, hq, hkv):
    lq = [5, 1, 13, 0, 9]
    lk = [7, 1, 13, 4, 6] if not causal else [5, 3, 13, 0, 12]
    q, k, v, _ = _rand(rng, lq, lk, hq, hkv, 8)
    scale = 1 / math.sqrt(8)
    o, lse = attn_fwd(q, k, v, _cu(lq), _cu(lk), causal=causal)
    bo, blse = brute_fwd(q.tolist(), k.tolist(), v.tolist(), _cu(lq), _cu(lk), causal, scale)
    assert np.allclose(o, bo, atol=1e-12, rtol=0)
    fin = np.isfinite(blse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], blse[fin], atol=1e-12, rtol=0)


def test_fwd_causal_lk_shorter_than_lq_has_empty_rows(rng):
    # bottom-right alignment: with Lk < Lq the first Lq - Lk rows see nothing
    lq, lk = [6], [2]
    q, k, v, _ = _rand(rng, lq, lk, 1, 1, 4)
    o, lse = attn_fwd(q, k, v, _cu(lq), _cu(lk), causal=True)
    assert np.all(o[:4] == 0) and np.all(np.isneginf(lse[0, :4]))
    assert np.all(np.isfinite(lse[0, 4:]))
    bo, blse = brute_fwd(q.tolist(), k.tolist(), v.tolist(), _cu(lq), _cu(lk), True, 0.5)
    assert np.allclose(o, bo, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_fwd_matches_torch_sdpa_with_document_mask(rng, causal):
    lengths = [17, 64, 3, 47, 1]
    q, k, v, _ = _rand(rng, lengths, lengths, 4, 2, 16)
    o, lse = attn_fwd(q, k, v, _cu(lengths), _cu(lengths), causal=causal)
    tq, tk, tv, mask = _torch_sdpa(q, k, v, lengths, causal, None)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    ref = ref.squeeze(0).permute(1, 0, 2).numpy()
    assert np.allclose(o, ref, atol=1e-10, rtol=0)


def test_single_token_document(rng):
    lengths = [1, 5, 1]
    q, k, v, _ = _rand(rng, lengths, lengths, 2, 1, 8)
    o, lse = attn_fwd(q, k, v, _cu(lengths), _cu(lengths))
    sc = 1 / math.sqrt(8)
    for t in (0, 6):
        for h in range(2):
            assert np.array_equal(o[t, h], v[t, 0])
            assert abs(lse[h, t] - sc * float(q[t, h] @ k[t, 0])) < 1e-13


def test_rows_of_p_sum_to_one(rng):
    # with V identically 1 every output is sum_j P_ij = 1
    lengths = [33, 7, 100]
    q, k, _, _ = _rand(rng, lengths, lengths, 2, 2, 8, scale=3.0)
    v = np.ones_like(k)
    o, _ = attn_fwd(q, k, v, _cu(lengths), _cu(lengths))
    assert np.max(np.abs(o - 1.0)) < 1e-13


def test_packing_invariance(rng):
    lengths = [40, 3, 77, 20]
    q, k, v, do = _rand(rng, lengths, lengths, 4, 2, 8)
    cu = _cu(lengths)
    o, lse = attn_fwd(q, k, v, cu, cu)
    dq, dk, dv = attn_bwd(q, k, v, do, cu, cu)
    for b, L in enumerate(lengths):
        s, e = cu[b], cu[b + 1]
        one = np.array([0, L], dtype=np.int32)
        o1, l1 = attn_fwd(q[s:e], k[s:e], v[s:e], one, one)
        g = attn_bwd(q[s:e], k[s:e], v[s:e], do[s:e], one, one)
        assert np.array_equal(o1, o[s:e]) and np.array_equal(l1, lse[:, s:e])
        for a, ref in zip(g, (dq, dk, dv)):
            assert np.allclose(a, ref[s:e], atol=1e-13, rtol=0)


def test_chunked_kv_merge_equals_full_attention(rng):
    # one document; queries = last chunk; keys cut into random chunks
    L, d = 96, 8
    q, k, v, _ = _rand(rng, [L], [L], 2, 2, d)
    o_full, lse_full = attn_fwd(q, k, v, _cu([L]), _cu([L]))
    q0 = 64
    for _ in range(3):
        cuts = np.sort(rng.choice(np.arange(1, q0), size=3, replace=False))
        bounds = [0, *cuts.tolist(), q0, L]
        os_, ls_ = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            nq = L - q0
            if b <= q0:  # key chunk fully before the query chunk: no mask
                o_p, l_p = attn_fwd(q[q0:], k[a:b], v[a:b], [0, nq], [0, b - a], causal=False)
            else:       # the query chunk itself: causal
                o_p, l_p = attn_fwd(q[q0:], k[a:b], v[a:b], [0, nq], [0, b - a], causal=True)
            os_.append(o_p)
            ls_.append(l_p)
        o_m, l_m = lse_merge(os_, ls_)
        assert np.allclose(o_m, o_full[q0:], atol=1e-12, rtol=0)
        assert np.allclose(l_m, lse_full[:, q0:], atol=1e-12, rtol=0)


def test_gqa_equals_mha_with_repeated_kv(rng):
    lengths = [9, 30]
    q, k, v, do = _rand(rng, lengths, lengths, 6, 2, 8)
    cu = _cu(lengths)
    o, lse = attn_fwd(q, k, v, cu, cu)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o2, lse2 = attn_fwd(q, kr, vr, cu, cu)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    dq, dk, dv = attn_bwd(q, k, v, do, cu, cu)
    dq2, dk2, dv2 = attn_bwd(q, kr, vr, do, cu, cu)
    assert np.allclose(dq, dq2, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(dk2.shape[0], 2, 3, -1).sum(2), atol=1e-12)
    assert np.allclose(dv, dv2.reshape(dv2.shape[0], 2, 3, -1).sum(2), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_central_finite_differences(rng, causal):
    lq = [4, 1, 6]
    lk = [4, 1, 6] if causal else [3, 2, 5]
    q, k, v, do = _rand(rng, lq, lk, 2, 1, 4)
    cq, ck = _cu(lq), _cu(lk)
    dq, dk, dv = attn_bwd(q, k, v, do, cq, ck, causal=causal)

    def loss(q_, k_, v_):
        return float(np.sum(attn_fwd(q_, k_, v_, cq, ck, causal=causal)[0] * do))

    eps = 1e-5
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        rel = np.linalg.norm(num - g) / max(np.linalg.norm(g), 1e-30)
        assert rel < 1e-6, rel


def test_bwd_matches_torch_autograd(rng):
    lengths = [17, 2, 40, 5]
    q, k, v, do = _rand(rng, lengths, lengths, 4, 2, 8)
    cu = _cu(lengths)
    dq, dk, dv = attn_bwd(q, k, v, do, cu, cu)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    mask = _doc_mask(lengths, True)
    kk = tk.repeat_interleave(2, dim=1).permute(1, 0, 2).unsqueeze(0)
    vv = tv.repeat_interleave(2, dim=1).permute(1, 0, 2).unsqueeze(0)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2).unsqueeze(0), kk, vv, attn_mask=mask)
    out.squeeze(0).permute(1, 0, 2).backward(torch.tensor(do))
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-10)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-10)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-10)


def test_bwd_closed_form_sums(rng):
    # sum_j dS_ij = 0 gives sum_j dK_j = 0; sum_j P_ij = 1 gives sum_j dV_j = sum_i dO_i
    lengths = [50, 13, 1, 70]
    q, k, v, do = _rand(rng, lengths, lengths, 4, 2, 8, scale=2.0)
    cu = _cu(lengths)
    dq, dk, dv = attn_bwd(q, k, v, do, cu, cu)
    for b in range(len(lengths)):
        s, e = cu[b], cu[b + 1]
        for g in range(2):
            assert np.max(np.abs(dk[s:e, g].sum(0))) < 1e-12
            ref = do[s:e, 2 * g:2 * g + 2].sum(axis=(0, 1))
            assert np.allclose(dv[s:e, g].sum(0), ref, atol=1e-12)


def test_row_sampled_versions_match_full(rng):
    lq = [30, 1, 64, 0, 20]
    lk = [30, 1, 64, 3, 20]
    q, k, v, do = _rand(rng, lq, lk, 4, 2, 8)
    cq, ck = _cu(lq), _cu(lk)
    dq, dk, dv, o, lse = attn_bwd(q, k, v, do, cq, ck, return_fwd=True)
    rows = np.array([0, 29, 30, 31, 50, 94, 114])
    heads = np.array([0, 3, 1, 2, 0, 3, 1])
    o_r, lse_r = attn_fwd_rows(q, k, v, cq, ck, rows, heads)
    assert np.allclose(o_r, o[rows, heads], atol=1e-13)
    assert np.allclose(lse_r, lse[heads, rows], atol=1e-13)
    dq_r, _, _ = attn_bwd_dq_rows(q, k, v, do, cq, ck, rows, heads)
    assert np.allclose(dq_r, dq[rows, heads], atol=1e-13)
    krows = np.array([0, 29, 30, 60, 93, 95, 97, 100, 117])
    kh = np.array([0, 1, 1, 0, 1, 0, 1, 0, 1])
    dk_r, dv_r = attn_bwd_dkv_rows(q, k, v, do, cq, ck, krows, kh)
    assert np.allclose(dk_r, dk[krows, kh], atol=1e-12)
    assert np.allclose(dv_r, dv[krows, kh], atol=1e-12)


def test_rows_versions_non_causal(rng):
    lq, lk = [12, 7], [5, 9]
    q, k, v, do = _rand(rng, lq, lk, 2, 1, 4)
    cq, ck = _cu(lq), _cu(lk)
    dq, dk, dv, o, lse = attn_bwd(q, k, v, do, cq, ck, causal=False, return_fwd=True)
    rows, heads = np.arange(19), np.arange(19) % 2
    o_r, _ = attn_fwd_rows(q, k, v, cq, ck, rows, heads, causal=False)
    assert np.allclose(o_r, o[rows, heads], atol=1e-13)
    kr = np.arange(14)
    dk_r, dv_r = attn_bwd_dkv_rows(q, k, v, do, cq, ck, kr, np.zeros(14, int), causal=False)
    assert np.allclose(dk_r, dk[kr, 0], atol=1e-12) and np.allclose(dv_r, dv[kr, 0], atol=1e-12)


def test_planted_mistake_is_caught(rng, monkeypatch):
    # a dropped max-subtraction sign or a wrong head mapping must break a pin
    lengths = [9, 4]
    q, k, v, _ = _rand(rng, lengths, lengths, 4, 2, 4)
    cu = _cu(lengths)
    good, _ = attn_fwd(q, k, v, cu, cu)
    orig = oracle.attention.visible
    monkeypatch.setattr(oracle.attention, "visible",
                        lambda r, lq, lk, c: orig(r + 1, lq, lk, c))  # off-by-one diagonal
    bad, _ = attn_fwd(q, k, v, cu, cu)
    bo, _ = brute_fwd(q.tolist(), k.tolist(), v.tolist(), cu, cu, True, 0.5)
    assert np.allclose(good, bo, atol=1e-12)
    assert not np.allclose(bad, bo, atol=1e-6)
