"""Per-document softmax attention in fp64, forward and analytic backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What is computed (the plain definition, no tiling, no online softmax):

  * Scaled dot-product attention per head, softmax(Q K^T / sqrt(d)) V
    (BASP page, Section II-A, scaled dot-product and multi-head attention;
    HSAP page, Section 2.2.1, the attention formula with Q, K, V of shape
    N x H x d).
  * Packed documents do not see each other: attention is computed only inside
    each segment delimited by the cumulative lengths (HSAP page, Section 2.1 and
    Figure 1, cu_len; NSP page, Section 2.2, segmented mask of packing).
  * Causal: a query sees the keys at or before its own position in its
    document (HSAP page, Section 1 and the "Causal Attn" legend of Figure 3).

Readings where the pages are silent:
  * scale defaults to 1/sqrt(d);
  * LSE is the natural-log log-sum-exp of the scaled scores, stored [Hq, Tq];
  * grouped-query attention maps q head h to kv head floor(h / (Hq / Hkv));
  * with Lq != Lk the causal diagonal is bottom-right aligned:
    key j is visible from query i iff j <= i + (Lk - Lq);
  * a query with no visible key has O = 0, LSE = -inf and zero gradient;
  * the backward is the exact gradient of the forward for an upstream dO.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .schedule import doc_table

_MAX_BLOCK_ELEMS = 1 << 23  # scores held at once per block: 64 MiB of fp64


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale)


def _rows_per_block(lk: int, row_block: int) -> int:
    return max(1, min(row_block, _MAX_BLOCK_ELEMS // max(lk, 1)))


def visible(rows: np.ndarray, lq: int, lk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), lk]: key j visible from doc-relative query row i."""
    cols = np.arange(lk)
    if not causal:
        return np.ones((len(rows), lk), dtype=bool)
    return cols[None, :] <= (rows[:, None] + (lk - lq))


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Row softmax of s restricted to vis; returns (P, LSE) with P=0, LSE=-inf on empty rows."""
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    has = np.isfinite(m)
    m0 = np.where(has, m, 0.0)
    e = np.exp(s - m0[:, None])
    tot = e.sum(axis=1)
    lse = np.where(has, m0 + np.log(np.where(has, tot, 1.0)), -np.inf)
    p = e / np.where(has, tot, 1.0)[:, None]
    return p, lse


def attn_fwd(q, k, v, cu_q, cu_k, causal: bool = True, scale: Optional[float] = None,
             row_block: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """O [Tq,Hq,d] and LSE [Hq,Tq] for packed documents; fp64 throughout."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    grp = hq // hkv
    sc = _scale(d, scale)
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    for qs, lq, ks, lk in doc_table(cu_q, cu_k, tq, tk):
        if lq == 0 or lk == 0:
            continue
        rb = _rows_per_block(lk, row_block)
        for h in range(hq):
            kb = k[ks:ks + lk, h // grp, :]
            vb = v[ks:ks + lk, h // grp, :]
            for r0 in range(0, lq, rb):
                r1 = min(lq, r0 + rb)
                s = sc * (q[qs + r0:qs + r1, h, :] @ kb.T)
                p, l = _softmax_rows(s, visible(np.arange(r0, r1), lq, lk, causal))
                o[qs + r0:qs + r1, h, :] = p @ vb
                lse[h, qs + r0:qs + r1] = l
    return o, lse


def attn_bwd(q, k, v, do, cu_q, cu_k, causal: bool = True, scale: Optional[float] = None,
             row_block: int = 512, return_fwd: bool = False):
    """dQ, dK, dV (fp64) of sum(O * dO) for the forward above.

    For each visible pair, with P the softmax probabilities, D_i = dO_i . O_i:
      dV_j += P_ij dO_i,   dP_ij = dO_i . V_j,   dS_ij = P_ij (dP_ij - D_i),
      dQ_i += scale dS_ij K_j,   dK_j += scale dS_ij Q_i,
    summed over the q heads that share a kv head.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = hq // hkv
    sc = _scale(d, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.full((hq, tq), -np.inf)
    for qs, lq, ks, lk in doc_table(cu_q, cu_k, tq, tk):
        if lq == 0 or lk == 0:
            continue
        rb = _rows_per_block(lk, row_block)
        for h in range(hq):
            g = h // grp
            kb = k[ks:ks + lk, g, :]
            vb = v[ks:ks + lk, g, :]
            for r0 in range(0, lq, rb):
                r1 = min(lq, r0 + rb)
                qb = q[qs + r0:qs + r1, h, :]
                dob = do[qs + r0:qs + r1, h, :]
                p, l = _softmax_rows(sc * (qb @ kb.T), visible(np.arange(r0, r1), lq, lk, causal))
                ob = p @ vb
                dd = np.sum(dob * ob, axis=1)
                ds = p * (dob @ vb.T - dd[:, None])
                dq[qs + r0:qs + r1, h, :] = sc * (ds @ kb)
                dk[ks:ks + lk, g, :] += sc * (ds.T @ qb)
                dv[ks:ks + lk, g, :] += p.T @ dob
                o[qs + r0:qs + r1, h, :] = ob
                lse[h, qs + r0:qs + r1] = l
    if return_fwd:
        return dq, dk, dv, o, lse
    return dq, dk, dv


def _locate(cu: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Document index of each packed row (documents of zero length are skipped)."""
    return np.searchsorted(cu, rows, side="right") - 1


def attn_fwd_rows(q, k, v, cu_q, cu_k, rows, heads, causal: bool = True,
                  scale: Optional[float] = None):
    """O [n,d] and LSE [n] of the given (packed row, q head) pairs only; O(Lk d) per pair."""
    o, lse, _ = _rows_common(q, k, v, None, cu_q, cu_k, rows, heads, causal, scale)
    return o, lse


def attn_bwd_dq_rows(q, k, v, do, cu_q, cu_k, rows, heads, causal: bool = True,
                     scale: Optional[float] = None):
    """dQ [n,d] of the given (packed row, q head) pairs; also returns their O and LSE."""
    o, lse, dq = _rows_common(q, k, v, do, cu_q, cu_k, rows, heads, causal, scale)
    return dq, o, lse


def _rows_common(q, k, v, do, cu_q, cu_k, rows, heads, causal, scale):
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = hq // hkv
    sc = _scale(d, scale)
    docs = doc_table(cu_q, cu_k, tq, tk)
    cuq = np.asarray(cu_q, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    n = len(rows)
    o = np.zeros((n, d))
    lse = np.full(n, -np.inf)
    dq = np.zeros((n, d)) if do is not None else None
    doc_of = _locate(cuq, rows)
    for key in sorted(set(zip(doc_of.tolist(), heads.tolist()))):
        b, h = key
        sel = np.nonzero((doc_of == b) & (heads == h))[0]
        qs, lq, ks, lk = docs[b]
        if lk == 0:
            continue
        g = h // grp
        kb = _f64(k[ks:ks + lk, g, :])
        vb = _f64(v[ks:ks + lk, g, :])
        rb = _rows_per_block(lk, 512)
        for c0 in range(0, len(sel), rb):
            idx = sel[c0:c0 + rb]
            r = rows[idx] - qs
            qb = _f64(q[rows[idx], h, :])
            p, l = _softmax_rows(sc * (qb @ kb.T), visible(r, lq, lk, causal))
            ob = p @ vb
            o[idx] = ob
            lse[idx] = l
            if do is not None:
                dob = _f64(np.asarray(do)[rows[idx], h, :])
                dd = np.sum(dob * ob, axis=1)
                ds = p * (dob @ vb.T - dd[:, None])
                dq[idx] = sc * (ds @ kb)
    return o, lse, dq


def attn_bwd_dkv_rows(q, k, v, do, cu_q, cu_k, krows, kheads, causal: bool = True,
                      scale: Optional[float] = None, row_block: int = 512):
    """dK [n,d] and dV [n,d] of the given (packed key row, kv head) pairs.

    Exact: for each sampled key the forward is recomputed for every query that
    can see it (LSE_i and D_i need the whole query row), so the cost is the
    number of such queries times Lk times d.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = hq // hkv
    sc = _scale(d, scale)
    docs = doc_table(cu_q, cu_k, tq, tk)
    cuk = np.asarray(cu_k, dtype=np.int64)
    krows = np.asarray(krows, dtype=np.int64)
    kheads = np.asarray(kheads, dtype=np.int64)
    n = len(krows)
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    doc_of = _locate(cuk, krows)
    for key in sorted(set(zip(doc_of.tolist(), kheads.tolist()))):
        b, g = key
        sel = np.nonzero((doc_of == b) & (kheads == g))[0]
        qs, lq, ks, lk = docs[b]
        if lq == 0:
            continue
        jj = krows[sel] - ks
        i_lo = max(0, int(jj.min()) - (lk - lq)) if causal else 0
        if i_lo >= lq:
            continue
        kb = _f64(k[ks:ks + lk, g, :])
        vb = _f64(v[ks:ks + lk, g, :])
        vj = vb[jj]
        rb = _rows_per_block(lk, row_block)
        acc_k = np.zeros((len(sel), d))
        acc_v = np.zeros((len(sel), d))
        for h in range(g * grp, (g + 1) * grp):
            for r0 in range(i_lo, lq, rb):
                r1 = min(lq, r0 + rb)
                qb = _f64(q[qs + r0:qs + r1, h, :])
                dob = _f64(do[qs + r0:qs + r1, h, :])
                vis = visible(np.arange(r0, r1), lq, lk, causal)
                p, _ = _softmax_rows(sc * (qb @ kb.T), vis)
                ob = p @ vb
                dd = np.sum(dob * ob, axis=1)
                pj = p[:, jj]
                dsj = pj * (dob @ vj.T - dd[:, None])
                acc_k += sc * (dsj.T @ qb)
                acc_v += pj.T @ dob
        dk[sel] = acc_k
        dv[sel] = acc_v
    return dk, dv
