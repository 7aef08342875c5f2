"""cu_seqlens validation, tile work lists, pair counts and the chunk pattern map.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Packing puts documents back to back with no padding, and the cumulative
lengths mark where each one starts (NSP page, Section 2.2; HSAP page,
Section 2.1, cu_len).  Each document is cut into query tiles of ``bq`` rows and
key tiles of ``bk`` rows; tiles never straddle two documents.  A tile pair
whose keys are all after the causal diagonal of all its queries carries no
visible pair: it is the "N" block of the HSAP page's Figure 3 and is never
issued.  The tile that meets the diagonal is the "A1" causal block.

Readings where the pages are silent:
  * cu arrays are int32, start at 0, never decrease and end at the total token
    count (packing has no padding);
  * the causal diagonal is bottom-right aligned when Lq != Lk;
  * work items are ordered longest first, ties by (document, tile), the same
    longest-first rule the NSP planner uses when it sorts samples by
    non-increasing length (NSP page, Section 4.1.3, Algorithm 1);
  * a forward item with no visible key tile is kept (its rows get O=0,
    LSE=-inf) and so is a backward item with no visible query tile (its key
    rows get dK=dV=0).
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

INT32_MAX = 2**31 - 1


def validate_cu(cu, total=None) -> np.ndarray:
    """Return cu as int64 after checking it is a valid int32 cumulative-length array."""
    a = np.asarray(cu)
    if a.ndim != 1 or a.size < 1:
        raise ValueError("cu_seqlens must be a 1-D array with at least one entry")
    if not np.issubdtype(a.dtype, np.integer):
        raise ValueError("cu_seqlens must be integers")
    a = a.astype(np.int64)
    if a[0] != 0:
        raise ValueError("cu_seqlens[0] must be 0")
    if np.any(np.diff(a) < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    if a[-1] > INT32_MAX or a.min() < 0:
        raise ValueError("cu_seqlens must fit int32")
    if total is not None and a[-1] != total:
        raise ValueError("cu_seqlens[-1] must equal the total token count")
    return a


def doc_table(cu_q, cu_k, total_q=None, total_k=None) -> List[Tuple[int, int, int, int]]:
    """Per document (q_start, Lq, k_start, Lk)."""
    a = validate_cu(cu_q, total_q)
    b = validate_cu(cu_k, total_k)
    if a.size != b.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    return [(int(a[i]), int(a[i + 1] - a[i]), int(b[i]), int(b[i + 1] - b[i]))
            for i in range(a.size - 1)]


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def fwd_items(cu_q, cu_k, causal: bool, bq: int, bk: int) -> np.ndarray:
    """Forward work list: int32 rows (doc, q_tile, first kv tile, kv tile count).

    A query tile's last row r sees keys up to r + (Lk - Lq); key tiles past the
    one holding that key are skipped.
    """
    items = []
    for b, (_, lq, _, lk) in enumerate(doc_table(cu_q, cu_k)):
        n_k = _ceil_div(lk, bk)
        for t in range(_ceil_div(lq, bq)):
            if causal:
                last_row = min(lq, (t + 1) * bq) - 1
                last_key = last_row + (lk - lq)
                n_kv = min(max(last_key // bk + 1, 0), n_k)
            else:
                n_kv = n_k
            items.append((b, t, 0, n_kv))
    items.sort(key=lambda it: (-it[3], it[0], it[1]))
    return np.asarray(items, dtype=np.int32).reshape(-1, 4)


def bwd_items(cu_q, cu_k, causal: bool, bq: int, bk: int) -> np.ndarray:
    """Backward work list: int32 rows (doc, kv_tile, first q tile, q tile count).

    Key j is first seen by query row j - (Lk - Lq); query tiles before the one
    holding that row are skipped.
    """
    items = []
    for b, (_, lq, _, lk) in enumerate(doc_table(cu_q, cu_k)):
        n_q = _ceil_div(lq, bq)
        for j in range(_ceil_div(lk, bk)):
            if causal:
                first_row = max(0, j * bk - (lk - lq))
                t0 = min(first_row // bq, n_q)
            else:
                t0 = 0
            items.append((b, j, t0, n_q - t0))
    items.sort(key=lambda it: (-it[3], it[0], it[1]))
    return np.asarray(items, dtype=np.int32).reshape(-1, 4)


def visible_pairs(cu_q, cu_k, causal: bool) -> int:
    """Number of (query, key) pairs that attention actually uses, per head."""
    tot = 0
    for _, lq, _, lk in doc_table(cu_q, cu_k):
        if not causal:
            tot += lq * lk
            continue
        off = lk - lq
        for i in range(lq):
            tot += min(max(i + off + 1, 0), lk)
    return tot


def issued_pairs(items: np.ndarray, bq: int, bk: int) -> int:
    """Pairs covered by the issued tiles (full tile area), per head."""
    return int(np.sum(np.asarray(items, dtype=np.int64)[:, 3])) * bq * bk if len(items) else 0


def useful_flops(cu_q, cu_k, causal: bool, hq: int, d: int, fwd: bool = True,
                 bwd: bool = True) -> int:
    """Useful FLOPs: 4 d per visible pair forward (QK^T and PV), 10 d backward
    (five contractions counting the score recompute), times the q heads."""
    vis = visible_pairs(cu_q, cu_k, causal)
    per = (4 if fwd else 0) + (10 if bwd else 0)
    return per * d * vis * hq


def block_patterns(cu, chunk: int) -> List[List[str]]:
    """Attention pattern of every (query chunk, key chunk) block of one packed sequence.

    The packed causal sequence with document mask is cut into equal chunks, one
    per ring rank, and each block is classified the way the HSAP page's
    Figure 3 (step 1) labels it: A1 diagonal causal block, A2 every pair
    visible, A3 only the top rows see keys (all key columns), A4 every row sees
    only the right-hand key columns, A5 only a top-right corner is visible,
    N nothing visible.
    """
    a = validate_cu(cu)
    total = int(a[-1])
    if total % chunk:
        raise ValueError("total length must be a multiple of the chunk")
    doc = np.searchsorted(a, np.arange(total), side="right") - 1
    n = total // chunk
    out = []
    for r in range(n):
        row = []
        x = np.arange(r * chunk, (r + 1) * chunk)
        for s in range(n):
            y = np.arange(s * chunk, (s + 1) * chunk)
            vis = (doc[x][:, None] == doc[y][None, :]) & (y[None, :] <= x[:, None])
            if r == s:
                row.append("A1")
                continue
            if not vis.any():
                row.append("N")
                continue
            rows_any = vis.any(axis=1)
            cols_any = vis.any(axis=0)
            if vis.all():
                row.append("A2")
            elif cols_any.all() and rows_any[0] and not rows_any.all():
                row.append("A3")
            elif rows_any.all() and cols_any[-1] and not cols_any.all():
                row.append("A4")
            elif rows_any[0] and cols_any[-1]:
                row.append("A5")
            else:
                row.append("?")
        out.append(row)
    return out
