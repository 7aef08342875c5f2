"""Combination of partial attention results computed over disjoint key chunks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Ring-style sequence parallelism keeps a rank's query block and lets key/value
blocks visit it one after another; the partial results are combined in the
online-softmax manner (HSAP page, Section 2.2.1, InterSP; BASP page,
Section VII, ring attention; the separate copy and rescale steps of the HSAP
page's Section 3.1, Table 1, and its Limitations paragraph).

The pages state no formula, so this is derived from the softmax definition:
a partial over key set C_k gives O_k = sum_{j in C_k} exp(S_j - LSE_k) V_j and
LSE_k = log sum_{j in C_k} exp(S_j).  Over the union of the disjoint sets,
LSE = log sum_k exp(LSE_k) and O = sum_k exp(LSE_k - LSE) O_k.  A partial whose
set holds no visible key has LSE_k = -inf and weight zero; if all are -inf the
result is O = 0, LSE = -inf.
"""
from __future__ import annotations

import numpy as np


def lse_merge(o_parts, lse_parts):
    """o_parts: list of [T,H,d]; lse_parts: list of [H,T].  Returns fp64 (O, LSE)."""
    if len(o_parts) == 0 or len(o_parts) != len(lse_parts):
        raise ValueError("need the same positive number of O and LSE partials")
    o = [np.asarray(x, dtype=np.float64) for x in o_parts]
    lse = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])  # [n,H,T]
    m = lse.max(axis=0)                                                    # [H,T]
    has = np.isfinite(m)
    m0 = np.where(has, m, 0.0)
    w = np.exp(lse - m0[None])                                             # [n,H,T]
    tot = w.sum(axis=0)
    out_lse = np.where(has, m0 + np.log(np.where(has, tot, 1.0)), -np.inf)
    wn = w / np.where(has, tot, 1.0)[None]
    out = np.zeros_like(o[0])
    for k in range(len(o)):
        out += wn[k].T[:, :, None] * o[k]
    return out, out_lse
