"""The Ulysses sequence<->head layout change of one GPU's shard.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Intra-group sequence parallelism holds a token shard with all heads,
[n, H, d], and an all-to-all moves the parallelism from tokens to heads, so
that afterwards each of the P ranks holds the full length for H/P heads
(HSAP page, Section 2.2.2; BASP page, Section II-C and Figure 2a; NSP page,
Section 2.1).  The local part of that step is the send-side pack: chunk p of
the output holds heads [p h, (p+1) h) of every token, h = H/P, laid out
[P, n, h, d] so each chunk is one contiguous message.  The inverse unpacks the
chunks received after attention back to [n, H, d].
"""
from __future__ import annotations

import numpy as np


def seq2head(x, sp_degree: int) -> np.ndarray:
    """[n, H, d] -> [P, n, H/P, d]; chunk p holds heads p*H/P .. (p+1)*H/P - 1."""
    x = np.asarray(x)
    n, H, d = x.shape
    if sp_degree <= 0 or H % sp_degree:
        raise ValueError("head count must be a multiple of the SP degree")
    h = H // sp_degree
    return np.ascontiguousarray(x.reshape(n, sp_degree, h, d).transpose(1, 0, 2, 3))


def head2seq(y) -> np.ndarray:
    """[P, n, h, d] -> [n, P*h, d], the inverse of seq2head."""
    y = np.asarray(y)
    P, n, h, d = y.shape
    return np.ascontiguousarray(y.transpose(1, 0, 2, 3).reshape(n, P * h, d))
