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


# ---------------------------------------------------------------------------
# Grouped-query attention under the Ulysses layout change.
#
# With GQA, query head h reads kv head floor(h * Hkv / Hq) (contiguous groups;
# the pages never mention GQA, this is the plain reading).  After the
# all-to-all, rank p holds query heads [p*Hq/P, (p+1)*Hq/P) for the whole
# sequence, so it needs exactly the kv heads those query heads read.  When
# Hkv >= P these are Hkv/P heads of their own; when Hkv < P several ranks need
# the same kv head, which is sent to each of them (replicated), and on the way
# back the gradients those ranks computed for it are summed.  (NSP page,
# Section 2.1, and BASP page, Section II-C: Q, K and V are all redistributed by
# the all-to-all; HSAP page, Section 2.2.2: heads are split over the ranks.)
# ---------------------------------------------------------------------------

def _check_gqa_split(sp_degree: int, n_heads_q: int, n_heads_kv: int):
    if sp_degree <= 0 or n_heads_q <= 0 or n_heads_kv <= 0:
        raise ValueError("degrees and head counts must be positive")
    if n_heads_q % sp_degree or n_heads_q % n_heads_kv:
        raise ValueError("sp_degree and n_heads_kv must divide n_heads_q")
    if n_heads_kv % sp_degree and sp_degree % n_heads_kv:
        raise ValueError("one of sp_degree, n_heads_kv must divide the other")


def rank_kv_heads(p: int, sp_degree: int, n_heads_q: int, n_heads_kv: int) -> list:
    """The kv heads read by rank p's query heads, in increasing order."""
    _check_gqa_split(sp_degree, n_heads_q, n_heads_kv)
    hq = n_heads_q // sp_degree
    return sorted({h * n_heads_kv // n_heads_q for h in range(p * hq, (p + 1) * hq)})


def kv_seq2head(x, sp_degree: int, n_heads_q: int) -> np.ndarray:
    """[n, Hkv, d] -> [P, n, hk, d]: chunk p holds the kv heads rank p needs.

    hk = Hkv/P when Hkv >= P, else 1 (each kv head then goes to P/Hkv ranks).
    """
    x = np.asarray(x)
    n, Hkv, d = x.shape
    heads = [rank_kv_heads(p, sp_degree, n_heads_q, Hkv) for p in range(sp_degree)]
    if len({len(hs) for hs in heads}) != 1:
        raise ValueError("ranks would hold different kv head counts")
    return np.ascontiguousarray(np.stack([x[:, hs, :] for hs in heads]))


def kv_head2seq_sum(y, n_heads_q: int, n_heads_kv: int, round_bf16: bool = False) -> np.ndarray:
    """[P, n, hk, d] -> [n, Hkv, d], the adjoint of kv_seq2head.

    Each kv head gets the sum of the chunks of every rank that held it, added
    in increasing rank order in y's dtype (float32 for bf16 data); with
    round_bf16 the sum is then rounded to bfloat16 (nearest, ties to even).
    """
    y = np.asarray(y)
    P, n, hk, d = y.shape
    out = np.zeros((n, n_heads_kv, d), dtype=y.dtype)
    seen = np.zeros(n_heads_kv, dtype=bool)
    for p in range(P):
        hs = rank_kv_heads(p, P, n_heads_q, n_heads_kv)
        if len(hs) != hk:
            raise ValueError("chunk head count does not match the head split")
        for j, g in enumerate(hs):
            if seen[g]:
                out[:, g, :] = out[:, g, :] + y[p, :, j, :]
            else:
                out[:, g, :] = y[p, :, j, :]
                seen[g] = True
    if round_bf16:
        out = round_to_bf16(out)
    return out


def round_to_bf16(a) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    r = ((bits + 0x7FFF + lsb) >> 16) << 16
    return (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def qkv_seq2head(q, k, v, sp_degree: int):
    """The three send-side packs of one Ulysses attention input: Q as
    seq2head, K and V as kv_seq2head for Q's head count."""
    hq = np.asarray(q).shape[1]
    return seq2head(q, sp_degree), kv_seq2head(k, sp_degree, hq), kv_seq2head(v, sp_degree, hq)


def qkv_head2seq(dq_y, dk_y, dv_y, n_heads_kv: int, round_bf16: bool = False):
    """The three receive-side unpacks of the attention input gradients:
    dQ as head2seq, dK and dV as kv_head2seq_sum."""
    P, n, hq, d = np.asarray(dq_y).shape
    Hq = P * hq
    return (head2seq(dq_y), kv_head2seq_sum(dk_y, Hq, n_heads_kv, round_bf16),
            kv_head2seq_sum(dv_y, Hq, n_heads_kv, round_bf16))
