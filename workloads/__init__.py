"""Seeded synthetic workloads for packed variable-length attention.

This module only draws random numbers and arranges them into shapes.  It holds
none of the attention arithmetic, so both the fp64 oracle checks and the HIP
path can take their inputs from here without sharing any of the method.

Length mixes follow the long-tailed corpora the pages describe: most samples
are short and a few are very long (NSP page, Section 3.1 and Figure 2a: the
bulk of samples lie below 8K tokens and a tiny fraction exceeds 128K).  The
pages' own datasets are not available; these generators stand in for them.

Recipe (stated once, used everywhere):
  * lengths:  ``rng = numpy.random.default_rng(seed)``, one draw per document,
    rounded half-up to an integer, clipped to ``[lo, hi]``, drawn until the token
    budget is filled; the last document is truncated to the budget.
  * tensors:  ``torch.Generator().manual_seed(seed)`` on the CPU; fp32
    ``randn`` for Q, K, V, dO in that order; Q is multiplied by ``q_scale`` in
    fp32; everything is rounded to bf16 (round-to-nearest-even by torch).
  * realised length lists are frozen in ``workloads/lengths/*.json`` so that
    parity does not depend on the numpy generator version.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LENGTHS_DIR = os.path.join(_HERE, "lengths")


def lognormal_lengths(seed: int, total: int, median: float, sigma: float,
                      lo: int, hi: int) -> List[int]:
    """Document lengths drawn from a lognormal with the given median and sigma."""
    rng = np.random.default_rng(seed)
    out, filled = [], 0
    while filled < total:
        x = rng.lognormal(math.log(median), sigma)
        n = int(np.clip(np.floor(x + 0.5), lo, hi))
        n = min(n, total - filled)
        out.append(n)
        filled += n
    return out


def pareto_lengths(seed: int, total: int, alpha: float, lo: int, hi: int) -> List[int]:
    """Document lengths ``lo * (1 + Lomax(alpha))``: a Pareto tail starting at ``lo``."""
    rng = np.random.default_rng(seed)
    out, filled = [], 0
    while filled < total:
        x = lo * (1.0 + rng.pareto(alpha))
        n = int(np.clip(np.floor(x + 0.5), lo, hi))
        n = min(n, total - filled)
        out.append(n)
        filled += n
    return out


def pareto_seed_rule(total: int = 131072, alpha: float = 1.1, lo: int = 128,
                     hi: int = 65536, max_seed: int = 1000) -> int:
    """Smallest seed >= 0 whose Pareto draw has one or two documents above 32768."""
    for s in range(max_seed):
        L = pareto_lengths(s, total, alpha, lo, hi)
        if 1 <= sum(1 for x in L if x > 32768) <= 2:
            return s
    raise RuntimeError("no seed satisfies the rule")


def cu_seqlens(lengths) -> np.ndarray:
    """Exclusive prefix sum of the lengths, int32, with a leading 0."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu.astype(np.int32)


def _frozen(name: str) -> Optional[List[int]]:
    path = os.path.join(LENGTHS_DIR, name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return [int(x) for x in json.load(f)["lengths"]]


@dataclass
class Workload:
    """One packed batch: the document lengths and the attention shape."""
    name: str
    lengths: List[int]
    hq: int
    hkv: int
    d: int
    causal: bool = True
    seed: int = 0
    q_scale: float = 1.0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def total(self) -> int:
        return int(sum(self.lengths))

    @property
    def cu(self) -> np.ndarray:
        return cu_seqlens(self.lengths)


def tiny() -> Workload:
    """4 documents [17, 64, 128, 47] (256 tokens), 4/4 heads, head_dim 64."""
    return Workload("tiny_256", [17, 64, 128, 47], hq=4, hkv=4, d=64, seed=0,
                    note="cu_seqlens [0,17,81,209,256]")


def longtail_16k() -> Workload:
    """16384 tokens, lognormal(median 512, sigma 1.2) lengths in [64, 8192], GQA 32/4, d 128."""
    L = _frozen("longtail_16k_seed0") or lognormal_lengths(0, 16384, 512.0, 1.2, 64, 8192)
    return Workload("longtail_16k", L, hq=32, hkv=4, d=128, seed=0,
                    note="lognormal(ln 512, 1.2) clipped [64,8192], seed 0")


def ulysses_384k() -> Workload:
    """One GPU's Ulysses share of one 393216-token sequence at degree 8: 4 q heads, 1 kv head."""
    return Workload("ulysses_384k", [393216], hq=4, hkv=1, d=128, seed=0,
                    note="single document, 4/1 heads after seq->head",
                    extra={"permute_tokens": 49152, "permute_heads": 32, "sp_degree": 8})


def ring_256k() -> Workload:
    """Ring share: query chunk 7 of a 262144-token sequence cut in 8 chunks of 32768."""
    return Workload("ring_256k", [262144], hq=8, hkv=8, d=128, seed=0,
                    note="8 chunks of 32768; query chunk 7 against kv chunks 0..7",
                    extra={"n_chunks": 8, "chunk": 32768, "q_chunk": 7})


def mixed_128k() -> Workload:
    """131072 tokens, Pareto(1.1) lengths in [128, 65536], GQA 32/4, d 128, Q x 3.0."""
    L = _frozen("mixed_128k") or pareto_lengths(pareto_seed_rule(), 131072, 1.1, 128, 65536)
    return Workload("mixed_128k", L, hq=32, hkv=4, d=128, seed=0, q_scale=3.0,
                    note="128*(1+Lomax(1.1)) clipped [128,65536]; length seed by rule")


ALL = {w().name: w for w in (tiny, longtail_16k, ulysses_384k, ring_256k, mixed_128k)}


def length_buckets(lengths):
    """Split document indices into the buckets <2K, 2K-16K, >16K tokens."""
    b = {"lt2k": [], "2k_16k": [], "gt16k": []}
    for i, n in enumerate(lengths):
        if n < 2048:
            b["lt2k"].append(i)
        elif n <= 16384:
            b["2k_16k"].append(i)
        else:
            b["gt16k"].append(i)
    return b


def randn_bf16(shape, gen, scale: float = 1.0):
    """fp32 standard normals from ``gen`` times ``scale``, rounded to bf16."""
    import torch
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(torch.bfloat16)


def make_tensors(w: Workload, tq: Optional[int] = None, tk: Optional[int] = None,
                 with_do: bool = True):
    """Q [Tq,Hq,d], K [Tk,Hkv,d], V [Tk,Hkv,d], dO [Tq,Hq,d] as bf16 CPU tensors."""
    import torch
    tq = w.total if tq is None else tq
    tk = w.total if tk is None else tk
    g = torch.Generator().manual_seed(w.seed)
    q = randn_bf16((tq, w.hq, w.d), g, w.q_scale)
    k = randn_bf16((tk, w.hkv, w.d), g)
    v = randn_bf16((tk, w.hkv, w.d), g)
    do = randn_bf16((tq, w.hq, w.d), g) if with_do else None
    return q, k, v, do


def sample_rows(n_rows: int, n_sample: int, seed: int = 1) -> np.ndarray:
    """``n_sample`` distinct row indices out of ``n_rows`` (sorted), seeded."""
    rng = np.random.default_rng(seed)
    n_sample = min(n_sample, n_rows)
    return np.sort(rng.choice(n_rows, size=n_sample, replace=False))


def random_lengths(rng: np.random.Generator, n_docs: int, lo: int, hi: int) -> List[int]:
    """Uniform integer lengths in [lo, hi] for small randomised tests."""
    return [int(x) for x in rng.integers(lo, hi + 1, size=n_docs)]
