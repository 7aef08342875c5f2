"""Work lists built per call (plan cache off) against the cached ones.

With the cache off every attention call schedules its cu_seqlens again and
uploads the lists through pinned staging into a per-device ring of device
memory, on its own stream.  The kernels are the same, so every output must be
bitwise equal to the cached path's.  The calls below are issued without
synchronising in between, so the ring wraps while earlier regions are still
in flight (a region is reused only after the event behind its readers has
completed), and it grows once: a batch of 16384 one-token documents has lists
larger than half of the first 1 MiB ring.
"""
import numpy as np
import pytest
import torch

import variable_length_sequence_amd as vl
import workloads
from gpu_helpers import random_case, require_gpu, say

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(5)
    cases = []
    lq, lk, q, k, v, do = random_case(rng, 7, 0, 700, 8, 2, 128, ragged_k=True, seed=5)
    cases.append(("ragged", lq, lk, q, k, v, do, True))
    lt = workloads.longtail_16k().lengths
    w = workloads.Workload("longtail", lt, hq=8, hkv=2, d=128, seed=6)
    q, k, v, do = workloads.make_tensors(w)
    cases.append(("longtail_16k_h8", lt, lt, q, k, v, do, True))
    for n in (4096, 16384):
        ones = [1] * n
        w = workloads.Workload("ones", ones, hq=2, hkv=1, d=64, seed=7)
        q, k, v, do = workloads.make_tensors(w)
        cases.append((f"ones_{n}", ones, ones, q, k, v, do, n == 4096))
    lq, lk, q, k, v, do = random_case(rng, 5, 1, 300, 4, 4, 64, seed=8)
    cases.append(("noncausal_d64", lq, lk, q, k, v, do, False))
    return cases


def _run(case, dev):
    name, lq, lk, q, k, v, do, causal = case
    cq, ck = workloads.cu_seqlens(lq), workloads.cu_seqlens(lk)
    o, lse = vl.varlen_attn_fwd(q, k, v, cq, ck, causal=causal)
    o32, lse32 = vl.varlen_attn_fwd(q, k, v, cq, ck, causal=causal, out_dtype=torch.float32)
    dq, dk, dv = vl.varlen_attn_bwd(q, k, v, o, do, lse, cq, ck, causal=causal)
    return {"o": o, "lse": lse, "o32": o32, "lse32": lse32, "dq": dq, "dk": dk, "dv": dv}


def test_plan_cache_off_matches_cached_bitwise():
    dev = require_gpu()
    cases = []
    for c in _cases():
        name, lq, lk, q, k, v, do, causal = c
        cases.append((name, lq, lk, q.to(dev), k.to(dev), v.to(dev), do.to(dev), causal))
    prev = vl.set_plan_cache(True)
    try:
        ref = {c[0]: _run(c, dev) for c in cases}
        torch.cuda.synchronize()
        assert vl.set_plan_cache(False) is True
        got = []
        # interleaved, no synchronisation: the ring wraps and grows with
        # earlier uploads and kernels still in flight
        for rep in range(4):
            for c in cases:
                got.append((rep, c[0], _run(c, dev)))
        torch.cuda.synchronize()
    finally:
        vl.set_plan_cache(prev)
    for rep, name, res in got:
        for key, val in res.items():
            assert torch.equal(val, ref[name][key]), f"{name} rep {rep}: {key} differs"
    say(f"plan cache off: {len(got)} calls of {len(cases)} patterns bitwise equal to cached")


def test_plan_cache_off_fresh_pattern_every_call():
    # a new packing every call, as in training: each one is scheduled and
    # uploaded on its own; the results match the cached path
    dev = require_gpu()
    rng = np.random.default_rng(11)
    batches = []
    for i in range(12):
        lq, lk, q, k, v, do = random_case(rng, int(rng.integers(1, 12)), 0, 600, 4, 2, 128,
                                          seed=100 + i)
        batches.append(("b%d" % i, lq, lk, q.to(dev), k.to(dev), v.to(dev), do.to(dev), True))
    prev = vl.set_plan_cache(False)
    try:
        got = [_run(b, dev) for b in batches]
        torch.cuda.synchronize()
        vl.set_plan_cache(True)
        ref = [_run(b, dev) for b in batches]
    finally:
        vl.set_plan_cache(prev)
    for b, res, rf in zip(batches, got, ref):
        for key, val in res.items():
            assert torch.equal(val, rf[key]), f"{b[0]}: {key} differs"


def test_plan_cache_off_two_streams():
    # calls alternate between two streams: each upload and its kernels run
    # on the caller's stream, and each ring region waits for its own
    # stream's event before it is handed out again
    dev = require_gpu()
    rng = np.random.default_rng(13)
    batches = []
    for i in range(8):
        lq, lk, q, k, v, do = random_case(rng, int(rng.integers(1, 9)), 1, 500, 4, 2, 128,
                                          seed=200 + i)
        batches.append(("s%d" % i, lq, lk, q.to(dev), k.to(dev), v.to(dev), do.to(dev), True))
    prev = vl.set_plan_cache(True)
    try:
        ref = [_run(b, dev) for b in batches]
    finally:
        vl.set_plan_cache(prev)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    prev = vl.set_plan_cache(False)
    try:
        got = []
        for rep in range(3):
            for i, b in enumerate(batches):
                with torch.cuda.stream(streams[(i + rep) % 2]):
                    got.append((b[0], i, _run(b, dev)))
        torch.cuda.synchronize()
    finally:
        vl.set_plan_cache(prev)
    for name, i, res in got:
        for key, val in res.items():
            assert torch.equal(val, ref[i][key]), f"{name}: {key} differs"


def test_plan_cache_keys_the_head_layout():
    # the dK/dV list depends on the head counts (which key tiles have their
    # q-head group cut), so one cu_seqlens pattern with two head layouts gets
    # two cached lists: each layout's outputs equal its per-call result
    dev = require_gpu()
    lens = [3000, 257, 131, 64, 500, 1]
    cu = workloads.cu_seqlens(lens)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    layouts = [(8, 2), (8, 8), (8, 1)]
    cuts = [int(vl.varlen_schedule_export_dkdv(cu, cu, True, hq, hkv, n_cu)[:, 5].max())
            for hq, hkv in layouts]
    assert len(set(cuts)) > 1, cuts   # the layouts really cut differently
    cases = []
    for i, (hq, hkv) in enumerate(layouts):
        w = workloads.Workload(f"heads_{hq}_{hkv}", lens, hq=hq, hkv=hkv, d=128, seed=30 + i)
        q, k, v, do = (t.to(dev) for t in workloads.make_tensors(w))
        cases.append((w.name, lens, lens, q, k, v, do, True))
    prev = vl.set_plan_cache(False)
    try:
        ref = {c[0]: _run(c, dev) for c in cases}
        vl.set_plan_cache(True)
        vl.cache_clear()
        got = {c[0]: _run(c, dev) for c in cases + cases}
    finally:
        vl.set_plan_cache(prev)
    for name, res in got.items():
        for key, val in res.items():
            assert torch.equal(val, ref[name][key]), f"{name}: {key} differs"
    say(f"plan cache with head layouts {layouts} (cuts {cuts}) equal to per-call lists")
