"""The attention step captured in a HIP graph: with the plan cache on, after
one eager call has built and cached the work lists for a cu_seqlens pattern,
varlen_attn_fwd and varlen_attn_bwd only launch kernels, so a training step
can capture them.
Every replay (with eager work and synchronisations in between) must equal the
eager result bit for bit."""
import numpy as np
import pytest
import torch

import variable_length_sequence_amd as vl
import workloads
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu

CASES = [  # lengths, hq, hkv, d  (head splits of 1 and 2: both deterministic)
    ("longtail_16k", None, 32, 4, 128),
    ("ragged", [1, 300, 77, 1024, 0, 513], 8, 8, 64),
]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name,lengths,hq,hkv,d", CASES)
def test_graph_replay_equals_eager(name, lengths, hq, hkv, d):
    dev = require_gpu()
    w = workloads.longtail_16k() if lengths is None else workloads.Workload(name, lengths, hq=hq,
                                                                            hkv=hkv, d=d)
    say(f"graph capture {name}: {len(w.lengths)} docs, {w.total} tokens, {w.hq}/{w.hkv} heads")
    q, k, v, do = (t.to(dev) for t in workloads.make_tensors(w))
    cu = w.cu
    ws = torch.empty(vl.bwd_workspace_bytes(w.total, w.total, w.hq, w.hkv, w.d), dtype=torch.uint8,
                     device=dev)
    bufs = dict(o=torch.empty_like(q), lse=torch.empty(w.hq, w.total, dtype=torch.float32,
                                                           device=dev),
                dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v))

    def step():
        vl.varlen_attn_fwd(q, k, v, cu, cu, out=bufs["o"], lse=bufs["lse"])
        vl.varlen_attn_bwd(q, k, v, bufs["o"], do, bufs["lse"], cu, cu, workspace=ws,
                           dq=bufs["dq"], dk=bufs["dk"], dv=bufs["dv"])

    prev = vl.set_plan_cache(True)
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()                               # builds and caches the work lists
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        eager = {n: t.clone() for n, t in bufs.items()}

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
        for r in range(3):
            for t in bufs.values():
                t.fill_(0)                      # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for n in bufs:
                assert torch.equal(_bits(bufs[n]), _bits(eager[n])), (n, r)
    finally:
        vl.set_plan_cache(prev)
