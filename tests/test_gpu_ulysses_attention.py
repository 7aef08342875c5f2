"""Ulysses attention end to end on one GPU with P emulated ranks.

Each rank holds a token shard of a packed batch; sp_qkv_seq2head packs its
Q, K, V for the exchange (kv heads replicated when Hkv < P); the all-to-all
is emulated by concatenating the chunks each rank receives; every rank runs
packed varlen attention over the whole sequence for its heads, and
sp_seq2head / sp_head2seq take O back to the token split.  The backward runs
the same way and sp_qkv_head2seq sums the replicas' kv gradients.  The result
must match the oracle's global GQA attention and gradients (HSAP page,
Section 2.2.2; BASP page, Section II-C).
"""
import numpy as np
import pytest
import torch

import oracle
import variable_length_sequence_amd as vl
import workloads
from gpu_helpers import (GRAD_REL_FRO, LSE_MAX_ABS, O_MAX_ABS, f64, lse_err, max_abs, rel_fro,
                         require_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lengths,P,hq,hkv,d", [
    ([300, 1200, 77, 500, 971], 4, 16, 2, 128),    # kv heads replicated to 2 ranks
    ([2048, 1024, 512, 512], 8, 32, 8, 64),         # one kv head per rank
])
def test_ulysses_attention_matches_global_attention(lengths, P, hq, hkv, d):
    dev = require_gpu()
    w = workloads.Workload("ulysses", lengths, hq=hq, hkv=hkv, d=d, seed=5)
    q, k, v, do = workloads.make_tensors(w)
    cu = w.cu
    N = int(cu[-1])
    assert N % P == 0
    n = N // P
    say(f"ulysses emulation: {len(lengths)} docs, {N} tokens, P={P}, {hq}/{hkv} heads, d={d}")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    rows = [slice(s * n, (s + 1) * n) for s in range(P)]
    packs = [vl.sp_qkv_seq2head(qd[r].contiguous(), kd[r].contiguous(), vd[r].contiguous(), P)
             for r in rows]
    do_packs = [vl.sp_seq2head(dod[r].contiguous(), P) for r in rows]

    def recv(chunks, p):        # what rank p receives: chunk p of every source, in source order
        return torch.cat([c[p] for c in chunks], 0).contiguous()

    o_heads, lse_heads, grads = [], [], []
    for p in range(P):
        qp = recv([pk[0] for pk in packs], p)
        kp = recv([pk[1] for pk in packs], p)
        vp = recv([pk[2] for pk in packs], p)
        dop = recv(do_packs, p)
        o_p, lse_p = vl.varlen_attn_fwd(qp, kp, vp, cu, cu, causal=True)
        grads.append(vl.varlen_attn_bwd(qp, kp, vp, o_p, dop, lse_p, cu, cu, causal=True))
        o_heads.append(o_p)
        lse_heads.append(lse_p)
    # O back to the token split: rank p sends its rows of source s back to s
    o_back = [vl.sp_head2seq(torch.stack([o_heads[p][r] for p in range(P)]).contiguous())
              for r in rows]
    o = torch.cat(o_back, 0)
    lse = torch.cat(lse_heads, 0)
    g_back = [vl.sp_qkv_head2seq(*(torch.stack([grads[p][i][r] for p in range(P)]).contiguous()
                                   for i in range(3)), hkv) for r in rows]
    dq = torch.cat([g[0] for g in g_back], 0)
    dk = torch.cat([g[1] for g in g_back], 0)
    dv = torch.cat([g[2] for g in g_back], 0)

    o_ref, lse_ref = oracle.attn_fwd(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                     cu, cu, True)
    dq_r, dk_r, dv_r = oracle.attn_bwd(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                       do.float().numpy(), cu, cu, True)
    assert max_abs(f64(o), o_ref) <= O_MAX_ABS
    assert lse_err(f64(lse), lse_ref) <= LSE_MAX_ABS
    for got, ref, name in ((dq, dq_r, "dq"), (dk, dk_r, "dk"), (dv, dv_r, "dv")):
        e = rel_fro(f64(got), ref)
        say(f"  {name} rel-Fro {e:.2e}")
        assert e <= GRAD_REL_FRO, name
