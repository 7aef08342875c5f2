"""Full-tensor GPU parity on one long document: 16384 tokens, 8 q heads
sharing 1 kv head, head_dim 128, causal.

Every element of O, LSE, dQ, dK and dV is compared with the fp64 oracle (the
plain per-document softmax and its analytic gradient), so the longest
accumulations are checked element by element: the first key tile's dK/dV
sum over all 512 query tiles of 32 rows x 8 q heads, and the last query
tile's O and dQ over 256 key tiles.  With a group of 8 q heads on one kv
head the backward cuts the group of the early key tiles into 4 slices and
of the middle ones into 2 (their fp32 partials added in a fixed order) and
keeps the late ones whole, the mix the 393216-token Ulysses share takes at
full size.  The attention is the one the pages define per document (BASP
page, Section II-A; HSAP page, Section 2.2.1); its gradient is recomputed
from the saved LSE (NSP page, Sections 2.3 and 4.2.2).
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


@pytest.mark.timeout(900)
def test_one_16k_document_full_tensors():
    dev = require_gpu()
    w = workloads.Workload("doc16k", [16384], hq=8, hkv=1, d=128, seed=5)
    q, k, v, do = workloads.make_tensors(w)
    cu = w.cu
    say(f"{w.name}: one document of {w.total} tokens, {w.hq}/{w.hkv} heads, d {w.d}")
    # the backward takes the split path: D plus room for four fp32 dK/dV partials
    delta = (w.total * w.hq * 4 + 255) // 256 * 256
    part = (4 * 2 * w.total * w.hkv * w.d * 4 + 255) // 256 * 256
    assert vl.bwd_workspace_bytes_cu(cu, cu, w.hq, w.hkv, w.d) == delta + part
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = vl.varlen_attn_fwd(qd, kd, vd, cu, cu, causal=True)
    dq, dk, dv = vl.varlen_attn_bwd(qd, kd, vd, o, dod, lse, cu, cu, causal=True)
    torch.cuda.synchronize()
    say(f"{w.name}: fp64 oracle on the full tensors")
    dq_r, dk_r, dv_r, o_r, lse_r = oracle.attn_bwd(q.float().numpy(), k.float().numpy(),
                                                   v.float().numpy(), do.float().numpy(), cu, cu,
                                                   causal=True, return_fwd=True)
    eo = max_abs(f64(o), o_r)
    el = lse_err(f64(lse), lse_r)
    eq, ek, ev = rel_fro(f64(dq), dq_r), rel_fro(f64(dk), dk_r), rel_fro(f64(dv), dv_r)
    # the keys with the longest accumulation: the first 128 (one dK/dV tile)
    ek0 = rel_fro(f64(dk[:128]), dk_r[:128])
    ev0 = rel_fro(f64(dv[:128]), dv_r[:128])
    # the queries with the longest accumulation: the last 128
    eq1 = rel_fro(f64(dq[-128:]), dq_r[-128:])
    msg = (f"{w.name}: O {eo:.3e} LSE {el:.3e} dQ {eq:.3e} dK {ek:.3e} dV {ev:.3e}; "
           f"first key tile dK {ek0:.3e} dV {ev0:.3e}; last query tile dQ {eq1:.3e}")
    say(msg)
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS, msg
    assert max(eq, ek, ev, ek0, ev0, eq1) <= GRAD_REL_FRO, msg
