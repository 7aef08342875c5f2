"""GPU parity of the ring share's backward at full size.

The ring share is query chunk 7 of one causal 262144-token sequence cut into
8 chunks of 32768 (8 q heads, 8 kv heads, head_dim 128).  Ring attention
runs the chunk's attention block by block over the key chunks (chunks 0-6
unmasked, chunk 7 causal) and merges the partial (O, LSE) pairs (HSAP page,
Section 2.2.1, InterSP ring; Section 3.2, Figure 3).  The backward of block
j, given the merged O and LSE, returns that block's share of dQ and the part
of dK and dV of key chunk j that comes from the chunk-7 queries; summed over
the blocks they are the gradient of attention restricted to those queries.

Checked against the oracle:
  * dQ on 512 sampled query rows per head (numpy default_rng(1)), computed by
    the oracle over the whole sequence;
  * dK and dV on 8 keys per key chunk per kv head, against the oracle's values
    stored in tests/golden/ring_256k_chunk7_bwd.npz (written by
    tests/golden/make_ring_bwd_golden.py, which calls only the oracle);
  * at every key, the closed-form sums of the restricted gradient: per kv
    head, sum_j dK_j = 0 and sum_j dV_j = sum over the chunk-7 queries of dO.
And the blockwise dQ against one call of the chunk against all its keys
(bottom-right-aligned causal), the same gradient computed without blocks.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import variable_length_sequence_amd as vl
import workloads
from gpu_helpers import GRAD_REL_FRO, f64, rel_fro, require_gpu, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "ring_256k_chunk7_bwd.npz")


@pytest.mark.timeout(900)
def test_ring_256k_chunk7_blockwise_backward():
    dev = require_gpu()
    gold = np.load(GOLDEN)
    w = workloads.ring_256k()
    n, c, qc = w.extra["n_chunks"], w.extra["chunk"], w.extra["q_chunk"]
    assert list(gold["shape"]) == [n, c, qc, w.hq, w.hkv, w.d, w.seed]
    q, k, v, do = workloads.make_tensors(w)
    q7 = q[qc * c:(qc + 1) * c].contiguous().to(dev)
    do7 = do[qc * c:(qc + 1) * c].contiguous().to(dev)
    kd, vd = k.to(dev), v.to(dev)
    one = np.array([0, c], np.int32)
    say(f"{w.name}: forward of query chunk {qc} over {n} key chunks, merged")
    parts_o, parts_l = [], []
    for j in range(n):
        o, l = vl.varlen_attn_fwd(q7, kd[j * c:(j + 1) * c], vd[j * c:(j + 1) * c], one, one,
                                  causal=(j == qc), out_dtype=torch.float32)
        parts_o.append(o)
        parts_l.append(l)
    om, lm = vl.attn_lse_merge(parts_o, parts_l, out_dtype=torch.bfloat16)
    del parts_o, parts_l
    say(f"{w.name}: blockwise backward with the merged O and LSE")
    dq = torch.zeros(c, w.hq, w.d, dtype=torch.float32, device=dev)
    dk = torch.empty_like(kd)
    dv = torch.empty_like(vd)
    for j in range(n):
        dq_j, dk[j * c:(j + 1) * c], dv[j * c:(j + 1) * c] = vl.varlen_attn_bwd(
            q7, kd[j * c:(j + 1) * c], vd[j * c:(j + 1) * c], om, do7, lm, one, one,
            causal=(j == qc))
        dq += dq_j.float()
    # the same gradient of dQ from one call over all keys
    dq1, _, _ = vl.varlen_attn_bwd(q7, kd, vd, om, do7, lm, one, np.array([0, n * c], np.int32),
                                   causal=True)
    torch.cuda.synchronize()
    dq, dq1, dk, dv = dq.cpu(), dq1.cpu(), dk.cpu(), dv.cpu()
    e_one = rel_fro(f64(dq), f64(dq1))

    rows, heads = workloads.sample_rows(c, 512, seed=1), None
    rows = np.concatenate([rows] * w.hq)
    heads = np.repeat(np.arange(w.hq), 512)
    full = np.array([0, n * c], np.int64)
    say(f"{w.name}: oracle dQ on {len(rows)} sampled rows")
    dq_r, _, _ = oracle.attn_bwd_dq_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                         do.float().numpy(), full, full, rows + qc * c, heads)
    eq = rel_fro(f64(dq[rows, heads]), dq_r)

    kr, kh = gold["krows"], gold["kheads"]
    ek = rel_fro(f64(dk[kr, kh]), gold["dk"])
    ev = rel_fro(f64(dv[kr, kh]), gold["dv"])
    per_chunk = []
    for j in range(n):
        sel = (kr >= j * c) & (kr < (j + 1) * c)
        per_chunk.append(max(rel_fro(f64(dk[kr[sel], kh[sel]]), gold["dk"][sel]),
                             rel_fro(f64(dv[kr[sel], kh[sel]]), gold["dv"][sel])))

    # closed-form sums over every key of the restricted gradient
    L = n * c
    dkd, dvd = dk.double(), dv.double()
    dod = do[qc * c:(qc + 1) * c].double()
    worst = 0.0
    for g in range(w.hkv):
        bound_k = GRAD_REL_FRO * np.sqrt(L) * float(dkd[:, g].norm())
        worst = max(worst, float(dkd[:, g].sum(0).norm()) / bound_k)
        bound_v = GRAD_REL_FRO * np.sqrt(L) * float(dvd[:, g].norm())
        worst = max(worst, float((dvd[:, g].sum(0) - dod[:, g].sum(0)).norm()) / bound_v)
    msg = (f"{w.name} backward: dQ {eq:.3e} (blockwise vs one call {e_one:.3e}); dK {ek:.3e} "
           f"dV {ev:.3e}; per key chunk {' '.join(f'{x:.2e}' for x in per_chunk)}; "
           f"sums {worst:.3f} of bound")
    say(msg)
    assert max(eq, ek, ev, *per_chunk) <= GRAD_REL_FRO, msg
    assert e_one <= 1e-2, msg
    assert worst <= 1.0, msg
