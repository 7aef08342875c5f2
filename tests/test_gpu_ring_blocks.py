"""GPU parity of ring attention over a packed causal batch, block by block.

The packed token axis is cut into contiguous chunks (one per ring rank); each
(query chunk, key chunk) block is one varlen_attn_fwd call whose documents
and causal flag come from varlen_ring_block (HSAP page, Section 3.2 and
Figure 3); attn_lse_merge over the key chunks gives the rows of a query
chunk (HSAP page, Section 2.2.1).  For the backward, every block runs
varlen_attn_bwd with the merged O and LSE; the blocks' dq shares summed over
key chunks and their dk/dv shares summed over query chunks must equal the
gradients of attention over the whole packed batch (fp64 oracle).
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


def _ring(lengths, n_chunks, hq, hkv, d, seed):
    dev = require_gpu()
    w = workloads.Workload("ring_packed", lengths, hq=hq, hkv=hkv, d=d, seed=seed)
    q, k, v, do = workloads.make_tensors(w)
    cu = w.cu
    total = int(cu[-1])
    assert total % n_chunks == 0
    c = total // n_chunks
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    blocks = {}
    classes = []
    o_rows, lse_rows = [], []
    for r in range(n_chunks):
        parts_o, parts_l = [], []
        row = []
        for s in range(n_chunks):
            cq, ck, causal, cls = vl.varlen_ring_block(cu, (r * c, (r + 1) * c), (s * c, (s + 1) * c))
            row.append(cls)
            if cls == "N":
                continue
            o_p, l_p = vl.varlen_attn_fwd(qd[r * c:(r + 1) * c], kd[s * c:(s + 1) * c],
                                          vd[s * c:(s + 1) * c], cq, ck, causal=causal,
                                          out_dtype=torch.float32)
            parts_o.append(o_p)
            parts_l.append(l_p)
            blocks[(r, s)] = (cq, ck, causal)
        classes.append(row)
        o_r, l_r = vl.attn_lse_merge(parts_o, parts_l, out_dtype=torch.bfloat16)
        o_rows.append(o_r)
        lse_rows.append(l_r)
    o = torch.cat(o_rows, 0)
    lse = torch.cat(lse_rows, 1).contiguous()
    # backward: each block with the merged O and LSE
    dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=dev)
    for (r, s), (cq, ck, causal) in blocks.items():
        g = vl.varlen_attn_bwd(qd[r * c:(r + 1) * c], kd[s * c:(s + 1) * c], vd[s * c:(s + 1) * c],
                               o[r * c:(r + 1) * c], dod[r * c:(r + 1) * c],
                               lse[:, r * c:(r + 1) * c].contiguous(), cq, ck, causal=causal)
        dq[r * c:(r + 1) * c] += g[0].float()
        dk[s * c:(s + 1) * c] += g[1].float()
        dv[s * c:(s + 1) * c] += g[2].float()
    torch.cuda.synchronize()
    rdq, rdk, rdv, ro, rlse = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), cu, cu, causal=True,
                                              return_fwd=True)
    eo = max_abs(f64(o), ro)
    el = lse_err(f64(lse), rlse)
    g = [rel_fro(f64(x), y) for x, y in ((dq, rdq), (dk, rdk), (dv, rdv))]
    say(f"ring {lengths} / {n_chunks} chunks: classes {classes}")
    say(f"  O max|err| {eo:.3e}  LSE max|err| {el:.3e}  rel-Fro dQ {g[0]:.3e} dK {g[1]:.3e} dV {g[2]:.3e}")
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS
    assert max(g) <= GRAD_REL_FRO
    return classes


def test_ring_blocks_hsap_figure3_packing():
    # the HSAP Figure 3 packing (documents ending at chunk positions 3.5, 5.5,
    # 6.5, 7) scaled from 8 to 64 tokens per chunk: every block class occurs
    classes = _ring([224, 128, 64, 32, 64], 8, 4, 2, 64, seed=3)
    seen = {x for row in classes for x in row}
    assert {"A1", "A2", "A3", "A4", "A5", "N"} <= seen


def test_ring_blocks_long_tail_packing_gqa_d128():
    rng = np.random.default_rng(11)
    lens = workloads.random_lengths(rng, 9, 1, 700)
    total = sum(lens)
    pad = (-total) % 512
    lens = list(lens) + ([pad] if pad else [])
    _ring(lens, 4, 8, 2, 128, seed=5)
