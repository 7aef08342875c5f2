"""GPU parity of varlen_attn_fwd_acc, the forward folded into running (O, LSE).

Ring attention over key chunks (HSAP page, Section 2.2.1) computed two ways on
the GPU -- accumulated in the forward's epilogue, and as fp32 partials
merged by attn_lse_merge -- must agree to fp32 rounding, and both must match
full attention of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import variable_length_sequence_amd as vl
import workloads
from gpu_helpers import LSE_MAX_ABS, O_MAX_ABS, f64, lse_err, max_abs, require_gpu, say

pytestmark = pytest.mark.gpu


def _chunked(q, k, v, blocks, dev):
    """blocks: (k_slice, cu_q, cu_k, causal) per key chunk."""
    tq, hq, d = q.shape
    o_acc = torch.zeros((tq, hq, d), dtype=torch.float32, device=dev)
    lse_acc = torch.full((hq, tq), float("-inf"), dtype=torch.float32, device=dev)
    parts_o, parts_l = [], []
    for ks, cq, ck, causal in blocks:
        vl.varlen_attn_fwd_acc(q, k[ks], v[ks], cq, ck, o_acc, lse_acc, causal=causal)
        o_p, l_p = vl.varlen_attn_fwd(q, k[ks], v[ks], cq, ck, causal=causal, out_dtype=torch.float32)
        parts_o.append(o_p)
        parts_l.append(l_p)
    o_m, l_m = vl.attn_lse_merge(parts_o, parts_l, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return o_acc, lse_acc, o_m, l_m


def _compare(o_acc, lse_acc, o_m, l_m, ro, rlse, tag):
    d_o = max_abs(f64(o_acc), f64(o_m))
    fin = torch.isfinite(l_m)
    assert torch.equal(torch.isfinite(lse_acc), fin), "-inf rows differ"
    d_l = float((lse_acc[fin] - l_m[fin]).abs().max()) if fin.any() else 0.0
    eo = max_abs(f64(o_acc), ro)
    el = lse_err(f64(lse_acc), rlse)
    say(f"{tag}: acc vs merge O {d_o:.2e} LSE {d_l:.2e}; vs oracle O {eo:.3e} LSE {el:.3e}")
    assert d_o <= 1e-4 and d_l <= 1e-5
    assert eo <= O_MAX_ABS and el <= LSE_MAX_ABS


def test_fwd_acc_ring_share_single_document():
    dev = require_gpu()
    n, c = 4, 512
    w = workloads.Workload("ring_small", [n * c], hq=8, hkv=2, d=128, seed=4)
    q, k, v, _ = workloads.make_tensors(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    r = n - 1   # the last query chunk sees every key chunk
    blocks = [(slice(s * c, (s + 1) * c), [0, c], [0, c], s == r) for s in range(n)]
    res = _chunked(qd[r * c:], kd, vd, blocks, dev)
    ro, rlse = oracle.attn_fwd(f64(q), f64(k), f64(v), w.cu, w.cu, causal=True)
    _compare(*res, ro[r * c:], rlse[:, r * c:], "single doc, 4 chunks")


def test_fwd_acc_packed_ring_blocks():
    dev = require_gpu()
    lens = [224, 128, 64, 32, 64]
    n = 8
    w = workloads.Workload("ring_packed", lens, hq=4, hkv=4, d=64, seed=6)
    q, k, v, _ = workloads.make_tensors(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    c = sum(lens) // n
    ro, rlse = oracle.attn_fwd(f64(q), f64(k), f64(v), w.cu, w.cu, causal=True)
    for r in (3, 5, 7):
        blocks = []
        for s in range(n):
            cq, ck, causal, cls = vl.varlen_ring_block(w.cu, (r * c, (r + 1) * c), (s * c, (s + 1) * c))
            if cls != "N":
                blocks.append((slice(s * c, (s + 1) * c), cq, ck, causal))
        res = _chunked(qd[r * c:(r + 1) * c], kd, vd, blocks, dev)
        _compare(*res, ro[r * c:(r + 1) * c], rlse[:, r * c:(r + 1) * c], f"packed ring, query chunk {r}")


def test_fwd_acc_rows_without_keys_keep_zero():
    dev = require_gpu()
    # Lq > Lk with the causal diagonal at the bottom right: the first rows see
    # no key in either chunk and must stay (0, -inf)
    lq, lk = 96, 40
    w = workloads.Workload("nokeys", [lq], hq=2, hkv=2, d=64, seed=8)
    q, k, v, _ = workloads.make_tensors(w, tq=lq, tk=lk)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    blocks = [(slice(0, lk), [0, lq], [0, lk], True)]
    o_acc, lse_acc, o_m, l_m = _chunked(qd, kd, vd, blocks, dev)
    ro, rlse = oracle.attn_fwd(f64(q), f64(k), f64(v), [0, lq], [0, lk], causal=True)
    _compare(o_acc, lse_acc, o_m, l_m, ro, rlse, "rows without keys")
    none = np.isneginf(rlse)
    assert none.any()
    assert np.all(f64(o_acc)[np.transpose(none)] == 0.0)
