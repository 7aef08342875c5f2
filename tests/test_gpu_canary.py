"""Out-of-bounds write guard: every output (and the backward's workspace) sits
in the middle of a larger buffer whose 4 KiB pads on both sides are filled
with a sentinel byte; after the call the pads must be untouched and the
inputs unchanged.

Batches are ragged the ways document ends fall (HSAP page, Section 2.1,
cu_len; NSP page, Section 2.2, packing without padding): documents ending in
the middle of a tile, one-token and empty documents, Lq != Lk, grouped
query heads, head_dim 64 and 128.  The copy kernels get odd shapes that take
their 16-, 8-, 4- and 2-byte paths.
"""
import numpy as np
import pytest
import torch

import variable_length_sequence_amd as vl
import workloads
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu

PAD = 4096
SENT = 0x5A


class Guarded:
    """A tensor carved out of a sentinel-filled buffer with PAD bytes each side."""

    def __init__(self, shape, dtype, dev):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((PAD + n + PAD,), SENT, dtype=torch.uint8, device=dev)
        self.t = self.buf[PAD:PAD + n].view(dtype).view(shape)

    def intact(self):
        b = self.buf.cpu()
        return bool((b[:PAD] == SENT).all()) and bool((b[PAD + self.n:] == SENT).all())


def _ragged(rng, hq, hkv, d, ragged_k):
    lq = [1, 0, 37, 128, 129, 255, 64, 3, 200]
    lk = list(lq)
    if ragged_k:
        lk = [max(0, x + int(rng.integers(-20, 40))) for x in lq]
    w = workloads.Workload("canary", lq, hq=hq, hkv=hkv, d=d, seed=11)
    q, k, v, do = workloads.make_tensors(w, tq=sum(lq), tk=sum(lk))
    return workloads.cu_seqlens(lq), workloads.cu_seqlens(lk), q, k, v, do


@pytest.mark.parametrize("hq,hkv,d,ragged_k,causal", [
    (4, 4, 64, False, True), (8, 2, 128, False, True), (8, 1, 128, True, True),
    (4, 2, 64, True, False), (32, 4, 128, False, True)])
def test_attention_writes_stay_inside_outputs(hq, hkv, d, ragged_k, causal):
    dev = require_gpu()
    rng = np.random.default_rng(hq * 100 + d)
    cq, ck, q, k, v, do = _ragged(rng, hq, hkv, d, ragged_k)
    tq, tk = q.shape[0], k.shape[0]
    say(f"canary attention hq={hq} hkv={hkv} d={d} Tq={tq} Tk={tk} causal={causal}")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    keep = [t.clone() for t in (qd, kd, vd, dod)]
    out = Guarded((tq, hq, d), torch.bfloat16, dev)
    lse = Guarded((hq, tq), torch.float32, dev)
    vl.varlen_attn_fwd(qd, kd, vd, cq, ck, causal=causal, out=out.t, lse=lse.t)
    out32 = Guarded((tq, hq, d), torch.float32, dev)
    lse32 = Guarded((hq, tq), torch.float32, dev)
    vl.varlen_attn_fwd(qd, kd, vd, cq, ck, causal=causal, out=out32.t, lse=lse32.t)
    acc_o = Guarded((tq, hq, d), torch.float32, dev)
    acc_l = Guarded((hq, tq), torch.float32, dev)
    acc_o.t.zero_()
    acc_l.t.fill_(-float("inf"))
    vl.varlen_attn_fwd_acc(qd, kd, vd, cq, ck, acc_o.t, acc_l.t, causal=causal)
    dq = Guarded((tq, hq, d), torch.bfloat16, dev)
    dk = Guarded((tk, hkv, d), torch.bfloat16, dev)
    dv = Guarded((tk, hkv, d), torch.bfloat16, dev)
    need = vl.bwd_workspace_bytes_cu(cq, ck, hq, hkv, d, causal)
    ws = Guarded((need,), torch.uint8, dev)
    vl.varlen_attn_bwd(qd, kd, vd, out.t, dod, lse.t, cq, ck, causal=causal, workspace=ws.t,
                       dq=dq.t, dk=dk.t, dv=dv.t)
    torch.cuda.synchronize()
    for name, g in (("O", out), ("LSE", lse), ("O fp32", out32), ("LSE fp32", lse32),
                    ("O acc", acc_o), ("LSE acc", acc_l), ("dQ", dq), ("dK", dk), ("dV", dv),
                    ("workspace", ws)):
        assert g.intact(), f"{name}: a write landed outside the tensor"
    for a, b in zip(keep, (qd, kd, vd, dod)):
        assert torch.equal(a, b), "an input was modified"


@pytest.mark.parametrize("n,H,d,P,dtype", [
    (37, 8, 128, 4, torch.bfloat16), (19, 6, 12, 3, torch.bfloat16), (7, 4, 6, 2, torch.bfloat16),
    (5, 2, 3, 2, torch.bfloat16), (23, 8, 64, 8, torch.float32), (11, 6, 5, 3, torch.float32)])
def test_permutes_write_stay_inside_outputs(n, H, d, P, dtype):
    dev = require_gpu()
    say(f"canary permute n={n} H={H} d={d} P={P} {dtype}")
    x = torch.randn(n, H, d, device=dev).to(dtype)
    x0 = x.clone()
    y = Guarded((P, n, H // P, d), dtype, dev)
    vl.sp_seq2head(x, P, out=y.t)
    back = Guarded((n, H, d), dtype, dev)
    vl.sp_head2seq(y.t, out=back.t)
    torch.cuda.synchronize()
    assert y.intact() and back.intact()
    assert torch.equal(back.t, x0) and torch.equal(x, x0)


@pytest.mark.parametrize("n,hq,hkv,d,P,dtype", [
    (29, 8, 2, 64, 4, torch.bfloat16), (13, 8, 8, 128, 8, torch.bfloat16),
    (9, 16, 2, 128, 8, torch.bfloat16), (17, 4, 4, 6, 2, torch.float32)])
def test_qkv_packs_stay_inside_outputs(n, hq, hkv, d, P, dtype):
    dev = require_gpu()
    say(f"canary qkv n={n} hq={hq} hkv={hkv} d={d} P={P} {dtype}")
    q = torch.randn(n, hq, d, device=dev).to(dtype)
    k = torch.randn(n, hkv, d, device=dev).to(dtype)
    v = torch.randn(n, hkv, d, device=dev).to(dtype)
    hk = hkv // P if hkv >= P else 1
    outs = (Guarded((P, n, hq // P, d), dtype, dev), Guarded((P, n, hk, d), dtype, dev),
            Guarded((P, n, hk, d), dtype, dev))
    vl.sp_qkv_seq2head(q, k, v, P, out=tuple(g.t for g in outs))
    backs = (Guarded((n, hq, d), dtype, dev), Guarded((n, hkv, d), dtype, dev),
             Guarded((n, hkv, d), dtype, dev))
    vl.sp_qkv_head2seq(*(g.t for g in outs), hkv, out=tuple(g.t for g in backs))
    torch.cuda.synchronize()
    assert all(g.intact() for g in outs + backs)
    assert torch.equal(backs[0].t, q)


@pytest.mark.parametrize("n_parts,T,H,d,in_dt,out_dt", [
    (3, 37, 4, 64, torch.float32, torch.bfloat16), (1, 5, 2, 8, torch.bfloat16, torch.float32),
    (8, 129, 8, 128, torch.float32, torch.float32), (5, 1, 3, 4, torch.bfloat16, torch.bfloat16)])
def test_merge_stays_inside_outputs(n_parts, T, H, d, in_dt, out_dt):
    dev = require_gpu()
    say(f"canary merge parts={n_parts} T={T} H={H} d={d}")
    parts = [torch.randn(T, H, d, device=dev).to(in_dt) for _ in range(n_parts)]
    lses = [torch.randn(H, T, device=dev) for _ in range(n_parts)]
    o = Guarded((T, H, d), out_dt, dev)
    l = Guarded((H, T), torch.float32, dev)
    vl.attn_lse_merge(parts, lses, out=o.t, lse_out=l.t)
    torch.cuda.synchronize()
    assert o.intact() and l.intact()
