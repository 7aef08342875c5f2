"""GPU parity of the fused Q/K/V Ulysses pack and its gradient unpack with the
GQA kv-head split (bit-exact against the oracle, replica sums included)."""
import numpy as np
import pytest
import torch

from oracle import permute as operm
import variable_length_sequence_amd as vl
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu

CASES = [  # n, Hq, Hkv, d, P, dtype
    (49152, 32, 4, 128, 8, torch.bfloat16),   # a 384K sequence's shard, 32 q / 4 kv heads: kv x2
    (49152, 32, 8, 128, 8, torch.bfloat16),   # one kv head per rank
    (1000, 32, 4, 128, 8, torch.bfloat16),
    (777, 8, 1, 64, 8, torch.bfloat16),       # one kv head on all 8 ranks
    (513, 16, 2, 64, 4, torch.float32),
    (129, 16, 16, 128, 4, torch.bfloat16),    # MHA
    (300, 8, 2, 6, 4, torch.bfloat16),        # 12-byte heads: 4-byte units
    (301, 8, 4, 4, 2, torch.bfloat16),        # 8-byte heads: 8-byte units
    (1, 4, 1, 128, 2, torch.float32),
    (0, 8, 2, 128, 4, torch.bfloat16),
]


def _bits(t):
    return t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


def _rand(g, shape, dtype, offset=0):
    """A random tensor of dtype, optionally a view `offset` elements into a larger buffer."""
    n = int(np.prod(shape))
    buf = torch.randn(n + offset, generator=g).to(dtype)
    return buf, buf[offset:].view(shape)


def _expected_unpack(yq, yk, yv, Hkv, dtype):
    """The oracle's unpack: bits of dq, dk, dv."""
    dq = operm.head2seq(_bits(yq))
    Hq = yq.shape[0] * yq.shape[2]
    out = [dq]
    for y in (yk, yv):
        s = operm.kv_head2seq_sum(y.cpu().float().numpy(), Hq, Hkv,
                                  round_bf16=dtype == torch.bfloat16)
        u = s.view(np.uint32)
        out.append((u >> 16).astype(np.uint16).view(np.int16) if dtype == torch.bfloat16
                   else u.view(np.int32))
    return out


def _check(n, Hq, Hkv, d, P, dtype, offset=0):
    dev = require_gpu()
    say(f"qkv permute n={n} Hq={Hq} Hkv={Hkv} d={d} P={P} {dtype} offset={offset}")
    g = torch.Generator().manual_seed(n + 7 * Hq + 3 * Hkv + d + P)
    hk = Hkv // P if Hkv >= P else 1
    xs = [_rand(g, (n, H, d), dtype, offset)[1] for H in (Hq, Hkv, Hkv)]
    xd = [x.to(dev) if offset == 0 else _rand_dev(x, offset, dev) for x in xs]
    y = vl.sp_qkv_seq2head(*xd, P)
    want = operm.qkv_seq2head(*(_bits(x) for x in xs), P)
    for got, ref in zip(y, want):
        assert np.array_equal(_bits(got), ref)
    # gradient side: random chunks as the exchange would deliver them
    ys = [_rand(g, (P, n, h, d), dtype)[1] for h in (Hq // P, hk, hk)]
    outs = [_empty_dev((n, H, d), dtype, offset, dev) for H in (Hq, Hkv, Hkv)]
    vl.sp_qkv_head2seq(*(t.to(dev) for t in ys), Hkv, out=outs)
    for got, ref in zip(outs, _expected_unpack(*ys, Hkv, dtype)):
        assert np.array_equal(_bits(got), ref)


def _rand_dev(x, offset, dev):
    buf = torch.zeros(x.numel() + offset, dtype=x.dtype, device=dev)
    v = buf[offset:].view(x.shape)
    v.copy_(x.to(dev))
    return v


def _empty_dev(shape, dtype, offset, dev):
    buf = torch.full((int(np.prod(shape)) + offset,), 7.0, dtype=dtype, device=dev)
    return buf[offset:].view(shape)


@pytest.mark.parametrize("n,Hq,Hkv,d,P,dtype", CASES)
def test_qkv_pack_and_unpack_bit_exact(n, Hq, Hkv, d, P, dtype):
    _check(n, Hq, Hkv, d, P, dtype)


@pytest.mark.parametrize("offset", [2, 4])
def test_qkv_misaligned_views(offset):
    # views 4 and 8 bytes into their buffers take the narrower copy units
    _check(515, 16, 2, 128, 8, torch.bfloat16, offset)


def test_qkv_round_trip_replicated_heads():
    dev = require_gpu()
    say("qkv round trip n=4096 Hq=32 Hkv=2 d=128 P=8")
    g = torch.Generator().manual_seed(5)
    q = torch.randn(4096, 32, 128, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(4096, 2, 128, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(4096, 2, 128, generator=g).to(torch.bfloat16).to(dev)
    dq, dk, dv = vl.sp_qkv_head2seq(*vl.sp_qkv_seq2head(q, k, v, 8), 2)
    assert torch.equal(dq, q)
    # each kv head went to 4 ranks: the sum is 4 x, exact in fp32 and in bf16
    assert torch.equal(dk, (4 * k.float()).to(torch.bfloat16))
    assert torch.equal(dv, (4 * v.float()).to(torch.bfloat16))
