"""GPU parity of the Ulysses permute (bit-exact) and the (O, LSE) merge."""
import numpy as np
import pytest
import torch

import oracle
import variable_length_sequence_amd as vl
from gpu_helpers import require_gpu, say, f64, max_abs, lse_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,H,d,P,dtype", [
    (49152, 32, 128, 8, torch.bfloat16),   # one GPU's Ulysses shard of a 384K sequence
    (1000, 32, 128, 8, torch.bfloat16),
    (777, 12, 64, 4, torch.bfloat16),
    (513, 6, 5, 3, torch.bfloat16),        # 20-byte runs: 4-byte units
    (300, 4, 6, 2, torch.bfloat16),        # 24-byte runs: 8-byte units
    (101, 3, 3, 3, torch.bfloat16),        # 6-byte runs: 2-byte units
    (129, 8, 8, 8, torch.float32),
    (64, 16, 128, 1, torch.bfloat16),
    (1, 2, 128, 2, torch.float32),
    (0, 8, 128, 4, torch.bfloat16),
])
def test_permute_bit_exact(n, H, d, P, dtype):
    dev = require_gpu()
    say(f"permute n={n} H={H} d={d} P={P} {dtype}")
    g = torch.Generator().manual_seed(n + H + d + P)
    x = torch.randn(n, H, d, generator=g).to(dtype)
    xd = x.to(dev)
    y = vl.sp_seq2head(xd, P)
    ref = oracle.seq2head(x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy(), P)
    got = y.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy()
    assert np.array_equal(got, ref)
    back = vl.sp_head2seq(y)
    assert torch.equal(back.cpu(), x)


def test_permute_all_to_all_emulation():
    dev = require_gpu()
    P, n, H, d = 8, 512, 32, 128
    h = H // P
    X = torch.randn(P * n, H, d).to(torch.bfloat16)
    sent = [vl.sp_seq2head(X[r * n:(r + 1) * n].contiguous().to(dev), P) for r in range(P)]
    for g in range(P):
        recv = torch.cat([sent[r][g] for r in range(P)], dim=0).cpu()
        assert torch.equal(recv, X[:, g * h:(g + 1) * h, :])


def _partials(n_parts, t, h, d, dtype, gen, neg_inf_frac=0.1):
    os_, ls_ = [], []
    for _ in range(n_parts):
        os_.append(torch.randn(t, h, d, generator=gen).to(dtype))
        l = torch.randn(h, t, generator=gen) * 4
        mask = torch.rand(h, t, generator=gen) < neg_inf_frac
        l[mask] = -float("inf")
        ls_.append(l)
    # some rows empty in every partial
    for l in ls_:
        l[:, :3] = -float("inf")
    return os_, ls_


@pytest.mark.parametrize("n_parts,in_dt,out_dt", [
    (8, torch.float32, torch.bfloat16), (8, torch.float32, torch.float32),
    (3, torch.bfloat16, torch.bfloat16), (1, torch.float32, torch.float32),
    (16, torch.bfloat16, torch.float32), (5, torch.float32, torch.float32)])
def test_merge_matches_oracle(n_parts, in_dt, out_dt):
    dev = require_gpu()
    say(f"merge parts={n_parts} {in_dt}->{out_dt}")
    gen = torch.Generator().manual_seed(n_parts)
    t, h, d = 1027, 8, 128
    os_, ls_ = _partials(n_parts, t, h, d, in_dt, gen)
    o, l = vl.attn_lse_merge([x.to(dev) for x in os_], [x.to(dev) for x in ls_], out_dtype=out_dt)
    ro, rl = oracle.lse_merge([f64(x) for x in os_], [f64(x) for x in ls_])
    # fp32 arithmetic; a bf16 result adds at most half an ulp (2^-9 relative)
    rel = 1e-5 if out_dt == torch.float32 else 2.0 ** -8
    assert np.all(np.abs(f64(o) - ro) <= rel * np.maximum(np.abs(ro), 1.0))
    assert lse_err(f64(l), rl) < 1e-4
    assert torch.all(o[:3] == 0)


def test_merge_head_dim_64_and_small():
    dev = require_gpu()
    gen = torch.Generator().manual_seed(3)
    for d in (4, 64, 256):
        os_, ls_ = _partials(4, 100, 3, d, torch.float32, gen)
        o, l = vl.attn_lse_merge([x.to(dev) for x in os_], [x.to(dev) for x in ls_],
                                 out_dtype=torch.float32)
        ro, rl = oracle.lse_merge([f64(x) for x in os_], [f64(x) for x in ls_])
        assert max_abs(f64(o), ro) < 1e-5
        assert lse_err(f64(l), rl) < 1e-4
