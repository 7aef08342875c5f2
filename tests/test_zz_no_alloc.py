"""varlen_attn_bwd_noalloc, the backward for callers that cannot allocate
device memory, against varlen_attn_bwd (which takes a caller workspace) on
the same inputs: two calls in a row on the GPU, the second with a smaller
batch, each compared to the existing entry point (the same kernels, split
and work lists, so the gradients agree bit for bit; the bar is the
gradients' relative Frobenius error <= 5e-2).  Also: a batch whose D and
work lists do not fit the 128 MiB scratch is rejected with VL_EWORKSPACE.
"""
import ctypes

import numpy as np
import pytest
import torch

import variable_length_sequence_amd as vl
import workloads
from gpu_helpers import GRAD_REL_FRO, f64, rel_fro, require_gpu, say


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(q, k, v, o, do, lse, cu, causal=True):
    L = vl.lib()
    cu = np.ascontiguousarray(np.asarray(cu, np.int32))
    ip = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.varlen_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), ip, ip,
                                   len(cu) - 1, tq, tk, hq, hkv, d, 0.0, int(causal), _ptr(dq),
                                   _ptr(dk), _ptr(dv), st)
    assert rc == 0, L.varlen_last_error().decode()
    return dq, dk, dv


@pytest.mark.gpu
def test_noalloc_backward_matches_workspace_backward():
    dev = require_gpu()
    # one 4096-token document with 32/4 heads (the q-head groups of its early
    # key tiles are cut: the scratch holds D and the fp32 dK/dV partials), then a smaller ragged
    # GQA batch
    big = workloads.Workload("doc4k", [4096], hq=32, hkv=4, d=128, seed=4)
    small = workloads.Workload("ragged", [1, 37, 129, 300, 64], hq=8, hkv=2, d=64, seed=3)
    say(f"compute units: {torch.cuda.get_device_properties(0).multi_processor_count}")
    need = vl.bwd_workspace_bytes_cu(big.cu, big.cu, big.hq, big.hkv, big.d)
    assert need > (big.total * big.hq * 4 + 255) // 256 * 256, "the split path is not exercised"
    for w in (big, small):
        q, k, v, do = (t.to(dev) for t in workloads.make_tensors(w))
        cu = w.cu
        o, lse = vl.varlen_attn_fwd(q, k, v, cu, cu)
        ref = vl.varlen_attn_bwd(q, k, v, o, do, lse, cu, cu)
        got = _noalloc(q, k, v, o, do, lse, cu)
        torch.cuda.synchronize()
        errs = [rel_fro(f64(g), f64(r)) for g, r in zip(got, ref)]
        same = all(torch.equal(g, r) for g, r in zip(got, ref))
        say(f"noalloc {w.name}: rel-Fro vs varlen_attn_bwd dQ/dK/dV {errs}; bitwise equal {same}")
        assert max(errs) <= GRAD_REL_FRO


def test_noalloc_rejects_calls_beyond_its_scratch():
    # D alone of 2^21 tokens x 32 q heads is 256 MiB: rejected before any device work
    L = vl.lib()
    T = 1 << 21
    cu = np.array([0, T], np.int32)
    ip = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    f = ctypes.c_void_p(1 << 20)
    rc = L.varlen_attn_bwd_noalloc(f, f, f, f, f, f, ip, ip, 1, T, T, 32, 4, 128, 0.0, 1, f, f, f, None)
    assert rc == -6
    assert b"scratch" in L.varlen_last_error()
