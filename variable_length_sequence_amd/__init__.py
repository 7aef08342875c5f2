"""Python binding of libvarlen: packed variable-length causal attention on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libvarlen.so`` (built in-tree by ``build.py``); PyTorch supplies
device memory and the current stream.  There is no CPU fallback: if the
library is missing every call raises.

Entry points (same names as the C ABI in ``include/varlen.h``):
  varlen_attn_fwd(q, k, v, cu_q, cu_k, causal=True, scale=None, out_dtype=bf16) -> (o, lse)
  varlen_attn_bwd(q, k, v, o, do, lse, cu_q, cu_k, causal=True, scale=None) -> (dq, dk, dv)
  attn_lse_merge(o_parts, lse_parts, out_dtype=bf16) -> (o, lse)
  sp_seq2head(x, sp_degree) -> y ;  sp_head2seq(y) -> x
  sp_qkv_seq2head(q, k, v, sp_degree) -> (yq, yk, yv)
  sp_qkv_head2seq(yq, yk, yv, n_heads_kv) -> (dq, dk, dv)
  basp_shard(rank, world, batch, seq_len) -> dict (host only)
  nsp_route(lengths, n_gpus, sp_max, cost, token_budget, prefix, beam) -> dict (host only)
  nsp_plan_cost(lengths, plan, n_gpus, sp_max, cost) -> dict (host only)
  varlen_schedule_export(cu_q, cu_k, causal, pass_, head_dim) -> dict (host only)
  varlen_schedule_export_dkdv(cu_q, cu_k, causal, hq, hkv, n_cu) -> int32 [n, 6] (host only)
  varlen_ring_block(cu, q_range, k_range) -> (cu_q, cu_k, causal, cls) (host only)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvarlen.so")

VL_BF16, VL_F32 = 0, 1
STATUS = {0: "VL_OK", -1: "VL_EINVAL", -2: "VL_ESHAPE", -3: "VL_ESEQLENS",
          -4: "VL_EUNSUPPORTED", -5: "VL_EHIP", -6: "VL_EWORKSPACE"}

EXPORTS = ["varlen_attn_fwd", "varlen_attn_bwd_workspace_size", "varlen_attn_bwd_workspace_size_cu",
           "varlen_attn_bwd", "varlen_attn_bwd_noalloc",
           "attn_lse_merge", "sp_seq2head", "sp_head2seq", "varlen_schedule_export",
           "varlen_schedule_export_dkdv",
           "varlen_last_error", "varlen_cache_clear", "varlen_set_plan_cache", "varlen_version",
           "varlen_profile_enable", "varlen_profile_read", "varlen_ring_block", "varlen_attn_fwd_acc", "sp_qkv_seq2head",
           "sp_qkv_head2seq", "basp_shard", "nsp_route", "nsp_plan_cost", "varlen_mfma_probe"]

RING_CLASSES = ("N", "A1", "A2", "A3", "A4", "A5")


class VarlenError(RuntimeError):
    """A libvarlen call returned a negative status."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class _CostModelC(ctypes.Structure):
    _fields_ = [("n_points", ctypes.c_int32), ("curve_len", ctypes.POINTER(ctypes.c_double)),
                ("fwd_tflops", ctypes.POINTER(ctypes.c_double)),
                ("bwd_tflops", ctypes.POINTER(ctypes.c_double)),
                ("fwd_flops_per_pair", ctypes.c_double), ("bwd_flops_per_pair", ctypes.c_double),
                ("bytes_per_token", ctypes.c_double * 4), ("a2a_gbs", ctypes.c_double),
                ("a2a_alpha_us", ctypes.c_double), ("dense_fwd_flops_per_token", ctypes.c_double),
                ("dense_bwd_flops_per_token", ctypes.c_double), ("dense_tflops", ctypes.c_double)]


_lib = None


def lib():
    """The loaded libvarlen.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m variable_length_sequence_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    pi32, pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    L.varlen_attn_fwd.argtypes = [vp, vp, vp, pi32, pi32, i32, i64, i64, i32, i32, i32, f32, i32,
                                  i32, vp, vp, vp]
    L.varlen_attn_fwd.restype = ctypes.c_int
    L.varlen_attn_fwd_acc.argtypes = [vp, vp, vp, pi32, pi32, i32, i64, i64, i32, i32, i32, f32,
                                      i32, vp, vp, vp]
    L.varlen_attn_fwd_acc.restype = ctypes.c_int
    L.varlen_attn_bwd_workspace_size.argtypes = [i64, i64, i32, i32, i32]
    L.varlen_attn_bwd_workspace_size.restype = ctypes.c_size_t
    L.varlen_attn_bwd_workspace_size_cu.argtypes = [pi32, pi32, i32, i64, i64, i32, i32, i32, i32]
    L.varlen_attn_bwd_workspace_size_cu.restype = ctypes.c_size_t
    L.varlen_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, pi32, pi32, i32, i64, i64, i32, i32, i32,
                                  f32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.varlen_attn_bwd.restype = ctypes.c_int
    L.varlen_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, pi32, pi32, i32, i64, i64, i32,
                                          i32, i32, f32, i32, vp, vp, vp, vp]
    L.varlen_attn_bwd_noalloc.restype = ctypes.c_int
    L.attn_lse_merge.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i64, i32, i32,
                                 vp, vp, i32, vp]
    L.attn_lse_merge.restype = ctypes.c_int
    for n in ("sp_seq2head", "sp_head2seq"):
        getattr(L, n).argtypes = [vp, vp, i64, i32, i32, i32, i32, vp]
        getattr(L, n).restype = ctypes.c_int
    for n in ("sp_qkv_seq2head", "sp_qkv_head2seq"):
        getattr(L, n).argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, vp]
        getattr(L, n).restype = ctypes.c_int
    L.basp_shard.argtypes = [i32, i32, i32, i64, pi32, pi32, pi32, pi32, pi64, pi64]
    L.basp_shard.restype = ctypes.c_int
    pd = ctypes.POINTER(ctypes.c_double)
    L.nsp_route.argtypes = [pi64, i32, i32, i32, ctypes.POINTER(_CostModelC), ctypes.c_double, i32,
                            i32, i32, i32, pi32, pi32, pd, pd, pd, pi32]
    L.nsp_route.restype = ctypes.c_int
    L.nsp_plan_cost.argtypes = [pi64, i32, i32, i32, ctypes.POINTER(_CostModelC), pi32, pi32, pd,
                                pd, pd]
    L.nsp_plan_cost.restype = ctypes.c_int
    L.varlen_mfma_probe.argtypes = [i32, i32, vp, pi64, vp]
    L.varlen_mfma_probe.restype = ctypes.c_int
    L.varlen_schedule_export.argtypes = [pi32, pi32, i32, i32, i32, i32, pi32, i64, pi64, pi64,
                                         pi64, pi32, pi32]
    L.varlen_schedule_export.restype = ctypes.c_int
    L.varlen_schedule_export_dkdv.argtypes = [pi32, pi32, i32, i32, i32, i32, i32, pi32, i64, pi64]
    L.varlen_schedule_export_dkdv.restype = ctypes.c_int
    L.varlen_ring_block.argtypes = [pi32, i32, i64, i64, i64, i64, pi32, pi32, pi32, pi32]
    L.varlen_ring_block.restype = ctypes.c_int
    L.varlen_last_error.argtypes = []
    L.varlen_last_error.restype = ctypes.c_char_p
    L.varlen_cache_clear.argtypes = []
    L.varlen_cache_clear.restype = None
    L.varlen_set_plan_cache.argtypes = [ctypes.c_int32]
    L.varlen_set_plan_cache.restype = ctypes.c_int
    L.varlen_version.argtypes = []
    L.varlen_version.restype = ctypes.c_int
    L.varlen_profile_enable.argtypes = [i32]
    L.varlen_profile_enable.restype = ctypes.c_int
    L.varlen_profile_read.argtypes = [i32, ctypes.c_char_p, i32, pi64, ctypes.POINTER(ctypes.c_double)]
    L.varlen_profile_read.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise VarlenError(rc, lib().varlen_last_error().decode())


def _cu_host(cu) -> np.ndarray:
    """cu_seqlens as a contiguous host int32 array (a device tensor is copied, which syncs)."""
    try:
        import torch
        if isinstance(cu, torch.Tensor):
            cu = cu.detach().to("cpu")
            return np.ascontiguousarray(cu.numpy().astype(np.int32))
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(cu, dtype=np.int32))


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _want(t, name: str, shape, dtypes, device=None):
    """Check a tensor argument before any pointer reaches the library: the C
    ABI derives every size from q and k, so a mismatched second input or
    output buffer would be read or written out of bounds."""
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise TypeError(f"{name} must be {names}, got {str(t.dtype).replace('torch.', '')}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _qkv_shapes(q, k, v):
    """(tq, hq, d, tk, hkv) of bf16 q [Tq,Hq,d] and k, v [Tk,Hkv,d]."""
    import torch
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [Tq, Hq, d] and k, v [Tk, Hkv, d]")
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if dk != d:
        raise ValueError(f"q and k must share head_dim, got {d} and {dk}")
    bf = (torch.bfloat16,)
    _want(q, "q", (tq, hq, d), bf)
    _want(k, "k", (tk, hkv, d), bf, q.device)
    _want(v, "v", (tk, hkv, d), bf, q.device)
    return tq, hq, d, tk, hkv


def _dev_ptr(t) -> ctypes.c_void_p:
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def varlen_attn_fwd(q, k, v, cu_q, cu_k, causal: bool = True, scale: Optional[float] = None,
                    out_dtype=None, out=None, lse=None):
    """Packed varlen attention forward.  q [Tq,Hq,d], k/v [Tk,Hkv,d] bf16 -> (o, lse[Hq,Tq])."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    cq, ck = _cu_host(cu_q), _cu_host(cu_k)
    tq, hq, d, tk, hkv = _qkv_shapes(q, k, v)
    if out is None:
        out = torch.empty((tq, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _want(out, "out", (tq, hq, d), (torch.bfloat16, torch.float32), q.device)
    _want(lse, "lse", (hq, tq), (torch.float32,), q.device)
    od = VL_F32 if out.dtype == torch.float32 else VL_BF16
    _check(lib().varlen_attn_fwd(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _iptr(cq), _iptr(ck),
                                 len(cq) - 1, tq, tk, hq, hkv, d, float(scale or 0.0), int(causal),
                                 od, _dev_ptr(out), _dev_ptr(lse), _stream()))
    return out, lse


def varlen_attn_fwd_acc(q, k, v, cu_q, cu_k, o_acc, lse_acc, causal: bool = True,
                        scale: Optional[float] = None):
    """Forward over these keys folded into running fp32 accumulators o_acc
    [Tq,Hq,d] and lse_acc [Hq,Tq] (in place; start from 0 and -inf)."""
    import torch
    cq, ck = _cu_host(cu_q), _cu_host(cu_k)
    tq, hq, d, tk, hkv = _qkv_shapes(q, k, v)
    _want(o_acc, "o_acc", (tq, hq, d), (torch.float32,), q.device)
    _want(lse_acc, "lse_acc", (hq, tq), (torch.float32,), q.device)
    _check(lib().varlen_attn_fwd_acc(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _iptr(cq), _iptr(ck),
                                     len(cq) - 1, tq, tk, hq, hkv, d, float(scale or 0.0),
                                     int(causal), _dev_ptr(o_acc), _dev_ptr(lse_acc), _stream()))
    return o_acc, lse_acc


def varlen_attn_bwd(q, k, v, o, do, lse, cu_q, cu_k, causal: bool = True,
                    scale: Optional[float] = None, workspace=None, dq=None, dk=None, dv=None):
    """Packed varlen attention backward -> (dq, dk, dv), bf16 (written into the
    given tensors when passed)."""
    import torch
    cq, ck = _cu_host(cu_q), _cu_host(cu_k)
    tq, hq, d, tk, hkv = _qkv_shapes(q, k, v)
    bf = (torch.bfloat16,)
    _want(o, "o", (tq, hq, d), bf, q.device)
    _want(do, "do", (tq, hq, d), bf, q.device)
    _want(lse, "lse", (hq, tq), (torch.float32,), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _want(dq, "dq", (tq, hq, d), bf, q.device)
    _want(dk, "dk", (tk, hkv, d), bf, q.device)
    _want(dv, "dv", (tk, hkv, d), bf, q.device)
    need = lib().varlen_attn_bwd_workspace_size_cu(_iptr(cq), _iptr(ck), len(cq) - 1, tq, tk, hq,
                                                   hkv, d, int(causal))
    if workspace is None:
        workspace = torch.empty(max(int(need), 256), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")
    _check(lib().varlen_attn_bwd(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(o), _dev_ptr(do),
                                 _dev_ptr(lse), _iptr(cq), _iptr(ck), len(cq) - 1, tq, tk, hq, hkv,
                                 d, float(scale or 0.0), int(causal), _dev_ptr(dq), _dev_ptr(dk),
                                 _dev_ptr(dv), _dev_ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dv


def bwd_workspace_bytes(tq: int, tk: int, hq: int, hkv: int, d: int) -> int:
    """Workspace bound for any batch of these sizes."""
    return int(lib().varlen_attn_bwd_workspace_size(tq, tk, hq, hkv, d))


def bwd_workspace_bytes_cu(cu_q, cu_k, hq: int, hkv: int, d: int, causal: bool = True) -> int:
    """Workspace this batch needs on the current device."""
    cq, ck = _cu_host(cu_q), _cu_host(cu_k)
    return int(lib().varlen_attn_bwd_workspace_size_cu(_iptr(cq), _iptr(ck), len(cq) - 1,
                                                       int(cq[-1]), int(ck[-1]), hq, hkv, d,
                                                       int(causal)))


def attn_lse_merge(o_parts: Sequence, lse_parts: Sequence, out_dtype=None, out=None, lse_out=None):
    """Merge partial (O [T,H,d], LSE [H,T]) results over disjoint key sets."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    n = len(o_parts)
    if n == 0 or n != len(lse_parts):
        raise ValueError("need the same positive number of O and LSE partials")
    if o_parts[0].dim() != 3:
        raise ValueError("partial O must be [T, H, d]")
    t, h, d = o_parts[0].shape
    in_dt = o_parts[0].dtype
    if in_dt not in (torch.bfloat16, torch.float32):
        raise TypeError("partial O must be bfloat16 or float32")
    dev = o_parts[0].device
    for i, (o, l) in enumerate(zip(o_parts, lse_parts)):
        _want(o, f"o_parts[{i}]", (t, h, d), (in_dt,), dev)
        _want(l, f"lse_parts[{i}]", (h, t), (torch.float32,), dev)
    if out is None:
        out = torch.empty((t, h, d), dtype=out_dtype, device=dev)
    if lse_out is None:
        lse_out = torch.empty((h, t), dtype=torch.float32, device=dev)
    _want(out, "out", (t, h, d), (torch.bfloat16, torch.float32), dev)
    _want(lse_out, "lse_out", (h, t), (torch.float32,), dev)
    op = (ctypes.c_void_p * n)(*[_dev_ptr(o).value for o in o_parts])
    lp = (ctypes.c_void_p * n)(*[_dev_ptr(l).value for l in lse_parts])
    idt = VL_F32 if in_dt == torch.float32 else VL_BF16
    odt = VL_F32 if out.dtype == torch.float32 else VL_BF16
    _check(lib().attn_lse_merge(n, op, lp, idt, t, h, d, _dev_ptr(out), _dev_ptr(lse_out), odt,
                                _stream()))
    return out, lse_out


def sp_seq2head(x, sp_degree: int, out=None):
    """[n, H, d] -> [P, n, H/P, d] (chunk p = heads p*H/P .. (p+1)*H/P - 1)."""
    import torch
    if x.dim() != 3:
        raise ValueError("x must be [n, H, d]")
    n, H, d = x.shape
    if sp_degree <= 0 or H % sp_degree:
        raise ValueError("sp_degree must divide the head count")
    if x.element_size() not in (2, 4):
        raise TypeError("elements must be 2 or 4 bytes")
    if out is None:
        out = torch.empty((sp_degree, n, H // sp_degree, d), dtype=x.dtype, device=x.device)
    _want(out, "out", (sp_degree, n, H // sp_degree, d), (x.dtype,), x.device)
    _check(lib().sp_seq2head(_dev_ptr(x), _dev_ptr(out), n, H, d, sp_degree, x.element_size(),
                             _stream()))
    return out


def sp_head2seq(y, out=None):
    """[P, n, h, d] -> [n, P*h, d], the inverse of sp_seq2head."""
    import torch
    if y.dim() != 4:
        raise ValueError("y must be [P, n, h, d]")
    P, n, h, d = y.shape
    if y.element_size() not in (2, 4):
        raise TypeError("elements must be 2 or 4 bytes")
    if out is None:
        out = torch.empty((n, P * h, d), dtype=y.dtype, device=y.device)
    _want(out, "out", (n, P * h, d), (y.dtype,), y.device)
    _check(lib().sp_head2seq(_dev_ptr(y), _dev_ptr(out), n, P * h, d, P, y.element_size(),
                             _stream()))
    return out


def _qkv_dtype(*ts):
    import torch
    dts = {t.dtype for t in ts}
    if len(dts) != 1 or dts.pop() not in (torch.bfloat16, torch.float32):
        raise TypeError("tensors must all be bfloat16 or all float32")
    return VL_BF16 if ts[0].dtype == torch.bfloat16 else VL_F32


def sp_qkv_seq2head(q, k, v, sp_degree: int, out=None):
    """Pack q [n,Hq,d], k/v [n,Hkv,d] for the Ulysses exchange in one launch.

    Returns (yq [P,n,Hq/P,d], yk, yv [P,n,hk,d]) with hk = Hkv/P, or 1 with each
    kv head replicated to the P/Hkv ranks that read it when Hkv < P."""
    import torch
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [n, Hq, d] and k, v [n, Hkv, d]")
    n, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != n or k.shape[2] != d:
        raise ValueError("k and v must be [n, Hkv, d] with q's n and d")
    if sp_degree <= 0 or hq % sp_degree:
        raise ValueError("sp_degree must divide n_heads_q")
    hk = hkv // sp_degree if hkv >= sp_degree else 1
    if out is None:
        out = (torch.empty((sp_degree, n, hq // sp_degree, d), dtype=q.dtype, device=q.device),
               torch.empty((sp_degree, n, hk, d), dtype=q.dtype, device=q.device),
               torch.empty((sp_degree, n, hk, d), dtype=q.dtype, device=q.device))
    dt = _qkv_dtype(q, k, v, *out)
    _want(out[0], "out[0]", (sp_degree, n, hq // sp_degree, d), (q.dtype,), q.device)
    _want(out[1], "out[1]", (sp_degree, n, hk, d), (q.dtype,), q.device)
    _want(out[2], "out[2]", (sp_degree, n, hk, d), (q.dtype,), q.device)
    for name, t in (("k", k), ("v", v)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    _check(lib().sp_qkv_seq2head(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), *map(_dev_ptr, out), n, hq,
                                 hkv, d, sp_degree, dt, _stream()))
    return out


def sp_qkv_head2seq(yq, yk, yv, n_heads_kv: int, out=None):
    """Unpack (dq, dk, dv) after the gradient exchange in one launch; the
    adjoint of sp_qkv_seq2head (replicated kv heads are summed in fp32)."""
    import torch
    if yq.dim() != 4:
        raise ValueError("yq must be [P, n, Hq/P, d]")
    P, n, hq, d = yq.shape
    if n_heads_kv <= 0:
        raise ValueError("n_heads_kv must be positive")
    hk = n_heads_kv // P if n_heads_kv >= P else 1
    _want(yk, "yk", (P, n, hk, d), (yq.dtype,), yq.device)
    _want(yv, "yv", (P, n, hk, d), (yq.dtype,), yq.device)
    if out is None:
        out = (torch.empty((n, P * hq, d), dtype=yq.dtype, device=yq.device),
               torch.empty((n, n_heads_kv, d), dtype=yq.dtype, device=yq.device),
               torch.empty((n, n_heads_kv, d), dtype=yq.dtype, device=yq.device))
    dt = _qkv_dtype(yq, yk, yv, *out)
    _want(out[0], "out[0]", (n, P * hq, d), (yq.dtype,), yq.device)
    _want(out[1], "out[1]", (n, n_heads_kv, d), (yq.dtype,), yq.device)
    _want(out[2], "out[2]", (n, n_heads_kv, d), (yq.dtype,), yq.device)
    _check(lib().sp_qkv_head2seq(_dev_ptr(yq), _dev_ptr(yk), _dev_ptr(yv), *map(_dev_ptr, out), n,
                                 P * hq, n_heads_kv, d, P, dt, _stream()))
    return out


def basp_shard(rank: int, world: int, batch: int, seq_len: int) -> dict:
    """Host-only: the batch-aware group and token shard of ``rank``."""
    i32 = [ctypes.c_int32(0) for _ in range(4)]
    i64 = [ctypes.c_int64(0) for _ in range(2)]
    _check(lib().basp_shard(rank, world, batch, seq_len, *map(ctypes.byref, i32),
                            *map(ctypes.byref, i64)))
    g, k, s0, s1 = (x.value for x in i32)
    return {"group": g, "group_size": k, "seq_begin": s0, "seq_end": s1,
            "tok_begin": i64[0].value, "tok_end": i64[1].value}


@dataclass
class CostModel:
    """Inputs of the NSP planner's per-GPU cost model (``vl_cost_model`` in
    include/varlen.h).  bytes_per_token: fwd prologue, fwd epilogue, bwd
    prologue, bwd epilogue."""
    curve_len: Sequence[float]
    fwd_tflops: Sequence[float]
    bwd_tflops: Sequence[float]
    fwd_flops_per_pair: float
    bwd_flops_per_pair: float
    bytes_per_token: Sequence[float]
    a2a_gbs: float
    a2a_alpha_us: float
    dense_fwd_flops_per_token: float = 0.0
    dense_bwd_flops_per_token: float = 0.0
    dense_tflops: float = 1.0

    def _c(self):
        arrs = [np.ascontiguousarray(np.asarray(a, dtype=np.float64))
                for a in (self.curve_len, self.fwd_tflops, self.bwd_tflops)]
        if not (len(arrs[0]) == len(arrs[1]) == len(arrs[2])):
            raise ValueError("curve arrays must have the same length")
        pd = ctypes.POINTER(ctypes.c_double)
        c = _CostModelC(len(arrs[0]), *(a.ctypes.data_as(pd) for a in arrs),
                        float(self.fwd_flops_per_pair), float(self.bwd_flops_per_pair),
                        (ctypes.c_double * 4)(*map(float, self.bytes_per_token)),
                        float(self.a2a_gbs), float(self.a2a_alpha_us),
                        float(self.dense_fwd_flops_per_token),
                        float(self.dense_bwd_flops_per_token), float(self.dense_tflops))
        return c, arrs   # keep the arrays alive while the struct is in use


CURVE_PATH = os.path.join(_HERE, "attn_curve_mi355x.json")


def ulysses_cost_model(n_heads_q: int, n_heads_kv: int, head_dim: int, sp_max: int,
                       curve: Optional[dict] = None, a2a_gbs: float = 7 * 153.0,
                       a2a_alpha_us: float = 10.0, elem_bytes: int = 2,
                       dense_fwd_flops_per_token: float = 0.0,
                       dense_bwd_flops_per_token: float = 0.0,
                       dense_tflops: float = 1000.0) -> CostModel:
    """Cost model of Ulysses attention with this library's kernels.

    Useful FLOPs per visible pair: 4 d Hq forward, 10 d Hq backward.  Exchanged
    bytes per token: forward prologue Q, K, V (kv heads counted once per rank
    that reads them: max(Hkv, sp_max) when Hkv < sp_max), forward epilogue O,
    backward prologue dO, backward epilogue dQ, dK, dV.  The throughput curve is
    the measured one shipped with the library (``attn_curve_mi355x.json``,
    written by ``measure_curve.py``) unless one is given; the all-to-all
    defaults are an MI355X node's 7 xGMI links of about 153 GB/s each."""
    import json
    if curve is None:
        with open(CURVE_PATH) as fh:
            curve = json.load(fh)
    kv = max(n_heads_kv, sp_max) if n_heads_kv < sp_max else n_heads_kv
    row = head_dim * elem_bytes
    return CostModel(curve["len"], curve["fwd_tflops"], curve["bwd_tflops"],
                     4.0 * head_dim * n_heads_q, 10.0 * head_dim * n_heads_q,
                     ((n_heads_q + 2 * kv) * row, n_heads_q * row, n_heads_q * row,
                      (n_heads_q + 2 * kv) * row),
                     a2a_gbs, a2a_alpha_us, dense_fwd_flops_per_token, dense_bwd_flops_per_token,
                     dense_tflops)


def _lengths(lengths) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(lengths, dtype=np.int64).reshape(-1))


def nsp_route(lengths, n_gpus: int, sp_max: int, cost: CostModel, token_budget: float,
              prefix: int = 8, beam: int = 16, monotone: bool = False, level_mask: int = -1) -> dict:
    """Host-only: NSP routing of a batch onto the SP tree.  Returns the node
    (depth, index) of each sample, per-GPU stage times, token loads, the load
    proxy max fwd + max bwd and whether the token budget holds."""
    L = _lengths(lengths)
    n = len(L)
    depth, index = np.zeros(max(n, 1), np.int32), np.zeros(max(n, 1), np.int32)
    f, b, t = (np.zeros(n_gpus, np.float64) for _ in range(3))
    ok = ctypes.c_int32(0)
    c, keep = cost._c()
    pd = ctypes.POINTER(ctypes.c_double)
    _check(lib().nsp_route(L.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, n_gpus, sp_max,
                           ctypes.byref(c), float(token_budget), prefix, beam, int(monotone),
                           level_mask, _iptr(depth), _iptr(index), f.ctypes.data_as(pd),
                           b.ctypes.data_as(pd), t.ctypes.data_as(pd), ctypes.byref(ok)))
    return {"plan": [(int(depth[j]), int(index[j])) for j in range(n)], "gpu_fwd": f,
            "gpu_bwd": b, "gpu_cost": f + b, "gpu_tokens": t,
            "load": float(f.max() + b.max()) if n_gpus else 0.0, "within_budget": bool(ok.value)}


def nsp_plan_cost(lengths, plan, n_gpus: int, sp_max: int, cost: CostModel) -> dict:
    """Host-only: per-GPU stage times and token loads of a given plan."""
    L = _lengths(lengths)
    n = len(L)
    depth = np.ascontiguousarray(np.array([d for d, _ in plan] or [0], np.int32))
    index = np.ascontiguousarray(np.array([i for _, i in plan] or [0], np.int32))
    f, b, t = (np.zeros(n_gpus, np.float64) for _ in range(3))
    c, keep = cost._c()
    pd = ctypes.POINTER(ctypes.c_double)
    _check(lib().nsp_plan_cost(L.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, n_gpus,
                               sp_max, ctypes.byref(c), _iptr(depth), _iptr(index),
                               f.ctypes.data_as(pd), b.ctypes.data_as(pd), t.ctypes.data_as(pd)))
    return {"gpu_fwd": f, "gpu_bwd": b, "gpu_cost": f + b, "gpu_tokens": t,
            "load": float(f.max() + b.max())}


def varlen_mfma_probe(iters: int = 4096, n_workgroups: int = 8192, sink=None) -> int:
    """Enqueue the matrix-core throughput probe on the current stream; returns
    its FLOPs (time it with events around the call)."""
    import torch
    if sink is None:
        sink = torch.empty(n_workgroups, dtype=torch.float32, device="cuda")
    f = ctypes.c_int64(0)
    _check(lib().varlen_mfma_probe(iters, n_workgroups, _dev_ptr(sink), ctypes.byref(f), _stream()))
    return int(f.value)


def varlen_schedule_export(cu_q, cu_k, causal: bool, pass_: int, head_dim: int) -> dict:
    """Host-only: the work list and pair counts the kernels use (no GPU needed)."""
    cq, ck = _cu_host(cu_q), _cu_host(cu_k)
    n = ctypes.c_int64(0)
    useful, issued = ctypes.c_int64(0), ctypes.c_int64(0)
    bq, bk = ctypes.c_int32(0), ctypes.c_int32(0)
    L = lib()
    _check(L.varlen_schedule_export(_iptr(cq), _iptr(ck), len(cq) - 1, int(causal), pass_,
                                    head_dim, None, 0, ctypes.byref(n), None, None, None, None))
    items = np.zeros((max(n.value, 1), 4), dtype=np.int32)
    _check(L.varlen_schedule_export(_iptr(cq), _iptr(ck), len(cq) - 1, int(causal), pass_,
                                    head_dim, _iptr(items), n.value, ctypes.byref(n),
                                    ctypes.byref(useful), ctypes.byref(issued), ctypes.byref(bq),
                                    ctypes.byref(bk)))
    return {"items": items[:n.value], "useful_pairs": useful.value, "issued_pairs": issued.value,
            "bq": bq.value, "bk": bk.value}


def varlen_schedule_export_dkdv(cu_q, cu_k, causal: bool, n_heads_q: int, n_heads_kv: int,
                                n_cu: int) -> np.ndarray:
    """Host-only: the dK/dV work list with its q-head split, rows (doc, kv_tile,
    first, count, slice, n_slices) in launch order (no GPU needed)."""
    cq, ck = _cu_host(cu_q), _cu_host(cu_k)
    n = ctypes.c_int64(0)
    L = lib()
    args = (_iptr(cq), _iptr(ck), len(cq) - 1, int(causal), n_heads_q, n_heads_kv, n_cu)
    _check(L.varlen_schedule_export_dkdv(*args, None, 0, ctypes.byref(n)))
    out = np.zeros((max(n.value, 1), 6), dtype=np.int32)
    _check(L.varlen_schedule_export_dkdv(*args, _iptr(out), n.value, ctypes.byref(n)))
    return out[:n.value]


def varlen_ring_block(cu, q_range, k_range):
    """Host-only: the attention call of one (query chunk, key chunk) block of
    ring attention over a packed causal batch -> (cu_q, cu_k, causal, cls),
    cls one of RING_CLASSES ("N": no call needed)."""
    c = _cu_host(cu)
    n = len(c) - 1
    cq = np.zeros(n + 1, dtype=np.int32)
    ck = np.zeros(n + 1, dtype=np.int32)
    causal, cls = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().varlen_ring_block(_iptr(c), n, int(q_range[0]), int(q_range[1]), int(k_range[0]),
                                   int(k_range[1]), _iptr(cq), _iptr(ck), ctypes.byref(causal),
                                   ctypes.byref(cls)))
    return cq, ck, bool(causal.value), RING_CLASSES[cls.value]


def profile_enable(on: bool = True):
    """Start (clearing earlier records) or stop per-kernel HIP-event timing."""
    _check(lib().varlen_profile_enable(int(on)))


def profile_read() -> dict:
    """{kernel name: (launches, total ms)} of the records since profile_enable(True)."""
    out, i = {}, 0
    buf = ctypes.create_string_buffer(128)
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    while lib().varlen_profile_read(i, buf, 128, ctypes.byref(n), ctypes.byref(ms)) == 0:
        out[buf.value.decode()] = (int(n.value), float(ms.value))
        i += 1
    return out


def cache_clear():
    lib().varlen_cache_clear()


def set_plan_cache(on: bool) -> bool:
    """Switch the per-pattern work-list cache (default off); returns the
    previous setting.  Off: every call schedules its cu_seqlens and enqueues
    the upload of its work lists on its stream.  On: a pattern's lists are
    uploaded once and reused (needed for HIP graph capture)."""
    return bool(lib().varlen_set_plan_cache(1 if on else 0))


def version() -> int:
    return int(lib().varlen_version())
