"""Shared helpers of the GPU parity tests (no tests here)."""
import sys

import numpy as np
import pytest
import torch

import variable_length_sequence_amd as vl
import workloads

# gates (O and the gradients from the workload definition; LSE chosen here,
# since it feeds the merge and the backward)
O_MAX_ABS = 2e-2
LSE_MAX_ABS = 2e-3
GRAD_REL_FRO = 5e-2


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X (torch.cuda.is_available() is False)")
    vl.lib()  # raises if libvarlen.so is missing
    return torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def f64(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def max_abs(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def lse_err(gpu, ref) -> float:
    """Max |err| over finite entries; the -inf pattern must match exactly."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), "-inf pattern differs"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(gpu[fin]))
    return max_abs(gpu[fin], ref[fin]) if fin.any() else 0.0


def random_case(rng, n_docs, lo, hi, hq, hkv, d, ragged_k=False, seed=0, q_scale=1.0):
    lq = workloads.random_lengths(rng, n_docs, lo, hi)
    lk = workloads.random_lengths(rng, n_docs, lo, hi) if ragged_k else list(lq)
    w = workloads.Workload("rand", lq, hq=hq, hkv=hkv, d=d, seed=seed, q_scale=q_scale)
    q, k, v, do = workloads.make_tensors(w, tq=sum(lq), tk=sum(lk))
    return lq, lk, q, k, v, do
