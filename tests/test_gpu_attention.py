"""GPU parity of varlen_attn_fwd / varlen_attn_bwd against the fp64 oracle.

Small and medium packed batches are compared element by element: the tiny
4-document batch, randomised ragged batches (zero-length and one-token
documents, Lq != Lk, non-causal, GQA, head_dim 64 and 128), a seeded sweep
of batch shapes, and the whole
16384-token long-tail batch.  Plus invariants that need no oracle: packing
invariance and re-run determinism (bitwise), single-token documents.
"""
import numpy as np
import pytest
import torch

import oracle
import variable_length_sequence_amd as vl
import workloads
from gpu_helpers import (GRAD_REL_FRO, LSE_MAX_ABS, O_MAX_ABS, f64, lse_err, max_abs,
                         random_case, rel_fro, require_gpu, say)

pytestmark = pytest.mark.gpu


def _run(q, k, v, do, lq, lk, causal, dev, out_dtype=torch.bfloat16, bwd=True):
    cq, ck = workloads.cu_seqlens(lq), workloads.cu_seqlens(lk)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = vl.varlen_attn_fwd(qd, kd, vd, cq, ck, causal=causal, out_dtype=out_dtype)
    res = {"o": o, "lse": lse}
    if bwd:
        ob = o if o.dtype == torch.bfloat16 else o.to(torch.bfloat16)
        dq, dk, dv = vl.varlen_attn_bwd(qd, kd, vd, ob, do.to(dev), lse, cq, ck, causal=causal)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return res


def _compare(res, q, k, v, do, lq, lk, causal, tag, bwd=True):
    cq, ck = workloads.cu_seqlens(lq), workloads.cu_seqlens(lk)
    if bwd:
        dq, dk, dv, o, lse = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), cq, ck,
                                             causal=causal, return_fwd=True)
    else:
        o, lse = oracle.attn_fwd(f64(q), f64(k), f64(v), cq, ck, causal=causal)
    eo = max_abs(f64(res["o"]), o)
    el = lse_err(f64(res["lse"]), lse)
    msg = f"{tag}: O max|err| {eo:.3e}  LSE max|err| {el:.3e}"
    if bwd:
        g = [rel_fro(f64(res[n]), r) for n, r in (("dq", dq), ("dk", dk), ("dv", dv))]
        msg += "  rel-Fro dQ {:.3e} dK {:.3e} dV {:.3e}".format(*g)
    say(msg)
    assert eo <= O_MAX_ABS, msg
    assert el <= LSE_MAX_ABS, msg
    if bwd:
        assert max(g) <= GRAD_REL_FRO, msg


def test_tiny_batch_fwd_bwd():
    dev = require_gpu()
    w = workloads.tiny()
    q, k, v, do = workloads.make_tensors(w)
    res = _run(q, k, v, do, w.lengths, w.lengths, True, dev)
    _compare(res, q, k, v, do, w.lengths, w.lengths, True, "tiny_256")


@pytest.mark.parametrize("seed,n_docs,lo,hi,hq,hkv,d,causal,ragged", [
    (1, 5, 0, 300, 4, 2, 128, True, False),
    (2, 7, 1, 200, 8, 1, 128, True, False),
    (3, 3, 100, 700, 2, 2, 64, True, False),
    (4, 6, 0, 260, 4, 4, 64, False, True),
    (5, 4, 1, 333, 6, 3, 128, False, True),
    (6, 5, 0, 400, 4, 2, 128, True, True),    # Lq != Lk: bottom-right diagonal, empty rows
    (7, 9, 1, 5, 4, 4, 128, True, False),     # many tiny documents
    (8, 2, 600, 1100, 16, 2, 128, True, False),
])
def test_random_batches(seed, n_docs, lo, hi, hq, hkv, d, causal, ragged):
    dev = require_gpu()
    rng = np.random.default_rng(seed)
    lq, lk, q, k, v, do = random_case(rng, n_docs, lo, hi, hq, hkv, d, ragged_k=ragged, seed=seed)
    say(f"case seed={seed} lq={lq} lk={lk} hq={hq} hkv={hkv} d={d} causal={causal}")
    res = _run(q, k, v, do, lq, lk, causal, dev)
    _compare(res, q, k, v, do, lq, lk, causal, f"seed{seed}")


def _sweep_case(seed):
    """Draw one batch shape from the seed: head dim, GQA group (1, 2, 3, 4 or
    8 q heads per kv head), causal or not, equal or ragged key lengths, 1-8
    documents with lengths up to 40, 300 or 1200 tokens."""
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128]))
    grp = int(rng.choice([1, 2, 3, 4, 8]))
    hkv = int(rng.integers(1, 4))
    causal = bool(rng.integers(0, 2))
    ragged = bool(rng.integers(0, 2))
    n_docs = int(rng.integers(1, 9))
    hi = int(rng.choice([40, 300, 1200]))
    lo = int(rng.integers(0, 2))
    return rng, n_docs, lo, hi, grp * hkv, hkv, d, causal, ragged


@pytest.mark.parametrize("seed", range(32))
def test_random_sweep(seed):
    """Seeded sweep over batch shapes (see _sweep_case), full tensors against
    the oracle, forward and backward."""
    dev = require_gpu()
    rng, n_docs, lo, hi, hq, hkv, d, causal, ragged = _sweep_case(seed)
    lq, lk, q, k, v, do = random_case(rng, n_docs, lo, hi, hq, hkv, d, ragged_k=ragged, seed=seed)
    say(f"sweep seed={seed} lq={lq} lk={lk} hq={hq} hkv={hkv} d={d} causal={causal}")
    res = _run(q, k, v, do, lq, lk, causal, dev)
    _compare(res, q, k, v, do, lq, lk, causal, f"sweep{seed}")


@pytest.mark.parametrize("causal,ragged", [(True, False), (False, False), (True, True), (False, True)])
def test_tile_boundary_lengths(causal, ragged):
    """Documents one short of, at and one past the 32-, 64- and 128-row tile
    edges (the forward runs 32-key tiles from lists of 64-key tiles and drops a
    last half no query sees); with ragged key lengths the causal diagonal is
    shifted both ways (Lq < Lk, and Lq > Lk with leading rows that see no
    key).  Full tensors against the oracle."""
    dev = require_gpu()
    lq = [31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 191, 192, 193, 1]
    lk = [l + d for l, d in zip(lq, [0, 1, -31, 32, -33, 64, 3, -50, 97, 2, -64, 31, 1, 0, -63, 40])] \
        if ragged else list(lq)
    w = workloads.Workload("edges", lq, hq=4, hkv=2, d=128, seed=21)
    q, k, v, do = workloads.make_tensors(w, tq=sum(lq), tk=sum(lk))
    say(f"edges lq={lq} lk={lk} causal={causal}")
    res = _run(q, k, v, do, lq, lk, causal, dev)
    _compare(res, q, k, v, do, lq, lk, causal, f"edges_{'causal' if causal else 'full'}{'_ragged' if ragged else ''}")


def test_fp32_output_and_softmax_range():
    dev = require_gpu()
    rng = np.random.default_rng(11)
    lq, lk, q, k, v, do = random_case(rng, 4, 50, 500, 4, 2, 128, seed=11, q_scale=3.0)
    res = _run(q, k, v, do, lq, lk, True, dev, out_dtype=torch.float32, bwd=False)
    assert res["o"].dtype == torch.float32
    _compare(res, q, k, v, do, lq, lk, True, "fp32-out", bwd=False)


@pytest.mark.parametrize("d,hq,hkv,causal", [(64, 8, 2, True), (128, 8, 2, True),
                                              (128, 8, 2, False)])
def test_head_split_batches(d, hq, hkv, causal):
    """One long document among short ones: the dK/dV pass cuts the q-head
    group of the long document's early key tiles into slices (fp32 partials
    summed by the convert kernel) while the other tiles keep theirs whole
    (bf16 written directly), for both head dims; full tensors against the
    oracle."""
    dev = require_gpu()
    lens = [3000, 257, 131, 64, 500, 1]
    cu = workloads.cu_seqlens(lens)
    d_only = (sum(lens) * hq * 4 + 255) // 256 * 256
    assert vl.bwd_workspace_bytes_cu(cu, cu, hq, hkv, d, causal=causal) > d_only   # the split path runs
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    cuts = vl.varlen_schedule_export_dkdv(cu, cu, causal, hq, hkv, n_cu)[:, 5]
    assert (cuts > 1).any() and (cuts == 1).any(), "both kinds of key tile"
    w = workloads.Workload(f"split_d{d}", lens, hq=hq, hkv=hkv, d=d, seed=11)
    q, k, v, do = workloads.make_tensors(w)
    say(f"case lens={lens} hq={hq} hkv={hkv} d={d} causal={causal}")
    res = _run(q, k, v, do, lens, lens, causal, dev)
    _compare(res, q, k, v, do, lens, lens, causal, f"split_d{d}_{'causal' if causal else 'full'}")


def test_longtail_16k_full():
    dev = require_gpu()
    w = workloads.longtail_16k()
    q, k, v, do = workloads.make_tensors(w)
    say(f"longtail_16k: {len(w.lengths)} docs, max {max(w.lengths)}")
    res = _run(q, k, v, do, w.lengths, w.lengths, True, dev)
    _compare(res, q, k, v, do, w.lengths, w.lengths, True, "longtail_16k")


def test_packing_invariance_and_determinism_bitwise():
    dev = require_gpu()
    rng = np.random.default_rng(21)
    lq, lk, q, k, v, do = random_case(rng, 5, 1, 400, 8, 2, 128, seed=21)
    # Every output is bitwise deterministic; O, LSE and dQ are also packing
    # invariant.  dK/dV sum a kv group's q heads, and how the library splits
    # that group over workgroups depends on the whole batch (the partial sums
    # are added in split order), so a document alone matches to tolerance.
    a = _run(q, k, v, do, lq, lk, True, dev)
    b = _run(q, k, v, do, lq, lk, True, dev)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), f"{n} not deterministic"
    cu = workloads.cu_seqlens(lq)
    for i, L in enumerate(lq):
        s, e = int(cu[i]), int(cu[i + 1])
        one = _run(q[s:e].contiguous(), k[s:e].contiguous(), v[s:e].contiguous(),
                   do[s:e].contiguous(), [L], [L], True, dev)
        assert torch.equal(one["o"], a["o"][s:e])
        assert torch.equal(one["lse"], a["lse"][:, s:e])
        assert torch.equal(one["dq"], a["dq"][s:e])
        for n in ("dk", "dv"):
            assert rel_fro(f64(one[n]), f64(a[n][s:e])) < 1e-2, n


def test_single_token_documents_return_v():
    dev = require_gpu()
    lens = [1, 1, 3, 1]
    w = workloads.Workload("ones", lens, hq=4, hkv=2, d=128)
    q, k, v, do = workloads.make_tensors(w)
    res = _run(q, k, v, do, lens, lens, True, dev, bwd=False)
    o = res["o"].cpu()
    for t in (0, 1, 5):
        for h in range(4):
            assert torch.equal(o[t, h], v[t, h // 2])
    lse = f64(res["lse"])
    sc = 1 / np.sqrt(128)
    for t in (0, 1, 5):
        for h in range(4):
            ref = sc * float(f64(q[t, h]) @ f64(k[t, h // 2]))
            assert abs(lse[h, t] - ref) < 1e-4


def test_rows_without_keys_and_empty_documents():
    dev = require_gpu()
    lq, lk = [5, 0, 70, 3], [2, 4, 0, 3]
    w = workloads.Workload("holes", lq, hq=2, hkv=1, d=128)
    q, k, v, do = workloads.make_tensors(w, tq=sum(lq), tk=sum(lk))
    res = _run(q, k, v, do, lq, lk, True, dev)
    o, lse = f64(res["o"]), f64(res["lse"])
    assert np.all(o[:3] == 0) and np.all(np.isneginf(lse[:, :3]))   # rows 0..2 see no key
    assert np.all(o[5:75] == 0) and np.all(np.isneginf(lse[:, 5:75]))  # doc with no keys
    assert np.all(f64(res["dq"])[5:75] == 0)
    assert np.all(f64(res["dk"])[2:6] == 0) and np.all(f64(res["dv"])[2:6] == 0)  # no queries
    _compare(res, q, k, v, do, lq, lk, True, "holes")
