#!/usr/bin/env python3
"""Benchmark of packed variable-length causal attention on one MI355X.

One step = the whole hot path over one synthetic packed batch:
varlen_attn_fwd and varlen_attn_bwd, each validating the cu_seqlens,
scheduling the work lists on the host and uploading them (the plan cache is
off, as for a freshly packed batch every step), then the kernels (forward;
dQ, which also stores D = rowsum(dO*O); dK/dV).  The same steps with cached work lists are
reported beside it.  The
headline workload is the 16384-token long-tail batch (lognormal lengths,
median 512, sigma 1.2, clipped to [64, 8192]; 32 q heads, 4 kv heads,
head_dim 128).  The metric is useful TFLOP/s: 4 d FLOPs per visible
(query, key) pair forward and 10 d backward, times the q heads; masked tiles
and masked elements are not counted.

Prints ONE JSON line.  Besides the headline it carries:
  roofline      the dominant kernel's algorithmic FLOPs per launch over its
                average HIP-event duration, against the bf16 dense MFMA peak;
  kernels       every kernel's launches, average time and roofline fraction;
  cpu_baseline  the fp64 oracle on the host cores for the same batch;
  extra         the other workloads: the Ulysses permute on one GPU's
                [49152, 32, 128] shard, the ring share (8 partial forwards +
                attn_lse_merge), the 384K Ulysses attention share and the
                131072-token Pareto batch per length bucket.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def _args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first copy this many MiB device-to-device (a plain copy of known "
                         "size, to calibrate hardware byte counters against)")
    ap.add_argument("--copy-kernels", action="store_true",
                    help="run only the bandwidth-bound kernels (Ulysses permutes, fused Q/K/V "
                         "pack, merge) and print their table (for hardware counter passes)")
    return ap.parse_args()


def useful(vl, cu_q, cu_k, causal, hq, d):
    pairs = vl.varlen_schedule_export(cu_q, cu_k, causal, 0, d)["useful_pairs"]
    return pairs, 4 * d * pairs * hq, 10 * d * pairs * hq


class Timer:
    """Wall clock plus HIP events on the current stream, bracketed by synchronize."""

    def __init__(self, torch):
        self.torch = torch

    def __enter__(self):
        t = self.torch
        t.cuda.synchronize()
        self.e0 = t.cuda.Event(enable_timing=True)
        self.e1 = t.cuda.Event(enable_timing=True)
        self.w0 = time.perf_counter()
        self.e0.record()
        return self

    def __exit__(self, *exc):
        self.e1.record()
        self.torch.cuda.synchronize()
        self.wall_ms = (time.perf_counter() - self.w0) * 1e3
        self.event_ms = self.e0.elapsed_time(self.e1)


def kernel_table(prof, flops, bytes_):
    out = {}
    for name, (n, ms) in prof.items():
        avg = ms / max(n, 1)
        rec = {"launches": n, "avg_ms": round(avg, 5)}
        if name in flops:
            tf = flops[name] / (avg * 1e-3) / 1e12
            rec.update(bound="mfma", achieved_tflops=round(tf, 2),
                       frac=round(tf / PEAK_BF16_TFLOPS, 4))
        elif name in bytes_:
            gbs = bytes_[name] / (avg * 1e-3) / 1e9
            rec.update(bound="hbm", achieved_gbs=round(gbs, 1), frac=round(gbs / PEAK_HBM_GBS, 4))
        out[name] = rec
    return out


def attn_step_fn(vl, torch, w, q, k, v, do, cu):
    ws = torch.empty(vl.bwd_workspace_bytes_cu(cu, cu, w.hq, w.hkv, w.d),
                     dtype=torch.uint8, device=q.device)

    def step():
        o, lse = vl.varlen_attn_fwd(q, k, v, cu, cu, causal=True)
        vl.varlen_attn_bwd(q, k, v, o, do, lse, cu, cu, causal=True, workspace=ws)
    return step


def bench_attention(vl, torch, w, steps, warmup, dev, tensors=None, profile=True,
                    plan_cache=False):
    """Times fwd+bwd steps.  With plan_cache False (the default) every call
    validates and schedules its cu_seqlens again and uploads the work lists,
    as a step over a freshly packed batch would."""
    import workloads
    q, k, v, do = tensors if tensors is not None else workloads.make_tensors(w)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    cu = w.cu
    step = attn_step_fn(vl, torch, w, q, k, v, do, cu)
    prev = vl.set_plan_cache(plan_cache)
    try:
        for _ in range(warmup):
            step()
        if profile:
            vl.profile_enable(True)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        with Timer(torch) as tm:
            ev[0].record()
            for i in range(steps):
                step()
                ev[i + 1].record()
    finally:
        vl.set_plan_cache(prev)
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    prof = vl.profile_read() if profile else {}
    if profile:
        vl.profile_enable(False)
    pairs, ffwd, fbwd = useful(vl, cu, cu, True, w.hq, w.d)
    ms = tm.wall_ms / steps
    del q, k, v, do
    return dict(ms=ms, event_ms=tm.event_ms / steps, pairs=pairs, flops_fwd=ffwd, flops_bwd=fbwd,
                tflops=(ffwd + fbwd) / (ms * 1e-3) / 1e12, prof=prof,
                median_ms=per_step[len(per_step) // 2], min_ms=per_step[0])


# kernel -> the sources its code comes from (a counter summary is valid only for
# the sources it was taken with)
KERNEL_SOURCES = {   # relative to csrc/; the build script holds the compile flags
    "attn_fwd": ["attn_fwd.hip", "common.h", "launch.h", "../build.py"],
    "bwd_dkdv": ["attn_bwd.hip", "common.h", "launch.h", "../build.py"],
    "bwd_dq": ["attn_bwd.hip", "common.h", "launch.h", "../build.py"],
}


def sources_sha256(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "variable_length_sequence_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("sources_sha256") != sources_sha256(kernel):
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attn_kernel_flops(pairs, hq, d):
    # algorithmic FLOPs each kernel must do per launch (per visible pair):
    # forward QK^T and PV; dK/dV kernel S, dP, dV, dK; dQ kernel only dQ
    # (its S and dP recompute is overhead of the split design)
    return {"attn_fwd": 4 * d * pairs * hq, "bwd_dkdv": 8 * d * pairs * hq,
            "bwd_dq": 2 * d * pairs * hq}


def cpu_baseline(w):
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    q, k, v, do = workloads.make_tensors(w)
    f = lambda t: t.float().numpy()
    qn, kn, vn, don = f(q), f(k), f(v), f(do)
    cu = w.cu
    t0 = time.perf_counter()
    oracle.attn_bwd(qn, kn, vn, don, cu, cu, causal=True, return_fwd=True)
    sec = time.perf_counter() - t0
    vis = oracle.schedule.visible_pairs(cu, cu, True)
    flops = 14 * w.d * vis * w.hq
    return {"value": round(flops / sec / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(sec, 2),
            "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "sample": f"full {w.name} batch, fp64 numpy forward + backward "
                      f"(O, LSE, dQ, dK, dV) of all {len(w.lengths)} documents x {w.hq} heads"}


def cpu_sampled_checks(full_rate_tflops):
    """The sampled oracle checks of the large workloads, timed on the host: the
    forward and dQ of 64 sampled query rows per q head (what the GPU parity
    tests compute per row), and the full oracle's time for each workload
    extrapolated from the full-oracle rate measured on the headline batch."""
    import numpy as np
    import oracle
    import workloads
    res = {}
    for wf in (workloads.ulysses_384k, workloads.ring_256k, workloads.mixed_128k):
        w = wf()
        q, k, v, do = workloads.make_tensors(w)
        f = lambda t: t.float().numpy()
        qn, kn, vn, don = f(q), f(k), f(v), f(do)
        del q, k, v, do
        cu = np.asarray(w.cu, np.int64)
        if w.name == "ring_256k":   # query chunk 7 of the sequence
            n, c, qc = w.extra["n_chunks"], w.extra["chunk"], w.extra["q_chunk"]
            base, span = qc * c, c
            pairs_full = 7 * c * c + c * (c + 1) // 2
        else:
            base, span = 0, w.total
            pairs_full = oracle.schedule.visible_pairs(cu, cu, True)
        rows = workloads.sample_rows(span, 64, seed=1) + base
        rows = np.concatenate([rows] * w.hq)
        heads = np.repeat(np.arange(w.hq), 64)
        t0 = time.perf_counter()
        oracle.attn_bwd_dq_rows(qn, kn, vn, don, cu, cu, rows, heads)
        sec = time.perf_counter() - t0
        doc = np.searchsorted(cu, rows, side="right") - 1
        vis = int(np.sum(rows - cu[doc] + 1))   # causal: a row sees its document's keys up to itself
        sflops = 8 * w.d * vis                  # per visible pair: S, PV, dP, dS K
        full_flops = 14 * w.d * pairs_full * w.hq
        res[w.name] = {"value": round(sflops / sec / 1e12, 5), "unit": "TFLOP/s",
                       "kind": "oracle", "seconds": round(sec, 2),
                       "sample": f"forward and dQ of 64 sampled query rows x {w.hq} q heads"
                                 + (" of query chunk 7" if w.name == "ring_256k" else ""),
                       "full_oracle_seconds_extrapolated": round(full_flops / (full_rate_tflops * 1e12), 1),
                       "extrapolated_from": "the full-oracle TFLOP/s of the longtail_16k batch in this run"}
        del qn, kn, vn, don
    return res


def measured_gemm_peak(torch, dev, n=8192, reps=20):
    """bf16 GEMM throughput of the vendor library (hipBLASLt via torch.matmul) on
    one n x n x n product: a measured stand-in for the reachable MFMA peak."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    with Timer(torch) as tm:
        for _ in range(reps):
            torch.matmul(a, b)
    del a, b
    return round(2 * n ** 3 * reps / (tm.event_ms * 1e-3) / 1e12, 1)


def measured_mfma_peak(vl, torch, dev, iters=4096, n_wg=8192, reps=3):
    """The library's matrix-core probe: independent MFMA chains with no memory
    traffic on every SIMD; the best of a few launches, in TFLOP/s."""
    sink = torch.empty(n_wg, dtype=torch.float32, device=dev)
    vl.varlen_mfma_probe(iters, n_wg, sink)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = vl.varlen_mfma_probe(iters, n_wg, sink)
        e1.record()
        torch.cuda.synchronize()
        t = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
        best = t if best is None else max(best, t)
    return round(best, 1)


def measured_copy_gbs(torch, dev, nbytes, reps=10):
    """Device-to-device copy of nbytes (read + write counted): the reference for
    the bandwidth-bound kernels."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1)
    dst = [torch.empty_like(src) for _ in range(2)]
    dst[0].copy_(src)
    with Timer(torch) as tm:
        for i in range(reps):
            dst[i % 2].copy_(src)
    del src, dst
    return round(2 * nbytes * reps / (tm.event_ms * 1e-3) / 1e9, 1)


def bench_permute(vl, torch, dev, steps):
    n, H, d, P = 49152, 32, 128, 8
    g = torch.Generator(device=dev).manual_seed(0)
    xs = [torch.randn(n, H, d, generator=g, device=dev).to(torch.bfloat16) for _ in range(2)]
    ys = [torch.empty(P, n, H // P, d, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    for i in range(2):
        vl.sp_seq2head(xs[i], P, out=ys[i])
        vl.sp_head2seq(ys[i], out=xs[i])
    vl.profile_enable(True)
    for i in range(steps):
        vl.sp_seq2head(xs[i % 2], P, out=ys[i % 2])     # alternate buffers: 768 MiB > MALL
        vl.sp_head2seq(ys[(i + 1) % 2], out=xs[(i + 1) % 2])
    prof = vl.profile_read()
    vl.profile_enable(False)
    nbytes = 2 * n * H * d * 2
    return prof, {"sp_seq2head": nbytes, "sp_head2seq": nbytes}


def bench_qkv_permute(vl, torch, dev, steps):
    """Fused Q/K/V pack and gradient unpack of a 384K sequence's shard with
    32 query / 4 kv heads over 8 ranks (each kv head sent to 2 ranks)."""
    n, hq, hkv, d, P = 49152, 32, 4, 128, 8
    g = torch.Generator(device=dev).manual_seed(0)
    bf = torch.bfloat16

    def xset():
        return [torch.randn(n, h, d, generator=g, device=dev).to(bf) for h in (hq, hkv, hkv)]

    def yset():
        return [torch.randn(P, n, h, d, generator=g, device=dev).to(bf) for h in (hq // P, 1, 1)]

    xs, ys = [xset(), xset()], [yset(), yset()]
    for i in range(2):
        vl.sp_qkv_seq2head(*xs[i], P, out=ys[i])
        vl.sp_qkv_head2seq(*ys[i], hkv, out=xs[i])
    vl.profile_enable(True)
    for i in range(steps):
        vl.sp_qkv_seq2head(*xs[i % 2], P, out=ys[i % 2])     # alternate buffers: > MALL
        vl.sp_qkv_head2seq(*ys[(i + 1) % 2], hkv, out=xs[(i + 1) % 2])
    prof = vl.profile_read()
    vl.profile_enable(False)
    nbytes = sum(t.numel() * 2 for t in xs[0]) + sum(t.numel() * 2 for t in ys[0])
    del xs, ys
    return prof, {"sp_qkv_seq2head": nbytes, "sp_qkv_head2seq": nbytes}


def bench_router(vl, reps=20):
    """Host-only: NSP routing of the Pareto batch onto a 64-GPU SP tree with
    the cost model fed by this library's measured throughput curve."""
    import workloads
    w = workloads.mixed_128k()
    P = 64
    cm = vl.ulysses_cost_model(w.hq, w.hkv, w.d, sp_max=P)
    budget = 2.0 * sum(w.lengths) / P
    t0 = time.perf_counter()
    for _ in range(reps):
        r = vl.nsp_route(w.lengths, P, P, cm, budget, 8, 16, True)
    us = (time.perf_counter() - t0) / reps * 1e6
    static = vl.nsp_plan_cost(w.lengths, [(0, 0)] * len(w.lengths), P, P, cm)
    leaves = vl.nsp_route(w.lengths, P, P, cm, budget, 0, 1)
    degs = sorted({P >> d for d, _ in r["plan"]}, reverse=True)
    return {"samples": len(w.lengths), "gpus": P, "prefix": 8, "beam": 16, "monotone": True,
            "us_per_plan": round(us, 1), "load_ms": round(r["load"] * 1e3, 4),
            "static_sp64_load_ms": round(static["load"] * 1e3, 4),
            "leaves_only_load_ms": round(leaves["load"] * 1e3, 4), "sp_degrees_used": degs,
            "within_budget": r["within_budget"]}


def bench_merge(vl, torch, dev, steps):
    """attn_lse_merge of 8 fp32 partials [32768, 8, 128] (the ring share's
    merge) into bf16, alternating two input sets."""
    n, H, d, P = 32768, 8, 128, 8
    g = torch.Generator(device=dev).manual_seed(0)
    parts = [[torch.randn(n, H, d, generator=g, device=dev) for _ in range(P)] for _ in range(2)]
    lses = [[torch.randn(H, n, generator=g, device=dev) for _ in range(P)] for _ in range(2)]
    for i in range(2):
        vl.attn_lse_merge(parts[i], lses[i])
    vl.profile_enable(True)
    for i in range(steps):
        vl.attn_lse_merge(parts[i % 2], lses[i % 2])
    prof = vl.profile_read()
    vl.profile_enable(False)
    nbytes = P * (n * H * d * 4 + H * n * 4) + n * H * d * 2 + H * n * 4
    del parts, lses
    return prof, {"lse_merge": nbytes}


def bench_ring(vl, torch, dev, steps):
    import numpy as np
    import workloads
    w = workloads.ring_256k()
    n, c, qc = w.extra["n_chunks"], w.extra["chunk"], w.extra["q_chunk"]
    q, k, v, do = workloads.make_tensors(w)
    qd = q[qc * c:(qc + 1) * c].contiguous().to(dev)
    dod = do[qc * c:(qc + 1) * c].contiguous().to(dev)
    kd, vd = k.to(dev), v.to(dev)
    del q, k, v, do
    one = np.array([0, c], np.int32)
    parts_o = [torch.empty(c, w.hq, w.d, dtype=torch.float32, device=dev) for _ in range(n)]
    parts_l = [torch.empty(w.hq, c, dtype=torch.float32, device=dev) for _ in range(n)]

    def step():
        for j in range(n):
            vl.varlen_attn_fwd(qd, kd[j * c:(j + 1) * c], vd[j * c:(j + 1) * c], one, one,
                               causal=(j == qc), out=parts_o[j], lse=parts_l[j])
        return vl.attn_lse_merge(parts_o, parts_l, out_dtype=torch.bfloat16)
    step()
    vl.profile_enable(True)
    with Timer(torch) as tm:
        for _ in range(steps):
            step()
    prof = vl.profile_read()
    vl.profile_enable(False)
    pairs = 7 * c * c + c * (c + 1) // 2
    flops = 4 * w.d * pairs * w.hq
    merge_bytes = n * (c * w.hq * w.d * 4 + c * w.hq * 4) + c * w.hq * w.d * 2 + c * w.hq * 4
    ms = tm.wall_ms / steps

    # the same share with the merge folded into the forward's epilogue
    o_acc = torch.empty(c, w.hq, w.d, dtype=torch.float32, device=dev)
    lse_acc = torch.empty(w.hq, c, dtype=torch.float32, device=dev)

    def step_acc():
        o_acc.zero_()
        lse_acc.fill_(float("-inf"))
        for j in range(n):
            vl.varlen_attn_fwd_acc(qd, kd[j * c:(j + 1) * c], vd[j * c:(j + 1) * c], one, one,
                                   o_acc, lse_acc, causal=(j == qc))
    step_acc()
    with Timer(torch) as tm2:
        for _ in range(steps):
            step_acc()
    ms2 = tm2.wall_ms / steps

    # the blockwise backward of the share: block j's backward with the merged
    # O and LSE gives its share of dQ (summed in fp32) and chunk j's dK, dV
    om, lm = step()
    dq = torch.empty(c, w.hq, w.d, dtype=torch.float32, device=dev)
    dk, dv = torch.empty_like(kd), torch.empty_like(vd)
    dq_j = torch.empty_like(qd)
    ws = torch.empty(max(vl.bwd_workspace_bytes_cu(one, one, w.hq, w.hkv, w.d, c), 256),
                     dtype=torch.uint8, device=dev)

    def step_bwd():
        dq.zero_()
        for j in range(n):
            vl.varlen_attn_bwd(qd, kd[j * c:(j + 1) * c], vd[j * c:(j + 1) * c], om, dod, lm, one,
                               one, causal=(j == qc), workspace=ws, dq=dq_j,
                               dk=dk[j * c:(j + 1) * c], dv=dv[j * c:(j + 1) * c])
            dq.add_(dq_j)
    step_bwd()
    vl.profile_enable(True)
    with Timer(torch) as tm3:
        for _ in range(steps):
            step_bwd()
    prof3 = vl.profile_read()
    vl.profile_enable(False)
    ms3 = tm3.wall_ms / steps
    bflops = 10 * w.d * pairs * w.hq
    return {"workload": w.name, "ms_per_step": round(ms, 3),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "useful_tflop": round(flops / 1e12, 3),
            "kernels": kernel_table(prof, {}, {"lse_merge": merge_bytes}),
            "attn_fwd_avg_ms": round(prof["attn_fwd"][1] / prof["attn_fwd"][0], 4),
            "fused_merge": {"ms_per_step": round(ms2, 3),
                            "tflops": round(flops / (ms2 * 1e-3) / 1e12, 2)},
            "backward": {"what": "8 block backwards with the merged O/LSE (dQ summed in fp32)",
                         "ms_per_step": round(ms3, 3),
                         "tflops": round(bflops / (ms3 * 1e-3) / 1e12, 2),
                         "useful_tflop": round(bflops / 1e12, 3),
                         "kernels": kernel_table(prof3, {}, {})},
            "fwd_merge_bwd": {"ms_per_step": round(ms + ms3, 3),
                              "tflops": round((flops + bflops) / ((ms + ms3) * 1e-3) / 1e12, 2)}}


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {a.gpus} is not supported "
              "(this build runs on one GPU and has no collectives)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import variable_length_sequence_amd as vl
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    vl.lib()
    # every timed attention call schedules its own work lists (see bench_attention)
    vl.set_plan_cache(False)
    dev = torch.device("cuda:0")
    if a.copy_mib > 0:
        n = a.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if a.copy_kernels:
        tabs = {}
        for name, fn in (("ulysses_permute_49152x32x128_P8", bench_permute),
                         ("ulysses_qkv_permute_49152_q32_kv4_d128_P8", bench_qkv_permute),
                         ("lse_merge_8x32768x8x128_f32", bench_merge)):
            prof, by = fn(vl, torch, dev, 10)
            tabs[name] = kernel_table(prof, {}, by)
        print(json.dumps({"copy_kernels": tabs}))
        return
    w = workloads.longtail_16k()
    print(f"[bench] {w.name}: {len(w.lengths)} docs, {w.total} tokens, "
          f"{a.warmup} warmup + {a.steps} timed steps", file=sys.stderr, flush=True)
    # the headline: no timing events inside the step
    r = bench_attention(vl, torch, w, a.steps, a.warmup, dev, profile=False)
    # the same steps again with every kernel bracketed by HIP events on its
    # launch stream: the per-kernel table and the roofline
    rp = bench_attention(vl, torch, w, a.steps, a.warmup, dev, profile=True)
    kflops = attn_kernel_flops(r["pairs"], w.hq, w.d)
    ktab = kernel_table(rp["prof"], kflops, {})
    dom = max((n for n in kflops if n in rp["prof"]), key=lambda n: rp["prof"][n][1])
    dom_avg = rp["prof"][dom][1] / rp["prof"][dom][0]
    achieved = kflops[dom] / (dom_avg * 1e-3) / 1e12
    cached = bench_attention(vl, torch, w, a.steps, a.warmup, dev, profile=False, plan_cache=True)
    print("[bench] matrix-core probe", file=sys.stderr, flush=True)
    probe = measured_mfma_peak(vl, torch, dev)
    out = {
        "metric": "packed varlen causal attn fwd+bwd TFLOP/s (useful FLOPs) on 1 MI355X; % MFMA peak",
        "value": round(r["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.total, "docs": len(w.lengths),
                   "max_doc": max(w.lengths), "n_heads_q": w.hq, "n_heads_kv": w.hkv,
                   "head_dim": w.d, "causal": True, "length_seed": 0,
                   "lengths": "lognormal(median 512, sigma 1.2) clipped [64, 8192]"},
        "pct_mfma_peak": round(100 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
        "measured_mfma_probe_tflops": probe,
        "pct_measured_mfma_peak": round(100 * r["tflops"] / probe, 2),
        "step_ms_median": round(r["median_ms"], 4),
        "step_ms_min": round(r["min_ms"], 4),
        "work_lists": "scheduled and uploaded by every call (plan cache off)",
        "ms_per_step_plan_cached": round(cached["ms"], 4),
        "useful_tflop_per_step": round((r["flops_fwd"] + r["flops_bwd"]) / 1e12, 4),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom, w.name),
                     "flops_per_launch": kflops[dom], "avg_launch_ms": round(dom_avg, 5),
                     "frac_of_measured_mfma_peak": round(achieved / probe, 4)},
        "kernels": ktab,
    }
    print(f"[bench] headline {out['value']} TFLOP/s, {out['ms_per_step']} ms/step", file=sys.stderr,
          flush=True)
    if not a.no_extra:
        extra = {}
        print("[bench] permute", file=sys.stderr, flush=True)
        prof, by = bench_permute(vl, torch, dev, 10)
        perm = kernel_table(prof, {}, by)
        perm["device_copy_same_bytes_gbs"] = measured_copy_gbs(torch, dev, by["sp_seq2head"] // 2)
        extra["ulysses_permute_49152x32x128_P8"] = perm
        print("[bench] qkv permute", file=sys.stderr, flush=True)
        prof, by = bench_qkv_permute(vl, torch, dev, 10)
        extra["ulysses_qkv_permute_49152_q32_kv4_d128_P8"] = kernel_table(prof, {}, by)
        print("[bench] router", file=sys.stderr, flush=True)
        extra["nsp_route_mixed_128k_64gpus"] = bench_router(vl)
        print("[bench] measured GEMM peak", file=sys.stderr, flush=True)
        extra["measured_bf16_gemm_tflops"] = measured_gemm_peak(torch, dev)
        print("[bench] ring share", file=sys.stderr, flush=True)
        extra["ring_256k_chunk7"] = bench_ring(vl, torch, dev, 2)
        torch.cuda.empty_cache()
        for wf, steps in ((workloads.ulysses_384k, 2), (workloads.mixed_128k, 3)):
            ww = wf()
            print(f"[bench] {ww.name}", file=sys.stderr, flush=True)
            rr = bench_attention(vl, torch, ww, steps, 1, dev)
            kf = attn_kernel_flops(rr["pairs"], ww.hq, ww.d)
            extra[ww.name] = {"ms_per_step": round(rr["ms"], 3), "tflops": round(rr["tflops"], 2),
                              "pct_mfma_peak": round(100 * rr["tflops"] / PEAK_BF16_TFLOPS, 2),
                              "useful_tflop": round((rr["flops_fwd"] + rr["flops_bwd"]) / 1e12, 3),
                              "kernels": kernel_table(rr["prof"], kf, {})}
            torch.cuda.empty_cache()
        # per length bucket of the Pareto batch: bucket-only packed sub-batches
        mw = workloads.mixed_128k()
        q, k, v, do = workloads.make_tensors(mw)
        cu = mw.cu
        buckets = {}
        for name, idx in workloads.length_buckets(mw.lengths).items():
            if not idx:
                continue
            rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in idx])
            sub = workloads.Workload(f"{mw.name}_{name}", [mw.lengths[i] for i in idx], hq=mw.hq,
                                     hkv=mw.hkv, d=mw.d)
            t = [x[rows].contiguous() for x in (q, k, v, do)]
            # short buckets get the headline's 5 warmup + 20 timed steps (a
            # step of the < 2K bucket is about a millisecond, and the first
            # steps after the long runs above are slower); the > 16K bucket
            # (about 0.2 s a step) keeps 1 + 3
            short = sub.total <= 32768
            rr = bench_attention(vl, torch, sub, 20 if short else 3, 5 if short else 1, dev,
                                 tensors=t, profile=False)
            buckets[name] = {"docs": len(idx), "tokens": sub.total, "ms_per_step": round(rr["ms"], 3),
                             "tflops": round(rr["tflops"], 2),
                             "useful_tflop": round((rr["flops_fwd"] + rr["flops_bwd"]) / 1e12, 3)}
            torch.cuda.empty_cache()
        extra["mixed_128k_buckets"] = buckets
        out["extra"] = extra
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
        if not a.no_extra:
            print("[bench] cpu baseline: sampled oracle checks", file=sys.stderr, flush=True)
            out["cpu_baseline"]["other_workloads"] = cpu_sampled_checks(out["cpu_baseline"]["value"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
