"""Measure this library's attention throughput per document length on the GPU
and write the curve the NSP planner's cost model reads
(``attn_curve_mi355x.json`` beside this file).

For each length L the batch packs max(1, tokens // L) causal documents of
length L (so short documents are measured the way a packed batch runs them)
with n_heads_q / n_heads_kv / head_dim heads; the forward and the backward are
timed separately with events on the current stream and reported as useful
TFLOP/s (4 d Hq and 10 d Hq FLOPs per visible pair).

    python -m variable_length_sequence_amd.measure_curve [--out PATH]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

LENGTHS = [128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072]


def measure(hq=32, hkv=4, d=128, tokens=65536, reps=5, lengths=LENGTHS):
    import torch
    import variable_length_sequence_amd as vl
    if not torch.cuda.is_available():
        raise RuntimeError("measuring the curve needs the GPU")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    out = {"len": [], "fwd_tflops": [], "bwd_tflops": [], "docs": [],
           "heads_q": hq, "heads_kv": hkv, "head_dim": d, "tokens_per_batch": tokens}
    for L in lengths:
        n = max(1, tokens // L)
        T = n * L
        cu = [i * L for i in range(n + 1)]
        q = torch.randn(T, hq, d, generator=g, device=dev).to(torch.bfloat16)
        k = torch.randn(T, hkv, d, generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn(T, hkv, d, generator=g, device=dev).to(torch.bfloat16)
        do = torch.randn(T, hq, d, generator=g, device=dev).to(torch.bfloat16)
        ws = torch.empty(vl.bwd_workspace_bytes(T, T, hq, hkv, d), dtype=torch.uint8, device=dev)
        pairs = n * L * (L + 1) // 2
        tf, tb = [], []
        for r in range(reps + 1):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            o, lse = vl.varlen_attn_fwd(q, k, v, cu, cu, causal=True)
            e[1].record()
            vl.varlen_attn_bwd(q, k, v, o, do, lse, cu, cu, causal=True, workspace=ws)
            e[2].record()
            torch.cuda.synchronize()
            if r:   # the first pass builds and uploads the work lists
                tf.append(e[0].elapsed_time(e[1]))
                tb.append(e[1].elapsed_time(e[2]))
        mf, mb = sorted(tf)[len(tf) // 2], sorted(tb)[len(tb) // 2]
        out["len"].append(float(L))
        out["docs"].append(n)
        out["fwd_tflops"].append(round(4.0 * d * hq * pairs / (mf * 1e-3) / 1e12, 2))
        out["bwd_tflops"].append(round(10.0 * d * hq * pairs / (mb * 1e-3) / 1e12, 2))
        print(f"L={L:6d} docs={n:4d} fwd {out['fwd_tflops'][-1]:8.2f} TFLOP/s "
              f"bwd {out['bwd_tflops'][-1]:8.2f} TFLOP/s", file=sys.stderr, flush=True)
        del q, k, v, do, ws, o, lse
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                  "attn_curve_mi355x.json"))
    a = ap.parse_args()
    curve = measure()
    with open(a.out, "w") as fh:
        json.dump(curve, fh, indent=1)
    print(a.out)


if __name__ == "__main__":
    main()
