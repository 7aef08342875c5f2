"""Writes ring_256k_chunk7_bwd.npz: the oracle's dK and dV of sampled keys for
the ring share's backward.

The ring share is query chunk 7 of one causal 262144-token sequence cut into
8 chunks of 32768 (8 q heads, 8 kv heads, head_dim 128; seeded synthetic
inputs from ``workloads``).  Ring attention computes that chunk's attention
block by block over the key chunks and merges the partial results (HSAP page,
Section 2.2.1, InterSP ring; Section 3.2, Figure 3).  The backward of block j,
run with the merged O and LSE, gives the part of dK and dV of key chunk j
that comes from the chunk-7 queries.  Summed over the blocks it is the
gradient of attention restricted to those queries: the oracle computes it
as one bottom-right-aligned causal problem of 32768 queries against all
262144 keys (key j visible from query i iff j <= i + 229376), with the
queries' dO.

Sample: 8 keys per key chunk per kv head, uniform within the chunk
(numpy default_rng(3)), 512 keys in all.  The exact gradient of a key needs
the softmax rows of every query that sees it, i.e. the whole 32768 x 262144
forward per head: minutes of fp64 work, hence a stored file.

Run from the repository root: python tests/golden/make_ring_bwd_golden.py
Calls only oracle/ and workloads/.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ring_256k_chunk7_bwd.npz")
PER_CHUNK = 8


def sample_keys(n_chunks, chunk, hkv, seed=3):
    rng = np.random.default_rng(seed)
    rows, heads = [], []
    for g in range(hkv):
        for j in range(n_chunks):
            r = np.sort(rng.choice(chunk, size=PER_CHUNK, replace=False)) + j * chunk
            rows.append(r)
            heads.append(np.full(PER_CHUNK, g))
    return np.concatenate(rows).astype(np.int64), np.concatenate(heads).astype(np.int64)


def main():
    w = workloads.ring_256k()
    n, c, qc = w.extra["n_chunks"], w.extra["chunk"], w.extra["q_chunk"]
    q, k, v, do = workloads.make_tensors(w)
    q7 = q[qc * c:(qc + 1) * c].float().numpy()
    do7 = do[qc * c:(qc + 1) * c].float().numpy()
    kn, vn = k.float().numpy(), v.float().numpy()
    krows, kheads = sample_keys(n, c, w.hkv)
    t0 = time.time()
    dk, dv = oracle.attn_bwd_dkv_rows(q7, kn, vn, do7, np.array([0, c]), np.array([0, n * c]),
                                      krows, kheads, causal=True)
    print(f"oracle: {time.time() - t0:.0f} s for {len(krows)} keys", flush=True)
    np.savez_compressed(OUT, krows=krows, kheads=kheads, dk=dk, dv=dv,
                        shape=np.array([n, c, qc, w.hq, w.hkv, w.d, w.seed]))
    print("wrote", OUT)


if __name__ == "__main__":
    main()
