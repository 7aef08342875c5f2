"""Write the realised document lengths of the seeded workloads to lengths/*.json.

Run once with ``python -m workloads.freeze_lengths``; the JSON files are then
what the tests and the benchmark read, so results do not depend on the numpy
generator version that happens to be installed.
"""
import json
import os
import sys

import numpy as np

from workloads import LENGTHS_DIR, lognormal_lengths, pareto_lengths, pareto_seed_rule


def main():
    os.makedirs(LENGTHS_DIR, exist_ok=True)
    lt = lognormal_lengths(0, 16384, 512.0, 1.2, 64, 8192)
    seed5 = pareto_seed_rule()
    mx = pareto_lengths(seed5, 131072, 1.1, 128, 65536)
    recs = {
        "longtail_16k_seed0": dict(
            lengths=lt, seed=0, total=16384,
            recipe="lognormal(median 512, sigma 1.2), round half up, clip [64, 8192], last truncated"),
        "mixed_128k": dict(
            lengths=mx, seed=seed5, total=131072,
            recipe="128*(1+pareto(1.1)), round half up, clip [128, 65536], last truncated; "
                   "seed = smallest with 1 or 2 documents above 32768"),
    }
    for name, rec in recs.items():
        rec["numpy"] = np.__version__
        with open(os.path.join(LENGTHS_DIR, name + ".json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(name, len(rec["lengths"]), "docs", file=sys.stderr)


if __name__ == "__main__":
    main()
