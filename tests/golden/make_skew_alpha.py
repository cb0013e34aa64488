"""Writes skew_alpha.json: the Zipf bias scale of the skewed-routing workload.

The skewed workload adds alpha * rank_e^(-1.1) to N(0,1) logits so that the
busiest expert receives about 1.35x its balanced share N*K/E of routes (the
imbalance one expert-parallel rank saw in the OpenPipe ART page "Price
HybridEP expert work and buffer growth at EP>1", Changes, first item).
alpha is found by bisection on the oracle's own top-K routing of the seeded
logits; nothing here touches the GPU path.

Run from the repository root:  python tests/golden/make_skew_alpha.py
"""

import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.abspath(os.path.join(os.path.dirname(__file__), "..", "..")))

import moe_inputs  # noqa: E402
from oracle import route_topk  # noqa: E402

TARGET = 1.35


def busiest_ratio(w, alpha):
    lg = moe_inputs.make_logits(w.N, w.E, w.seed, alpha)
    ids, _ = route_topk(lg, w.K)
    load = np.bincount(ids.ravel(), minlength=w.E)
    return load.max() / (w.N * w.K / w.E)


def main():
    w = moe_inputs.WORKLOADS["skew_zipf_n4096_e128_k8_f1.0"]
    lo, hi = 0.0, 2.0
    assert busiest_ratio(w, lo) < TARGET < busiest_ratio(w, hi)
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if busiest_ratio(w, mid) < TARGET:
            lo = mid
        else:
            hi = mid
    alpha = hi
    out = {
        "workload": "skew_zipf_n4096_e128_k8 (N=4096, E=128, K=8, seed 3)",
        "zipf_s": moe_inputs.ZIPF_S,
        "target_busiest_over_balanced": TARGET,
        "alpha": alpha,
        "busiest_over_balanced": float(busiest_ratio(w, alpha)),
        "written_by": "tests/golden/make_skew_alpha.py (oracle routing only)",
    }
    path = os.path.join(os.path.dirname(__file__), "skew_alpha.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")
    print(json.dumps(out, indent=2))


if __name__ == "__main__":
    main()
