"""Finds the router-bias scale of the skewed-routing prefill workload.

The workload asks for expert popularity following Zipf(s = 1.2), with the 10
hottest experts taking about half of all T*k assignments.  The bias of expert e
is alpha * ln(pmf(rank_e)) (see workloads.zipf_bias); this script bisects alpha
on a separate calibration draw (T = 4096 tokens) using the oracle's router, and
writes tests/golden/zipf_alpha.json.  alpha is rounded to a multiple of 2**-10
so the constant in workloads is exact.

Run:  python tests/golden/make_zipf_alpha.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import moe  # noqa: E402
from tests.oracle_helpers import to_f64  # noqa: E402

CAL_T = 4096
TARGET = 0.50


def top10_share(alpha, x):
    w = workloads.WORKLOADS["prefill_zipf_shard0_w4a16"]
    G = to_f64(workloads.gen_gate(w, alpha=alpha))
    ids = moe.route(x, G, w.k)["ids"]
    counts = np.bincount(ids.reshape(-1), minlength=w.E)
    return np.sort(counts)[::-1][:10].sum() / ids.size, counts


def main():
    w = workloads.WORKLOADS["prefill_zipf_shard0_w4a16"]
    cal = workloads.replace(w, hidden_seed=w.hidden_seed + 1000)
    x = to_f64(workloads.gen_hidden(cal, T=CAL_T))
    lo, hi = 0.0, 2.0
    for _ in range(24):
        mid = 0.5 * (lo + hi)
        share, _ = top10_share(mid, x)
        if share < TARGET:
            lo = mid
        else:
            hi = mid
    alpha = round(0.5 * (lo + hi) * 1024) / 1024
    share, counts = top10_share(alpha, x)
    out = {"alpha": alpha, "top10_share": float(share), "calibration_T": CAL_T,
           "max_expert_share": float(counts.max() / (CAL_T * w.k)),
           "empty_experts": int((counts == 0).sum()),
           "recipe": "bisection of alpha for top-10 share 0.5 on hidden seed+1000, T=4096, "
                     "oracle router; alpha rounded to 2**-10"}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_alpha.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
