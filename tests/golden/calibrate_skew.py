"""Fits the Zipf bias scale of the skewed workload (T=8192, E=256, H=7168,
I=2048, k=8) so that the hottest expert receives about ten times the mean
load R/E, on the seed-0 draw.  Routing uses only the oracle.  Prints the value
to store as SKEW_LAMBDA in moe_layer_amd/workloads.py.

    python tests/golden/calibrate_skew.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from moe_layer_amd.workloads import CONFIGS, Workload  # noqa: E402


def load_ratio(w, base, lam):
    c = w.cfg
    lg = (base + w.router_bias(lam)[None, :]).astype(np.float32)
    ids, _ = oracle.route(lg, c.topk)
    counts = np.bincount(ids.reshape(-1), minlength=c.E)
    return counts.max() / (c.T * c.topk / c.E), int((counts == 0).sum())


def main():
    w = Workload(CONFIGS["skew"])
    base = w.router_product()
    lo, hi = 0.0, 0.5
    for _ in range(30):
        mid = (lo + hi) / 2
        r, _ = load_ratio(w, base, mid)
        if r < 10.0:
            lo = mid
        else:
            hi = mid
    lam = round((lo + hi) / 2, 4)
    r, dead = load_ratio(w, base, lam)
    print(f"SKEW_LAMBDA = {lam}  (max load / mean = {r:.3f}, experts with no rows = {dead})")


if __name__ == "__main__":
    main()
