"""Choose the router-bias offset of the skewed 128-expert workload.

The workload asks for 8 hot experts that receive about half of the T*k routing
assignments.  This script bisects the offset added to the hot experts' bias
(before it is rounded to bf16) until the share, computed with the fp64
reference's routing on the full T=8192 seeded input, is 0.50.  The result is
written into ``synth.C4_HOT_BETA`` by hand; the CPU tests re-check the share.

Run: python tests/golden/find_c4_beta.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))

import oracle  # noqa: E402
import synth  # noqa: E402


def hot_share(beta: float) -> float:
    L = synth.make_layer(4, hot_beta=beta)
    h = oracle.widen(L.h, "bf16")
    s = oracle.router_logits(h, oracle.widen(L.w_router, "bf16"), oracle.widen(L.b_router, "bf16"))
    idx = oracle.select_topk(s, L.k)
    return float(np.isin(idx, L.hot_set).mean())


def main():
    lo, hi = 0.0, 4.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if hot_share(mid) < 0.5:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 3)
    print(f"beta = {beta}  hot share = {hot_share(beta):.4f}")


if __name__ == "__main__":
    main()
