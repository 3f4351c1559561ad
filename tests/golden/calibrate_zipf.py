"""Calibrate the strength of the Zipf-shaped router correction bias.

The skewed GLM-5 prefill workload (16384 tokens, 256 experts, top-8) asks for an
expert popularity that follows a Zipf law of exponent 1.1.  The bias of expert e
is U(-0.01, 0.01) - beta * 1.1 * ln(rank_e).  This script finds, on the seed-0
inputs, the beta for which the least-squares slope of ln(load) against ln(rank)
over load ranks 2..128 is -1.1, by bisection, and writes it with the realised
histogram summary to zipf_beta.json beside this file.  Router scores come from
the CPU oracle; only the bias changes between bisection steps.

Run:  python tests/golden/calibrate_zipf.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

TARGET = -1.1


def slope_of(counts):
    load = np.sort(counts)[::-1].astype(np.float64)
    ranks = np.arange(1, len(load) + 1)
    sel = slice(1, 128)
    ok = load[sel] > 0
    return float(np.polyfit(np.log(ranks[sel][ok]), np.log(load[sel][ok]), 1)[0])


def main(seed=0):
    cfg = workloads.config("glm5_prefill_zipf")
    small = workloads.draw_small(cfg, seed, zipf_beta=0.0)
    dt = oracle.DTYPES[cfg.dtype]
    h = oracle.rmsnorm(small["x"], small["norm_w"], dt, cfg.eps)
    _, scores = oracle.router_scores(h, small["router_w"], dt)
    base_bias = small["corr_bias"]  # beta = 0: the uniform part only
    ranks = workloads.zipf_ranks(cfg, seed)

    def stats(beta):
        bias = (base_bias - beta * cfg.zipf_s * np.log(ranks)).astype(np.float32)
        idx, _, _ = oracle.select(scores, bias, cfg.k, cfg.routed_scale)
        cnt, _ = oracle.counts(idx, cfg.E)
        return slope_of(cnt), cnt

    lo, hi = 0.0, 0.2
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        s, _ = stats(mid)
        if s > TARGET:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 4)
    s, cnt = stats(beta)
    out = dict(beta=beta, slope=s, seed=seed, max_load=int(cnt.max()),
               experts_below_10=int((cnt < 10).sum()), empty_experts=int((cnt == 0).sum()),
               sorted_loads=sorted(cnt.tolist(), reverse=True))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_beta.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v for k, v in out.items() if k != "sorted_loads"}))


if __name__ == "__main__":
    main()
