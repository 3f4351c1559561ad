"""Margin filter for graded workloads (test infrastructure).

Exact routing parity is only well defined when no token's k-th and (k+1)-th
selection keys are closer than the rounding noise of either side.  Every token
whose oracle margin is below ``MIN_MARGIN`` has its row of x redrawn from its own
stream (tensor id 10, token, attempt), up to 64 attempts.
"""
import numpy as np

import oracle
import workloads

MIN_MARGIN = 1e-4
MAX_ATTEMPTS = 64


def route_small(cfg, small):
    dt = oracle.DTYPES[cfg.dtype]
    return oracle.route(small["x"], small["norm_w"], small["router_w"], small["corr_bias"], cfg.k,
                        cfg.routed_scale, dt, cfg.eps)


def filtered_small(cfg, seed=0, zipf_beta=None):
    """draw_small with low-margin rows redrawn; returns (small, routing, n_redrawn)."""
    cfg = workloads.config(cfg)
    small = workloads.draw_small(cfg, seed, zipf_beta)
    r = route_small(cfg, small)
    bad = np.nonzero(r["margin"] < MIN_MARGIN)[0]
    n_redrawn = len(bad)
    attempt = 0
    while len(bad):
        attempt += 1
        if attempt > MAX_ATTEMPTS:
            raise RuntimeError("could not reach the routing margin for %d tokens" % len(bad))
        small["x"][bad] = workloads.redraw_rows(cfg, seed, bad, attempt)
        sub = dict(small, x=small["x"][bad])
        rs = route_small(cfg, sub)
        for key in ("h", "logits", "scores", "idx", "w", "margin"):
            r[key][bad] = rs[key]
        bad = bad[rs["margin"] < MIN_MARGIN]
    return small, r, n_redrawn
