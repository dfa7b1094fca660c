"""Find the Zipf logit-bias strength that gives the local experts a ~6x load skew.

TEST INFRASTRUCTURE ONLY. Run as ``python -m oracle.calibrate_zipf``; it prints alpha, which
is then written by hand into datagen (ZIPF_ALPHA_KIMI). Skew = (local pairs / E_loc) /
(N K / E): the load a local expert sees relative to a perfectly balanced router. It uses only
the oracle's top-k and datagen's seeded logits (a sample of 8 segments).
"""
from __future__ import annotations

import numpy as np

import datagen
from .moe_oracle import topk_gating


def skew(cfg, segments=8):
    c = cfg.replace(S=segments)
    idx, _ = topk_gating(datagen.logits(c), c.K)
    local = ((idx >= c.e0) & (idx < c.e0 + c.E_loc)).sum()
    return (local / c.E_loc) / (c.N * c.K / c.E)


def main(target=6.0):
    base = datagen.CONFIGS["kimi_mx_skew"]
    lo, hi = 0.0, 3.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if skew(base.replace(zipf_alpha=mid)) < target:
            lo = mid
        else:
            hi = mid
    a = round(0.5 * (lo + hi), 2)
    print(f"alpha={a} skew={skew(base.replace(zipf_alpha=a)):.3f}")


if __name__ == "__main__":
    main()
