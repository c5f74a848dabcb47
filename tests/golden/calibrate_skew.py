"""Find the router-offset scale beta of the two skewed-routing recipes.

Mixtral-shape prefill: router_bias = beta * z with z ~ N(0,1) per expert,
beta chosen so that max/mean tokens per expert is 3 (the 3-5 range of
practical max/mean expert load, section 11.2.3 of the chapter "MoE model
inference", jsqmd.com).  Zipf skew: router_bias = -beta * ln k with
k ~ Zipf(1.1) per expert, beta chosen for max/mean 5.

Only the oracle's router and the input generator are used.  The result is
written to skew_calibration.json next to this script; the beta values are
then copied into the input generator's config table as dyadic constants
(multiples of 1/1024, so they are exact in any float format).

usage: python tests/golden/calibrate_skew.py [--check]
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import datagen as D  # noqa: E402
import oracle as O   # noqa: E402


def _raw(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def load_stats(cfg, beta):
    """max/mean load, number of empty experts and counts for offset scale beta."""
    x = O.decode(_raw(D.tokens(cfg)), cfg.act)
    wr = O.decode(_raw(D.router_weight(cfg)), cfg.act)
    rb = D.router_bias(cfg.replace(offset_beta=beta))
    logits = O.router_logits(x, wr, None if rb is None else rb.numpy())
    idx = O.select_experts(logits, cfg.K)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    mean = cfg.S * cfg.K / cfg.E
    return counts.max() / mean, int((counts == 0).sum()), counts


def calibrate(cfg, target, lo=0.0, hi=4.0, steps=22):
    x = O.decode(_raw(D.tokens(cfg)), cfg.act)
    wr = O.decode(_raw(D.router_weight(cfg)), cfg.act)
    base = x @ wr.T                       # float64 router product without offset
    unit = D.router_bias(cfg.replace(offset_beta=1.0)).numpy().astype(np.float64)
    mean = cfg.S * cfg.K / cfg.E

    def ratio(beta):
        rb = (beta * unit).astype(np.float32)
        logits = (base + rb.astype(np.float64)[None, :]).astype(np.float32)
        idx = O.select_experts(logits, cfg.K)
        return np.bincount(idx.reshape(-1), minlength=cfg.E).max() / mean

    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        if ratio(mid) < target:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi) * 1024) / 1024
    return beta


def main():
    check = "--check" in sys.argv
    out = {}
    for name, target in (("mixtral_prefill", 3.0), ("zipf_skew", 5.0)):
        cfg = D.CONFIGS[name]
        beta = cfg.offset_beta if check else calibrate(cfg, target)
        r, zeros, counts = load_stats(cfg, beta)
        out[name] = {"target_max_over_mean": target, "beta": beta,
                     "max_over_mean": float(r), "zero_experts": zeros,
                     "counts": counts.tolist()}
        print(name, "beta", beta, "max/mean %.4f" % r, "zero experts", zeros, flush=True)
    if not check:
        with open(os.path.join(HERE, "skew_calibration.json"), "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
