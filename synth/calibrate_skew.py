"""Calibrate the skewed-load router bias (writes synth/skew_alpha.json).

Runs only the oracle's router (logits, scores, keys, top-k) on the seeded
inputs of the skewed layer and bisects the bias scale alpha so that the busiest
expert receives 4.0x the mean load (T*k/E).  Usage:
    python -m synth.calibrate_skew
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402

TARGET = 4.0


def loads(cfg, logits, scores, alpha):
    b = synth.skew_bias(cfg, alpha)
    keys = O.selection_keys(logits, scores, b, cfg.score)
    idx, _ = O.select_topk(keys, cfg.k)
    return np.bincount(idx.reshape(-1), minlength=cfg.E)


def main():
    out = {}
    for cfg in synth.CONFIGS:
        if cfg.bias != "zipf":
            continue
        inp = synth.make_inputs(cfg, with_dy=False, skew_alpha=0.0, parts=("x", "router"))
        x = synth.as_f64(inp["x"], cfg.dtype)
        logits = O.router_logits(x, inp["w_router"])
        scores = O.router_scores(logits, cfg.score)
        mean = cfg.T * cfg.k / cfg.E
        lo, hi = 0.0, 1.0
        for _ in range(40):
            mid = 0.5 * (lo + hi)
            if loads(cfg, logits, scores, mid).max() / mean < TARGET:
                lo = mid
            else:
                hi = mid
        alpha = hi
        c = loads(cfg, logits, scores, alpha)
        out[cfg.name] = dict(alpha=alpha, max_over_mean=float(c.max() / mean),
                             empty_experts=int((c == 0).sum()), loads=c.tolist())
        print(cfg.name, out[cfg.name]["alpha"], out[cfg.name]["max_over_mean"], out[cfg.name]["empty_experts"])
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_alpha.json"), "w") as fh:
        json.dump(out, fh, indent=1)


if __name__ == "__main__":
    main()
