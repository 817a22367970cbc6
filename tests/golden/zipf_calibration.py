"""Fix beta of the prefill workload's Zipf selection-bias term.

The prefill workload (T = 4096 tokens on the GLM-like layer) asks for expert
load following Zipf(s = 1.1).  Exact Zipf is out of reach at top-8 (the head
expert would need more selections than there are tokens), so the selection
bias gets a term -1.1 * beta * ln(rank_e) over a seeded rank permutation, and
beta is chosen by bisection so that the least-squares slope of
log(load) against log(rank), over the ranks that are neither saturated
(load < 95% of T) nor empty, is -1.1.

Uses only the oracle's routing and the seeded generator.  Run:
    python tests/golden/zipf_calibration.py
It prints beta and the realised load histogram; the value is stored as
GLM_PREFILL_ZIPF_BETA in synth/__init__.py and in zipf_calibration.json.
"""
import dataclasses
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

SEED = 1
T = 4096
TARGET = -1.1


def loads_for(beta, logits, base_shape):
    shape = dataclasses.replace(base_shape, zipf_beta=beta)
    _, bias = synth.router(shape, SEED)
    idx, _ = oracle.select(logits, bias, shape.top_k, shape.rsf)
    counts = np.bincount(idx.reshape(-1), minlength=shape.n_experts)
    perm = synth.permutation(SEED, synth.tag(0, synth.KIND_ZIPF_PERM), shape.n_experts)
    return counts[perm]  # load by rank 1..E


def slope(load_by_rank):
    r = np.arange(1, load_by_rank.size + 1)
    m = (load_by_rank > 0) & (load_by_rank < 0.95 * T)
    if m.sum() < 8:
        return 0.0
    return float(np.polyfit(np.log(r[m]), np.log(load_by_rank[m]), 1)[0])


def main():
    base = synth.GLM
    wr, _ = synth.router(base, SEED)
    x = synth.hidden(base, SEED, T)
    logits = oracle.router_logits(x, wr)
    lo, hi = 0.0, 1.0
    s_hi = slope(loads_for(hi, logits, base))
    assert s_hi < TARGET, s_hi
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if slope(loads_for(mid, logits, base)) < TARGET:
            hi = mid
        else:
            lo = mid
    beta = float(np.float32(hi))
    lr = loads_for(beta, logits, base)
    rec = dict(beta=beta, slope=slope(lr), seed=SEED, tokens=T,
               load_by_rank=lr.tolist(), distinct_experts=int((lr > 0).sum()))
    print(json.dumps({k: rec[k] for k in ("beta", "slope", "distinct_experts")}))
    print("head loads:", lr[:16].tolist())
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_calibration.json"), "w") as f:
        json.dump(rec, f)


if __name__ == "__main__":
    main()
