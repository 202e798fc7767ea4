"""Draft-noise sigma for the batch-sweep workloads.

The sweep compares a 16-node tree with a gamma = 5 chain on an 8B-shaped
layer at a chosen mean acceptance of 0.5, 0.8 or 0.9. Target logits are
N(0, 3^2) over a 128256-token vocabulary and draft logits are target +
N(0, sigma^2). A draft drawn from q is accepted with probability
sum_x min(p(x), q(x)) (radar-34b blog, section 2: accept with min(1, p/q)).
This script finds, by bisection, the sigma at which that overlap averaged
over 256 sampled rows equals each target, with the oracle's float64 softmax,
and writes ``sweep_sigma.txt`` beside this file. The synthetic generator
reads the table; it holds no softmax of its own.
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sweep_sigma.txt")
V, ROWS, SIGMA_T, SEED = 128256, 256, 3.0, 3
TARGETS = (0.5, 0.8, 0.9)


def mean_overlap(t: np.ndarray, n: np.ndarray, sigma: float) -> float:
    p = oracle.softmax(t)
    q = oracle.softmax(t + np.float32(sigma) * n)
    return float(np.minimum(p, q).sum(axis=1).mean())


def main():
    rng = np.random.default_rng(SEED)
    t = rng.standard_normal((ROWS, V), dtype=np.float32) * np.float32(SIGMA_T)
    n = rng.standard_normal((ROWS, V), dtype=np.float32)
    lines = ["# Draft-noise sigma of the batch-sweep workloads (8B-shaped layer, vocab",
             f"# {V}, target logits N(0, {SIGMA_T:g}^2), draft = target + N(0, sigma^2)): the",
             "# sigma at which the mean over 256 sampled rows of sum_x min(p(x), q(x)),",
             "# the acceptance probability of a draft drawn from q, equals the target.",
             "# Written by sweep_sigma.py with the oracle's float64 softmax.",
             "# acceptance sigma realised"]
    for a in TARGETS:
        lo, hi = 0.0, 8.0          # overlap falls from 1 as sigma grows
        for _ in range(24):
            mid = 0.5 * (lo + hi)
            if mean_overlap(t, n, mid) > a:
                lo = mid
            else:
                hi = mid
        s = 0.5 * (lo + hi)
        got = mean_overlap(t, n, s)
        assert abs(got - a) < 0.005, (a, s, got)
        lines.append(f"{a:g} {s:.6f} {got:.6f}")
        print(lines[-1], flush=True)
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
