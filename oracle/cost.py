"""The speedup model of speculative decoding (float64).

LLM Primer ch. 9, section 9.3: the speedup of a speculative step is the
expected number of accepted tokens divided by (T_draft / T_decode + 1 +
alpha * N), where alpha is the verification overhead per candidate position
(typically 0.05 to 0.15) and N the number of candidates. With N growing,
alpha * N eventually dominates, so there is a best N (the pages put it at
6 to 8 for an acceptance rate of 0.8 and 10 to 12 for 0.9), and as the
acceptance rate approaches 1 the speedup approaches 1 / alpha.

Readings: "expected accepted tokens" counts every token a step emits
(accepted candidates plus the one drawn at the stopping node), which for a
chain of N candidates accepted with probability p each is
sum_{i=0}^{N} p^i (jisaku.com glossary, linear-speculation closed form);
for a tree, with the draft's own estimate of acceptance (the product of q
along a node's path), it is 1 + the sum over candidate nodes of their path
products.
"""

from __future__ import annotations

import math

import numpy as np


def speedup(expected_emitted: float, draft_ratio: float, alpha: float, n: int) -> float:
    """E[emitted] / (T_draft/T_decode + 1 + alpha * N)."""
    return float(expected_emitted) / (float(draft_ratio) + 1.0 + float(alpha) * n)


def chain_expected_emitted(p: float, n: int) -> float:
    """sum_{i=0}^{n} p^i, term by term."""
    total, term = 0.0, 1.0
    for _ in range(n + 1):
        total += term
        term *= p
    return total


def best_chain_length(p: float, draft_ratio: float, alpha: float, n_max: int):
    """The N in [1, n_max] with the largest model speedup for a chain (the
    smallest such N on ties); returns (N, speedup)."""
    best_n, best_s = 0, -math.inf
    for n in range(1, n_max + 1):
        s = speedup(chain_expected_emitted(p, n), draft_ratio, alpha, n)
        if s > best_s:
            best_n, best_s = n, s
    return best_n, best_s


def tree_expected_emitted(parent, logq) -> float:
    """1 + sum over non-root nodes of exp(sum of log q along the path)."""
    par = np.asarray(parent)
    lq = np.asarray(logq, dtype=np.float64)
    total = 1.0
    for i in range(1, par.shape[0]):
        s, j = 0.0, i
        while j != 0:
            s += min(float(lq[j]), 0.0)
            j = int(par[j])
        total += math.exp(s)
    return total


def alpha_from_times(n_values, step_us) -> float:
    """Per-position overhead from verification times T(N): the least-squares
    slope of T(N) / T(1) - 1 against N - 1 (through the origin), with T(1)
    the time at the smallest N given, which must be 1."""
    n = np.asarray(n_values, dtype=np.float64)
    t = np.asarray(step_us, dtype=np.float64)
    if n[0] != 1:
        raise ValueError("the first N must be 1")
    x = n - 1.0
    y = t / t[0] - 1.0
    return float((x * y).sum() / (x * x).sum())
